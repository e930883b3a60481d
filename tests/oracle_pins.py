"""Pins that fix the oracle to something other than itself.

Each `pin_*` function takes a decode callable with the oracle's signature

    decode(q, L_K, L_V, B_K, B_V, seq_lens, scales=None, softmax_scale=None)
        -> float64 [B, Hq, d]

and raises AssertionError when the callable disagrees with what the pages and
the mathematics fix.  The oracle must pass every pin; each deliberately broken
copy of it (a dropped term, a wrong index, a swapped operand; see
test_oracle_mutants.py) must fail at least one.

What each pin rests on:
  golden       hand-derived closed-form fixtures under tests/golden/
  brute        40-digit decimal nested loops (oracle.brute), exact far past fp64
  sdpa         r = d with identity factors reduces the method to ordinary dense
               attention: torch's scaled_dot_product_attention, float64 on CPU
  t1           one valid token: softmax weight 1, out = dequantized L_V[0] B_V
  q0           q = 0: equal scores, out = mean of the rebuilt V rows
  permutation  attention is a set function of the (K, V) rows: reordering or
               duplicating every token leaves the output unchanged
  gqa          grouped query heads equal per-head attention with each kv-head's
               latents and factors copied to its group
  ragged       a sequence's output equals that of the dense problem truncated to
               its length, whatever the padding holds
  int8         int8 latents with scales equal float latents holding scale * int
  absorbed     the factored route (q B_K^T) . L_K^T, (p L_V) B_V agrees
  scale        scaling q by c and the softmax scale by 1/c changes nothing;
               the default scale is 1/sqrt(d)
"""
from __future__ import annotations

import glob
import json
import math
import os

import numpy as np

import oracle
from oracle import brute
import workloads

GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")


def _f64(w: workloads.Workload):
    """float64 views of a drawn workload, in the oracle's argument order."""
    q = oracle.as_float64(w.q, w.q_dtype)
    LK = oracle.as_float64(w.L_K, w.latent_dtype)
    LV = oracle.as_float64(w.L_V, w.latent_dtype)
    BK = oracle.as_float64(w.B_K, w.factor_dtype)
    BV = oracle.as_float64(w.B_V, w.factor_dtype)
    sc = None if w.scales is None else w.scales.astype(np.float64)
    return q, LK, LV, BK, BV, w.seq_lens.copy(), sc


def rel_rowmax(a: np.ndarray, b: np.ndarray) -> float:
    """max over rows of ||a - b||_inf / ||b||_inf (rows are the last axis)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    num = np.abs(a - b).max(axis=1)
    den = np.maximum(np.abs(b).max(axis=1), 1e-300)
    return float((num / den).max())


def load_golden():
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json"))):
        with open(path) as fh:
            out.append(json.load(fh))
    return out


# ---------------------------------------------------------------- pins

def pin_golden(decode):
    for f in load_golden():
        arr = lambda k: np.asarray(f[k], dtype=np.float64)  # noqa: E731
        sc = None if f["scales"] is None else arr("scales")
        got = decode(arr("q"), arr("L_K"), arr("L_V"), arr("B_K"), arr("B_V"),
                     np.asarray(f["seq_lens"], dtype=np.int64), scales=sc,
                     softmax_scale=f["softmax_scale"])
        exp = arr("expected")
        err = np.abs(got - exp).max() / max(np.abs(exp).max(), 1.0)
        assert err <= f["tol"], f"golden {f['name']}: err {err:.3e} > {f['tol']}"


BRUTE_CASES = [
    # (workload, overrides) - tiny shapes, ragged lengths, float and int8
    ("tiny", dict(B=2, Hq=4, Hkv=4, d=4, r=2, T=5, seq_lens=[5, 3])),
    ("tiny", dict(B=2, Hq=4, Hkv=2, d=8, r=4, T=17, seq_lens=[17, 9])),
    ("tiny", dict(B=2, Hq=4, Hkv=1, d=8, r=2, T=2, seq_lens=[1, 2])),
    ("tiny", dict(B=1, Hq=2, Hkv=2, d=4, r=4, T=1)),
    ("int8", dict(B=2, Hq=4, Hkv=2, d=4, r=2, T=5, seq_lens=[4, 5])),
    ("int8", dict(B=2, Hq=4, Hkv=4, d=8, r=4, T=17, seq_lens=[17, 1])),
    ("gqa_vlm", dict(B=1, Hq=4, Hkv=1, d=8, r=4, T=9, image_tokens=3)),
]


def pin_brute(decode, cases=BRUTE_CASES, tol=1e-13):
    for name, ov in cases:
        ov = dict(ov)
        w = workloads.make(name, seed=ov.pop("seed", 11), **ov)
        args = _f64(w)
        got = decode(*args[:6], scales=args[6])
        ref = brute.decode_decimal(*args[:6], scales=args[6])
        ref = np.array([[[float(x) for x in row] for row in rb] for rb in ref])
        err = rel_rowmax(got, ref)
        assert err <= tol, f"brute {name} {ov}: rel err {err:.3e}"


def pin_sdpa(decode):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    for (B, Hq, Hkv, d, T, int8) in [(2, 4, 2, 8, 13, False), (1, 3, 3, 16, 40, False),
                                     (2, 2, 1, 4, 7, True)]:
        r = d
        eye = np.broadcast_to(np.eye(d), (Hkv, d, d)).copy()
        q = rng.standard_normal((B, Hq, d))
        if int8:
            LK = rng.integers(-127, 128, (B, Hkv, T, r)).astype(np.float64)
            LV = rng.integers(-127, 128, (B, Hkv, T, r)).astype(np.float64)
            sc = rng.uniform(0.005, 0.02, (2, B, Hkv, T))
            K = LK * sc[0][..., None]
            V = LV * sc[1][..., None]
        else:
            LK = rng.standard_normal((B, Hkv, T, r))
            LV = rng.standard_normal((B, Hkv, T, r))
            sc = None
            K, V = LK, LV
        lens = np.full(B, T)
        got = decode(q, LK, LV, eye, eye, lens, scales=sc)
        G = Hq // Hkv
        Kr = torch.from_numpy(np.repeat(K, G, axis=1))        # [B, Hq, T, d]
        Vr = torch.from_numpy(np.repeat(V, G, axis=1))
        qt = torch.from_numpy(q)[:, :, None, :]                 # [B, Hq, 1, d]
        ref = F.scaled_dot_product_attention(qt, Kr, Vr, scale=1.0 / math.sqrt(d))
        ref = ref[:, :, 0, :].numpy()
        err = rel_rowmax(got, ref)
        assert err <= 1e-12, f"sdpa B{B} Hq{Hq} Hkv{Hkv} d{d} int8={int8}: {err:.3e}"


def pin_t1(decode):
    for name in ("tiny", "int8"):
        w = workloads.make(name, seed=3, B=2, Hq=4, Hkv=2, d=8, r=4, T=6,
                           seq_lens=[1, 1])
        q, LK, LV, BK, BV, lens, sc = _f64(w)
        got = decode(q, LK, LV, BK, BV, lens, scales=sc)
        for b in range(2):
            for h in range(4):
                g = h // 2
                lv = LV[b, g, 0] * (sc[1, b, g, 0] if sc is not None else 1.0)
                exp = lv @ BV[g]
                assert np.allclose(got[b, h], exp, rtol=1e-13, atol=1e-13 * np.abs(exp).max()), \
                    f"T=1 {name} b{b} h{h}"


def pin_q0(decode):
    for name in ("tiny", "int8"):
        w = workloads.make(name, seed=4, B=1, Hq=2, Hkv=1, d=8, r=4, T=11)
        q, LK, LV, BK, BV, lens, sc = _f64(w)
        q[:] = 0.0
        got = decode(q, LK, LV, BK, BV, lens, scales=sc)
        lv = LV[0, 0] * (sc[1, 0, 0][:, None] if sc is not None else 1.0)
        exp = (lv @ BV[0]).mean(axis=0)
        assert rel_rowmax(got[0], np.stack([exp, exp])) <= 1e-13, f"q=0 {name}"


def pin_permutation(decode):
    w = workloads.make("int8", seed=6, B=2, Hq=4, Hkv=2, d=8, r=4, T=9)
    q, LK, LV, BK, BV, lens, sc = _f64(w)
    base = decode(q, LK, LV, BK, BV, lens, scales=sc)
    perm = np.random.default_rng(0).permutation(9)
    got = decode(q, LK[:, :, perm], LV[:, :, perm], BK, BV, lens,
                 scales=sc[:, :, :, perm])
    assert rel_rowmax(got, base) <= 1e-13, "token permutation changed the output"
    dup = np.repeat(np.arange(9), 2)
    got = decode(q, LK[:, :, dup], LV[:, :, dup], BK, BV, lens * 2,
                 scales=sc[:, :, :, dup])
    assert rel_rowmax(got, base) <= 1e-13, "duplicating every token changed the output"


def pin_gqa(decode):
    w = workloads.make("gqa_vlm", seed=7, B=2, Hq=8, Hkv=2, d=8, r=4, T=10,
                       image_tokens=4, seq_lens=[10, 6])
    q, LK, LV, BK, BV, lens, sc = _f64(w)
    got = decode(q, LK, LV, BK, BV, lens)
    G = 4
    mha = decode(q, np.repeat(LK, G, axis=1), np.repeat(LV, G, axis=1),
                 np.repeat(BK, G, axis=0), np.repeat(BV, G, axis=0), lens)
    assert rel_rowmax(got, mha) <= 1e-13, "GQA differs from replicated MHA"
    # and the replicated problem is not trivially head-independent
    assert rel_rowmax(mha[:, 0], mha[:, G]) > 1e-3


def pin_ragged(decode):
    for name in ("llm7b", "int8"):
        w = workloads.make(name, seed=8, B=3, Hq=2, Hkv=2, d=8, r=4, T=12,
                           seq_lens=[12, 5, 1], pad="nan")
        q, LK, LV, BK, BV, lens, sc = _f64(w)
        got = decode(q, LK, LV, BK, BV, lens, scales=sc)
        assert np.isfinite(got).all(), f"{name}: padding leaked into the output"
        for b, n in enumerate(lens):
            sub = decode(q[b:b + 1], LK[b:b + 1, :, :n], LV[b:b + 1, :, :n], BK, BV,
                         np.array([n]), scales=None if sc is None else sc[:, b:b + 1, :, :n])
            assert rel_rowmax(got[b], sub[0]) <= 1e-14, f"{name} b{b}: ragged != truncated"


def pin_int8(decode):
    w = workloads.make("int8", seed=9, B=2, Hq=4, Hkv=2, d=8, r=4, T=7, seq_lens=[7, 4])
    q, LK, LV, BK, BV, lens, sc = _f64(w)
    got = decode(q, LK, LV, BK, BV, lens, scales=sc)
    fk = LK * sc[0][..., None]
    fv = LV * sc[1][..., None]
    ref = decode(q, fk, fv, BK, BV, lens)
    assert rel_rowmax(got, ref) <= 1e-14, "int8 path != float path on dequantized values"


def pin_absorbed(decode):
    for name, ov in (("gqa_vlm", dict(B=2, Hq=8, Hkv=2, d=16, r=4, T=30, image_tokens=5)),
                     ("int8", dict(B=2, Hq=2, Hkv=2, d=8, r=4, T=9, seq_lens=[9, 3]))):
        w = workloads.make(name, seed=10, **ov)
        args = _f64(w)
        a = decode(*args[:6], scales=args[6])
        b = oracle.decode_absorbed(*args[:6], scales=args[6])
        assert rel_rowmax(a, b) <= 1e-12, f"{name}: absorbed route disagrees"


def pin_scale(decode):
    w = workloads.make("tiny", seed=12, B=1, Hq=2, Hkv=2, d=16, r=4, T=8)
    q, LK, LV, BK, BV, lens, sc = _f64(w)
    base = decode(q, LK, LV, BK, BV, lens)
    explicit = decode(q, LK, LV, BK, BV, lens, softmax_scale=0.25)  # 1/sqrt(16)
    assert rel_rowmax(explicit, base) <= 1e-15, "default scale is not 1/sqrt(d)"
    got = decode(q * 4.0, LK, LV, BK, BV, lens, softmax_scale=1.0 / 16)
    assert rel_rowmax(got, base) <= 1e-14, "scale does not multiply the logits"


ALL_PINS = [pin_golden, pin_brute, pin_sdpa, pin_t1, pin_q0, pin_permutation,
            pin_gqa, pin_ragged, pin_int8, pin_absorbed, pin_scale]

"""GPU parity of the attention-aware adaptive-rank decode (AttentionPack
page, section 2.B) against the fp64 oracle's decode_adaptive, through the
C-ABI: the output (gate as for lrattn_decode: 2e-3 for bf16/int8 inputs,
1e-5 for fp32) and the updated importance scores (the step's head-averaged
attention weights, computed in fp32 from the logits, within 1e-4 of the
largest term of the update)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import TOL, rel_rowmax, say, to_device

pytestmark = pytest.mark.gpu


def _importance(w, seed, grid=False):
    rng = np.random.default_rng(seed)
    imp = rng.uniform(0.0, 1.0, (w.batch, w.num_kv_heads, w.max_seq_len))
    if grid:     # values on a grid that holds the threshold itself
        imp = np.round(imp * 4) / 4
    return imp.astype(np.float32)


def _run(w, dev, imp, k, thr, decay, **kw):
    import torch
    import rank_kv_cache_head_amd as lr
    t = torch.from_numpy(imp.copy()).cuda()
    out = lr.adaptive_decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"],
                             dev["seq_lens"], t, low_rank=k, threshold=thr, decay=decay,
                             scales=dev["scales"], softmax_scale=w.softmax_scale, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), t.cpu().numpy()


def _ref(w, imp, k, thr, decay, sel=None):
    f = oracle.as_float64
    sl = slice(None) if sel is None else sel
    sc = None if w.scales is None else w.scales[:, sl].astype(np.float64)
    return oracle.decode_adaptive(f(w.q[sl], w.q_dtype), f(w.L_K[sl], w.latent_dtype),
                                  f(w.L_V[sl], w.latent_dtype), f(w.B_K, w.factor_dtype),
                                  f(w.B_V, w.factor_dtype), w.seq_lens[sl],
                                  imp[sl].astype(np.float64), thr, k, decay, scales=sc,
                                  softmax_scale=w.softmax_scale)


def _check_update(got, ref, imp_in, decay, lens):
    for b, n in enumerate(lens):
        assert np.array_equal(got[b, :, n:], imp_in[b, :, n:]), "entries past seq_len changed"
        a = (ref[b, :, :n] - decay * imp_in[b, :, :n].astype(np.float64)) / max(1 - decay, 1e-30)
        scale = (1 - decay) * np.abs(a).max() + decay * np.abs(imp_in[b, :, :n]).max()
        assert np.abs(got[b, :, :n] - ref[b, :, :n]).max() <= 1e-4 * scale, b


CASES = {
    "gqa_bf16_r64": ("gqa_vlm", dict(B=3, Hq=8, Hkv=2, T=1200, seq_lens=[1200, 500, 7])),
    "mha_bf16_r32": ("llm7b", dict(B=2, Hq=4, Hkv=4, T=1000, seq_lens=[1000, 321])),
    "bf16_r48_g1": ("ragged", dict(B=2, Hq=2, Hkv=2, T=1500, seq_lens=[1500, 64])),
    "g8_bf16_r32": ("gqa_vlm", dict(B=2, Hq=16, Hkv=2, r=32, T=800, seq_lens=[800, 333])),
    "int8_g4": ("int8", dict(B=2, Hq=8, Hkv=2, T=1100, seq_lens=[1100, 99])),
    "int8_g1": ("int8", dict(B=2, Hq=4, Hkv=4, T=900, seq_lens=[900, 1])),
    "fp32_r16": ("tiny", dict(B=2, T=256, seq_lens=[256, 31])),
    # two heads per kv-head; T not a multiple of 4 (one token per thread in
    # the score update)
    "g2_bf16_odd_T": ("gqa_vlm", dict(B=2, Hq=4, Hkv=2, T=1001, seq_lens=[1001, 250])),
    # the matrix-core kernel's other shapes (8 heads at r = 64, 4 at r = 32)
    "g8_bf16_r64": ("gqa_vlm", dict(B=2, Hq=16, Hkv=2, T=700, seq_lens=[700, 129])),
    "g4_bf16_r32": ("gqa_vlm", dict(B=2, Hq=8, Hkv=2, r=32, T=600, seq_lens=[600, 77])),
    # r = 128: a row is two 128-byte lines, and a low row's second line is
    # not read (matrix-core kernel at 4 and 8 heads, VALU kernel at 1)
    "g4_bf16_r128": ("gqa_vlm", dict(B=2, Hq=8, Hkv=2, r=128, T=900, seq_lens=[900, 301])),
    "g8_bf16_r128": ("gqa_vlm", dict(B=2, Hq=16, Hkv=2, r=128, T=500, seq_lens=[500, 64])),
    "g1_bf16_r128": ("llm7b", dict(B=2, Hq=2, Hkv=2, r=128, T=700, seq_lens=[700, 150])),
    # 8 heads per kv-head on the VALU kernel (r = 48 is not a multiple of 32)
    "g8_bf16_r48": ("ragged", dict(B=2, Hq=16, Hkv=2, T=900, seq_lens=[900, 203])),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_adaptive_decode_matches_oracle(case):
    base, kw = CASES[case]
    w = workloads.make(base, **kw)
    dev = to_device(w)
    r = w.rank
    for k, thr, decay, grid, splits in ((r // 2, 0.5, 0.9, False, 0), (1, 0.25, 0.0, True, 3),
                                        (r, 0.5, 0.5, False, 1), (r // 4, -1.0, 1.0, False, 0),
                                        (r // 4, 2.0, 0.3, True, 7)):
        imp = _importance(w, seed=k + int(10 * decay), grid=grid)
        say(f"adaptive {case} low_rank={k} thr={thr} decay={decay} splits={splits}")
        out, new = _run(w, dev, imp, k, thr, decay, num_splits=splits)
        ref_out, ref_imp = _ref(w, imp, k, thr, decay)
        err = rel_rowmax(out, ref_out)
        assert err <= TOL[w.latent_dtype], (k, thr, decay, err)
        _check_update(new, ref_imp, imp, decay, w.seq_lens)


def test_adaptive_full_rank_equals_decode():
    """Every token important (threshold -inf): the output is lrattn_decode's
    to fp32 accuracy (the same reduction order on the VALU kernel)."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = workloads.make("llm7b", B=2, Hq=4, Hkv=4, T=1000, seq_lens=[1000, 400])
    dev = to_device(w)
    say("adaptive full rank == decode")
    out, _ = _run(w, dev, _importance(w, 1), 4, -np.inf, 0.5)
    ref = lr.decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"],
                    softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    assert rel_rowmax(out, ref.cpu().numpy().astype(np.float64)) <= 2e-5


def test_adaptive_deterministic_and_nan_padding():
    kw = dict(B=2, Hq=8, Hkv=2, T=1024, seq_lens=[1024, 300])
    wz = workloads.make("gqa_vlm", pad="zero", **kw)
    wn = workloads.make("gqa_vlm", pad="nan", **kw)
    imp = _importance(wz, 3)
    say("adaptive determinism / NaN padding")
    res = [_run(w, to_device(w), imp, 16, 0.5, 0.8) for w in (wz, wn, wz)]
    for o, i in res[1:]:
        assert np.array_equal(o, res[0][0]) and np.array_equal(i, res[0][1])
    assert np.isfinite(res[1][0]).all()


def test_adaptive_full_size_gqa_vlm():
    """gqa_vlm at full size, half the tokens at rank 16; every sequence
    against the oracle (output and updated scores, one sequence at a time
    in float64)."""
    w = workloads.make("gqa_vlm")
    say("adaptive full gqa_vlm: inputs")
    dev = to_device(w)
    imp = _importance(w, 4)
    say("adaptive full gqa_vlm: decode")
    out, new = _run(w, dev, imp, 16, 0.5, 0.9)
    err = 0.0
    for b in range(w.batch):
        sel = [b]
        ref_out, ref_imp = _ref(w, imp, 16, 0.5, 0.9, sel=sel)
        err = max(err, rel_rowmax(out[sel], ref_out))
        _check_update(new[sel], ref_imp, imp[sel], 0.9, w.seq_lens[sel])
    say(f"  err {err:.3e}")
    assert err <= TOL[w.latent_dtype], err


def test_adaptive_full_size_r128_bench_setting():
    """The benchmark's r = 128 leg at full size: gqa_vlm's batch, heads and
    lengths over a 256-byte-row cache, low rank 64 below threshold 0.5 with
    decay 1.0 (half the rows skip their second 128-byte line); every
    sequence against the oracle."""
    w = workloads.make("gqa_vlm", r=128, factor_std=1.0 / np.sqrt(128))
    say("adaptive full gqa_vlm r=128: inputs")
    dev = to_device(w)
    imp = _importance(w, 5)
    say("adaptive full gqa_vlm r=128: decode")
    out, new = _run(w, dev, imp, 64, 0.5, 1.0)
    assert np.array_equal(new, imp)      # decay 1.0 keeps the scores
    err = 0.0
    for b in range(w.batch):
        sel = [b]
        ref_out, _ = _ref(w, imp, 64, 0.5, 1.0, sel=sel)
        err = max(err, rel_rowmax(out[sel], ref_out))
    say(f"  err {err:.3e}")
    assert err <= TOL[w.latent_dtype], err


@pytest.mark.parametrize("base,kw", [
    # matrix-core kernel, 4 heads at r = 64 (2048-row chunks): three chunks, the last partial
    ("gqa_vlm", dict(B=2, Hq=8, Hkv=2, T=5000, seq_lens=[5000, 2100])),
    # matrix-core kernel, 8 heads at r = 64 (1024-row chunks)
    ("gqa_vlm", dict(B=1, Hq=16, Hkv=2, T=3000, seq_lens=[2999])),
    # VALU kernel, one head per kv-head (4096-row chunks)
    ("llm7b", dict(B=2, Hq=2, Hkv=2, T=9000, seq_lens=[9000, 4097])),
    # VALU kernel, int8 latents, 4 heads (1024-row chunks)
    ("int8", dict(B=1, Hq=8, Hkv=2, T=2500, seq_lens=[2500])),
])
def test_adaptive_logits_in_several_chunks(base, kw):
    """One partition per sequence, longer than the LDS chunk of logits the
    partition kernel stages: the logits leave in several chunks (the last
    one partial) and the score update must still match the oracle."""
    w = workloads.make(base, **kw)
    dev = to_device(w)
    imp = _importance(w, 7)
    k = w.rank // 2
    say(f"adaptive chunks {base} {kw}")
    out, new = _run(w, dev, imp, k, 0.5, 0.6, num_splits=1)
    ref_out, ref_imp = _ref(w, imp, k, 0.5, 0.6)
    err = rel_rowmax(out, ref_out)
    say(f"  err {err:.3e}")
    assert err <= TOL[w.latent_dtype], err
    _check_update(new, ref_imp, imp, 0.6, w.seq_lens)

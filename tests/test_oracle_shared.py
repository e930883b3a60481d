"""Pins for the oracle's shared-latent decode (CPU only).

Two independent reductions to the pinned per-head decode: (1) when every
query head of a stream carries the same factor, the shared decode is ordinary
grouped decode with that stream as the kv-head; (2) replicating each stream's
latents once per query head turns it into a per-head cache (Hkv = Hq) with the
per-head factors.  Planted mistakes must fail one of them.
"""
import numpy as np
import pytest

import oracle
import workloads


def _case(seed, S=2, Hq=8, lt="bf16"):
    base = "int8" if lt == "i8" else "gqa_vlm"
    kw = dict(B=3, Hq=Hq, Hkv=Hq, d=16, r=8, T=30, seq_lens=[30, 11, 1], factor_std=0.35)
    if lt != "i8":
        kw["latent_dtype"] = lt
    w = workloads.make(base, seed=seed, **kw)
    f = oracle.as_float64
    q = f(w.q, w.q_dtype)
    BK, BV = f(w.B_K, w.factor_dtype), f(w.B_V, w.factor_dtype)   # [Hq, r, d]: per head
    LK, LV = f(w.L_K, w.latent_dtype)[:, :S], f(w.L_V, w.latent_dtype)[:, :S]
    sc = None if w.scales is None else w.scales[:, :, :S].astype(np.float64)
    return q, LK, LV, BK, BV, w.seq_lens, sc


def pin_same_factor_is_gqa(dec):
    q, LK, LV, BK, BV, lens, sc = _case(1)
    Hq, S = q.shape[1], LK.shape[1]
    G = Hq // S
    BKs = np.repeat(BK[::G][:S], G, axis=0)          # head h uses its stream's factor
    BVs = np.repeat(BV[::G][:S], G, axis=0)
    got = dec(q, LK, LV, BKs, BVs, lens, scales=sc)
    ref = oracle.decode(q, LK, LV, BK[::G][:S], BV[::G][:S], lens, scales=sc)
    assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()


def pin_replicated_latent_is_per_head(dec):
    for lt in ("bf16", "i8"):
        q, LK, LV, BK, BV, lens, sc = _case(2, lt=lt)
        Hq, S = q.shape[1], LK.shape[1]
        G = Hq // S
        rep = lambda a: np.repeat(a, G, axis=1)
        ref = oracle.decode(q, rep(LK), rep(LV), BK, BV, lens,
                            scales=None if sc is None else np.repeat(sc, G, axis=2))
        got = dec(q, LK, LV, BK, BV, lens, scales=sc)
        assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max(), lt


PINS = [pin_same_factor_is_gqa, pin_replicated_latent_is_per_head]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_shared_pin(pin):
    pin(oracle.decode_shared)


def _mutant(kind):
    def dec(q, LK, LV, BK, BV, lens, scales=None, softmax_scale=None):
        Bsz, Hq, d = q.shape
        S, T = LK.shape[1], LK.shape[2]
        G = Hq // S
        out = np.zeros((Bsz, Hq, d))
        for b in range(Bsz):
            n = int(lens[b])
            for h in range(Hq):
                s_ = h % S if kind == "stream_modulo" else h // G
                lk, lv = LK[b, s_, :n], LV[b, s_, :n]
                if scales is not None:
                    lk = lk * scales[0, b, s_, :n, None]
                    lv = lv * scales[1, b, s_, :n, None]
                fk = BK[s_] if kind == "factor_by_stream" else BK[h]
                fv = BK[h] if kind == "v_uses_bk" else BV[h]
                K, V = lk @ fk, lv @ fv
                sc_ = K @ q[b, h] / np.sqrt(d)
                e = np.exp(sc_ - sc_.max())
                out[b, h] = (e / e.sum()) @ V
        return out
    return dec


@pytest.mark.parametrize("kind", ["stream_modulo", "factor_by_stream", "v_uses_bk"])
def test_shared_mutant_caught(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except Exception:
            caught.append(pin.__name__)
    assert caught, kind


def test_unmutated_shared_copy_passes():
    for pin in PINS:
        pin(_mutant(None))

"""Pins for the oracle's decode with per-modality factors (CPU only).

AttentionPack page, section 2.A compresses image and text tokens apart.  The
oracle's decode_modal is reduced to the pinned per-head decode three ways:
(1) equal factor sets give decode itself; (2) an image block of 0 tokens, or
one covering the whole sequence, gives decode with the text or the image set;
(3) the two sets are one factor of rank 2r over a widened latent whose first r
columns hold the image tokens' latents (zeros elsewhere) and whose last r hold
the text tokens' -- so decode of that widened cache must equal decode_modal.
Planted mistakes (boundary off by one, image block at the end, a set applied
to the wrong one of K and V) must each fail a pin.
"""
import numpy as np
import pytest

import oracle
import workloads


def _case(seed, lt="bf16", lens=(30, 11, 1), T=30):
    base = "int8" if lt == "i8" else "gqa_vlm"
    kw = dict(B=len(lens), Hq=4, Hkv=2, d=16, r=8, T=T, seq_lens=list(lens), factor_std=0.35)
    w = workloads.make(base, seed=seed, **kw)
    w2 = workloads.make(base, seed=seed + 100, **kw)      # the second factor set
    f = oracle.as_float64
    q = f(w.q, w.q_dtype)
    BK = np.stack([f(w.B_K, w.factor_dtype), f(w2.B_K, w2.factor_dtype)])
    BV = np.stack([f(w.B_V, w.factor_dtype), f(w2.B_V, w2.factor_dtype)])
    LK, LV = f(w.L_K, w.latent_dtype), f(w.L_V, w.latent_dtype)
    sc = None if w.scales is None else w.scales.astype(np.float64)
    return q, LK, LV, BK, BV, w.seq_lens, sc


def _close(got, ref, tol=1e-13):
    assert np.abs(got - ref).max() <= tol * np.abs(ref).max()


def pin_equal_sets_is_decode(dec):
    q, LK, LV, BK, BV, lens, sc = _case(1)
    BK2, BV2 = np.stack([BK[0], BK[0]]), np.stack([BV[0], BV[0]])
    for ni in (0, 5, 30):
        _close(dec(q, LK, LV, BK2, BV2, lens, ni, scales=sc),
               oracle.decode(q, LK, LV, BK[0], BV[0], lens, scales=sc))


def pin_whole_sequence_one_set(dec):
    for lt in ("bf16", "i8"):
        q, LK, LV, BK, BV, lens, sc = _case(2, lt=lt)
        _close(dec(q, LK, LV, BK, BV, lens, 0, scales=sc),
               oracle.decode(q, LK, LV, BK[1], BV[1], lens, scales=sc))
        _close(dec(q, LK, LV, BK, BV, lens, 30, scales=sc),
               oracle.decode(q, LK, LV, BK[0], BV[0], lens, scales=sc))


def pin_widened_latent(dec):
    for lt, ni in (("bf16", 7), ("i8", 12), ("bf16", 1)):
        q, LK, LV, BK, BV, lens, sc = _case(3, lt=lt)
        T = LK.shape[2]
        img = (np.arange(T) < ni)[None, None, :, None]
        wide = lambda L: np.concatenate([np.where(img, L, 0.0), np.where(img, 0.0, L)], axis=3)
        BKw = np.concatenate([BK[0], BK[1]], axis=1)      # [Hkv, 2r, d]
        BVw = np.concatenate([BV[0], BV[1]], axis=1)
        _close(dec(q, LK, LV, BK, BV, lens, ni, scales=sc),
               oracle.decode(q, wide(LK), wide(LV), BKw, BVw, lens, scales=sc))


PINS = [pin_equal_sets_is_decode, pin_whole_sequence_one_set, pin_widened_latent]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_modal_pin(pin):
    pin(oracle.decode_modal)


def _mutant(kind):
    """decode_modal with one planted mistake, restated from its definition."""
    def dec(q, L_K, L_V, B_K, B_V, seq_lens, image_tokens, scales=None, softmax_scale=None):
        Bsz, Hq, d = q.shape
        Hkv = L_K.shape[1]
        out = np.empty((Bsz, Hq, d))
        for b in range(Bsz):
            n = int(seq_lens[b])
            ni = min(image_tokens + (1 if kind == "boundary" else 0), n)
            for h in range(Hq):
                g = h // (Hq // Hkv)
                sK = scales[0, b, g, :n] if scales is not None else None
                sV = scales[1, b, g, :n] if scales is not None else None
                Lk = oracle.dequantize(L_K[b, g, :n], sK)
                Lv = oracle.dequantize(L_V[b, g, :n], sV)
                if kind == "image_last":
                    k_parts = [Lk[:n - ni] @ B_K[1, g], Lk[n - ni:] @ B_K[0, g]]
                    v_parts = [Lv[:n - ni] @ B_V[1, g], Lv[n - ni:] @ B_V[0, g]]
                else:
                    vi = 1 if kind == "v_text_set" else 0
                    k_parts = [Lk[:ni] @ B_K[0, g], Lk[ni:] @ B_K[1, g]]
                    v_parts = [Lv[:ni] @ B_V[vi, g], Lv[ni:] @ B_V[1, g]]
                out[b, h] = oracle.attend(q[b, h], np.concatenate(k_parts),
                                          np.concatenate(v_parts), 1.0 / np.sqrt(d))
        return out
    return dec


@pytest.mark.parametrize("kind", ["boundary", "image_last", "v_text_set"])
def test_planted_modal_mistakes_are_caught(kind):
    dec = _mutant(kind)
    caught = 0
    for pin in PINS:
        try:
            pin(dec)
        except AssertionError:
            caught += 1
    assert caught >= 1, kind

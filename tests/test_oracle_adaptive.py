"""Pins for the oracle's attention-aware adaptive-rank decode (CPU only).

AttentionPack page, section 2.B: tokens with a high moving-average attention
score are rebuilt at full rank, the others at a reduced rank, and the step
updates the score.  decode_adaptive is pinned by:
  - reductions to the pinned decode: every token at full rank (threshold
    -inf) is decode; every token at low rank (threshold +inf) is decode of
    the cache cut to its first low_rank coordinates; a mixed cache is decode
    of the cache whose low-importance rows have coordinates >= low_rank set to
    zero (a score equal to the threshold counts as important); low_rank = r
    ignores the threshold;
  - closed forms of the update: with q = 0 every attention weight is 1/n, so
    importance' = decay * importance + (1 - decay) / n; with decay = 1 the
    score is unchanged; entries past seq_len never change;
  - an invariant: each head's weights sum to one, so for every (b, g)
    sum_t (importance' - decay * importance) = 1 - decay.
Planted mistakes must each fail one pin.
"""
import numpy as np
import pytest

import oracle
import workloads


def _case(seed, lt="bf16", lens=(24, 9, 1), T=24, r=8):
    base = "int8" if lt == "i8" else "gqa_vlm"
    w = workloads.make(base, seed=seed, B=len(lens), Hq=4, Hkv=2, d=16, r=r, T=T,
                       seq_lens=list(lens), factor_std=0.35, q_std=2.0)
    f = oracle.as_float64
    rng = np.random.default_rng(seed)
    imp = rng.uniform(0.0, 1.0, (len(lens), 2, T))
    return (f(w.q, w.q_dtype), f(w.L_K, w.latent_dtype), f(w.L_V, w.latent_dtype),
            f(w.B_K, w.factor_dtype), f(w.B_V, w.factor_dtype), w.seq_lens,
            None if w.scales is None else w.scales.astype(np.float64), imp)


def _close(got, ref, tol=1e-13):
    assert np.abs(got - ref).max() <= tol * max(np.abs(ref).max(), 1e-300)


def pin_full_rank_is_decode(dec):
    for lt in ("bf16", "i8"):
        q, LK, LV, BK, BV, lens, sc, imp = _case(1, lt)
        out, _ = dec(q, LK, LV, BK, BV, lens, imp, -np.inf, 3, 0.5, scales=sc)
        _close(out, oracle.decode(q, LK, LV, BK, BV, lens, scales=sc))
        out, _ = dec(q, LK, LV, BK, BV, lens, imp, np.inf, LK.shape[3], 0.5, scales=sc)
        _close(out, oracle.decode(q, LK, LV, BK, BV, lens, scales=sc))


def pin_low_rank_is_cut_cache(dec):
    q, LK, LV, BK, BV, lens, sc, imp = _case(2)
    k = 3
    out, _ = dec(q, LK, LV, BK, BV, lens, imp, np.inf, k, 0.5, scales=sc)
    _close(out, oracle.decode(q, LK[..., :k], LV[..., :k], BK[:, :k], BV[:, :k], lens,
                              scales=sc))


def pin_mixed_is_zeroed_cache(dec):
    for lt, k, tau, ties in (("bf16", 5, 0.5, False), ("i8", 2, 0.3, False),
                             ("bf16", 1, 0.7, False), ("bf16", 4, 0.5, True)):
        q, LK, LV, BK, BV, lens, sc, imp = _case(3, lt)
        if ties:   # scores on a grid holding the threshold itself: equal means full rank
            imp = np.round(imp * 4) / 4
        low = (imp < tau)[..., None] & (np.arange(LK.shape[3]) >= k)
        out, _ = dec(q, LK, LV, BK, BV, lens, imp, tau, k, 0.5, scales=sc)
        _close(out, oracle.decode(q, np.where(low, 0.0, LK), np.where(low, 0.0, LV), BK, BV,
                                  lens, scales=sc))


def pin_uniform_attention_update(dec):
    q, LK, LV, BK, BV, lens, sc, imp = _case(4)
    for decay in (0.0, 0.25, 0.9):
        _, new = dec(np.zeros_like(q), LK, LV, BK, BV, lens, imp, 0.5, 3, decay, scales=sc)
        for b, n in enumerate(lens):
            _close(new[b, :, :n], decay * imp[b, :, :n] + (1 - decay) / n)
            assert np.array_equal(new[b, :, n:], imp[b, :, n:])


def pin_weights_sum_to_one(dec):
    for lt in ("bf16", "i8"):
        q, LK, LV, BK, BV, lens, sc, imp = _case(5, lt)
        for decay in (0.0, 0.8):
            _, new = dec(q, LK, LV, BK, BV, lens, imp, 0.4, 2, decay, scales=sc)
            for b, n in enumerate(lens):
                tot = (new[b, :, :n] - decay * imp[b, :, :n]).sum(axis=1)
                _close(tot, np.full(2, 1.0 - decay))
        _, same = dec(q, LK, LV, BK, BV, lens, imp, 0.4, 2, 1.0, scales=sc)
        assert np.array_equal(same, imp)


PINS = [pin_full_rank_is_decode, pin_low_rank_is_cut_cache, pin_mixed_is_zeroed_cache,
        pin_uniform_attention_update, pin_weights_sum_to_one]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_adaptive_pin(pin):
    pin(oracle.decode_adaptive)


def _mutant(kind):
    """decode_adaptive with one planted mistake, restated from its definition."""
    def dec(q, L_K, L_V, B_K, B_V, seq_lens, importance, threshold, low_rank, decay,
            scales=None, softmax_scale=None):
        Bsz, Hq, d = q.shape
        _, Hkv, T, r = L_K.shape
        G = Hq // Hkv
        out = np.empty((Bsz, Hq, d))
        imp = importance.copy()
        for b in range(Bsz):
            n = int(seq_lens[b])
            for g in range(Hkv):
                sK = scales[0, b, g, :n] if scales is not None else None
                sV = scales[1, b, g, :n] if scales is not None else None
                Lk = oracle.dequantize(L_K[b, g, :n], sK)
                Lv = oracle.dequantize(L_V[b, g, :n], sV)
                cmp = importance[b, g, :n] > threshold if kind == "strict" else \
                    importance[b, g, :n] >= threshold
                kk = np.where(cmp, r, low_rank)
                if kind == "flipped":
                    kk = np.where(cmp, low_rank, r)
                K = np.stack([Lk[t, :kk[t]] @ B_K[g, :kk[t]] for t in range(n)])
                kv = np.full(n, r) if kind == "v_full" else kk
                V = np.stack([Lv[t, :kv[t]] @ B_V[g, :kv[t]] for t in range(n)])
                a = np.zeros(n)
                for h in range(g * G, (g + 1) * G):
                    s_ = (K @ q[b, h]) / np.sqrt(d)
                    e = np.exp(s_ - s_.max())
                    prob = e / e.sum()
                    out[b, h] = prob @ V
                    a += prob if kind == "head_sum" else prob / G
                if kind == "decay_swapped":
                    imp[b, g, :n] = (1 - decay) * importance[b, g, :n] + decay * a
                else:
                    imp[b, g, :n] = decay * importance[b, g, :n] + (1 - decay) * a
        return out, imp
    return dec


@pytest.mark.parametrize("kind", ["flipped", "v_full", "head_sum", "decay_swapped", "strict"])
def test_planted_adaptive_mistakes_are_caught(kind):
    dec = _mutant(kind)
    caught = 0
    for pin in PINS:
        try:
            pin(dec)
        except AssertionError:
            caught += 1
    assert caught >= 1, kind


def test_clean_restatement_passes():
    dec = _mutant("none")
    for pin in PINS:
        pin(dec)

"""Each plausible mistake planted in a copy of the oracle must fail a pin (CPU only).

The copies below restate the oracle's definition with exactly one planted
mistake each.  If a mistake slipped through every pin, the pins would not be
strong enough to trust the oracle; this test guards against that.
"""
import numpy as np
import pytest

import oracle_pins as P


def make_mutant(kind):
    def decode(q, L_K, L_V, B_K, B_V, seq_lens, scales=None, softmax_scale=None):
        Bsz, Hq, d = q.shape
        _, Hkv, T, r = L_K.shape
        G = Hq // Hkv
        if softmax_scale is not None:
            alpha = softmax_scale
        elif kind == "alpha_rank":
            alpha = 1.0 / np.sqrt(r)
        elif kind == "alpha_missing":
            alpha = 1.0
        else:
            alpha = 1.0 / np.sqrt(d)
        out = np.zeros((Bsz, Hq, d))
        for b in range(Bsz):
            n = int(seq_lens[b])
            if kind == "len_plus_one":
                n = min(n + 1, T)
            if kind == "len_minus_one":
                n = max(n - 1, 1)
            for h in range(Hq):
                g = h % Hkv if kind == "gqa_modulo" else h // G
                lk = L_K[b, g, :n].copy()
                lv = (L_K if kind == "v_from_key_latent" else L_V)[b, g, :n].copy()
                if scales is not None and kind != "no_dequant":
                    lk *= scales[0, b, g, :n][:, None]
                    vs = 0 if kind == "k_scale_for_v" else 1
                    lv *= scales[vs, b, g, :n][:, None]
                bk = B_K[g]
                bv = B_K[g] if kind == "v_uses_bk" else B_V[g]
                if kind == "factor_layout":
                    bk = bk.reshape(d, r).T
                K = lk @ bk
                V = lv @ bv
                qv = q[b, g] if kind == "kv_head_query" else q[b, h]
                s = alpha * (K @ qv)
                if kind == "sign_flip":
                    s = -s
                e = np.exp(s - s.max())
                p = e if kind == "no_normalize" else e / e.sum()
                out[b, h] = p @ V
        return out
    return decode


MUTANTS = ["alpha_rank", "alpha_missing", "len_plus_one", "len_minus_one",
           "gqa_modulo", "v_from_key_latent", "no_dequant", "k_scale_for_v",
           "v_uses_bk", "factor_layout", "kv_head_query", "sign_flip",
           "no_normalize"]


def test_unmutated_copy_passes():
    dec = make_mutant(None)
    for pin in P.ALL_PINS:
        pin(dec)


@pytest.mark.parametrize("kind", MUTANTS)
def test_mutant_is_caught(kind):
    dec = make_mutant(kind)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(dec)
        except Exception:  # an assertion or a shape error both expose the mistake
            caught.append(pin.__name__)
    assert caught, f"planted mistake {kind!r} passed every pin"

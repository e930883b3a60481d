"""The oracle's rotated-key decode against its pins, and planted mistakes
against the same pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_rotary_pins as P


@pytest.mark.parametrize("pin", P.ALL_ROTARY_PINS, ids=lambda f: f.__name__)
def test_oracle_rotary_pin(pin):
    pin(oracle.decode_rotated)


def make_mutant(kind):
    """decode_rotated restated with one planted mistake."""
    def rot(x, row):
        h = x.shape[-1] // 2
        c, s = row[..., :h], row[..., h:]
        if kind == "cos_sin_swapped":
            c, s = s, c
        if kind == "interleaved_pairs":
            a, b = x[..., 0::2], x[..., 1::2]
            y = np.empty_like(x)
            y[..., 0::2], y[..., 1::2] = a * c - b * s, a * s + b * c
            return y
        a, b = x[..., :h], x[..., h:]
        if kind == "sign":
            s = -s
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)

    def dec(q, LK, LV, BK, BV, lens, rope, scales=None, softmax_scale=None):
        Bsz, Hq, d = q.shape
        Hkv, T = LK.shape[1], LK.shape[2]
        G = Hq // Hkv
        alpha = softmax_scale if softmax_scale is not None else 1.0 / np.sqrt(d)
        out = np.zeros((Bsz, Hq, d))
        for b in range(Bsz):
            n = int(lens[b])
            for g in range(Hkv):
                lk, lv = LK[b, g, :n], LV[b, g, :n]
                if scales is not None:
                    lk = lk * scales[0, b, g, :n, None]
                    lv = lv * scales[1, b, g, :n, None]
                kpos = np.minimum(np.arange(n) + (1 if kind == "key_pos_plus_one" else 0), T - 1)
                K = lk @ BK[g]
                K = K if kind == "keys_unrotated" else rot(K, rope[kpos])
                V = lv @ BV[g]
                if kind == "values_rotated":
                    V = rot(V, rope[:n])
                qpos = min(n, T - 1) if kind == "query_pos_n" else n - 1
                for h in range(g * G, (g + 1) * G):
                    qq = q[b, h] if kind == "query_unrotated" else rot(q[b, h], rope[qpos])
                    s = alpha * (K @ qq)
                    e = np.exp(s - s.max())
                    out[b, h] = (e / e.sum()) @ V
        return out
    return dec


MUTANTS = ["cos_sin_swapped", "interleaved_pairs", "sign", "key_pos_plus_one",
           "keys_unrotated", "values_rotated", "query_pos_n", "query_unrotated"]


def test_unmutated_copy_passes():
    for pin in P.ALL_ROTARY_PINS:
        pin(make_mutant(None))


@pytest.mark.parametrize("kind", MUTANTS)
def test_rotary_mutant_is_caught(kind):
    caught = []
    for pin in P.ALL_ROTARY_PINS:
        try:
            pin(make_mutant(kind))
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {kind!r} passed every pin"

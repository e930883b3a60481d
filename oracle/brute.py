"""Brute-force check of the oracle in 40-digit decimal arithmetic.

TEST INFRASTRUCTURE.  Only the tests may import this module.

Plain nested loops over Python `decimal.Decimal` values, written straight from
the definition (WSVD page, section 2.A: per-head latent times per-head factor
rebuilds K and V; section 2.C: attention over the rebuilt keys and values):

    K[t][i] = sum_j Lk[t][j] * Bk[j][i]          (after Lk[t][j] *= sK[t] for int8)
    s[t]    = alpha * sum_i q[i] * K[t][i]
    p[t]    = exp(s[t]) / sum_u exp(s[u])
    o[i]    = sum_t p[t] * V[t][i]

`Decimal.exp` is correctly rounded at the context precision, so with 40
significant digits the result is exact far beyond float64.  Inputs are
converted from float64 exactly (Decimal(float) is exact).  For tiny shapes only.
"""
from __future__ import annotations

from decimal import Decimal, getcontext, localcontext
from typing import List, Optional

__all__ = ["decode_decimal"]


def _D(x) -> Decimal:
    return Decimal(float(x))


def decode_decimal(q, L_K, L_V, B_K, B_V, seq_lens, scales=None,
                   softmax_scale: Optional[float] = None, digits: int = 40):
    """Nested lists out[b][h][i] of Decimal.  Arguments as float64 numpy arrays."""
    Bsz, Hq, d = q.shape
    _, Hkv, T, r = L_K.shape
    group = Hq // Hkv
    out: List = []
    with localcontext() as ctx:
        ctx.prec = digits
        if softmax_scale is None:
            alpha = Decimal(1) / Decimal(d).sqrt()
        else:
            alpha = _D(softmax_scale)
        for b in range(Bsz):
            n = int(seq_lens[b])
            rows_b = []
            for h in range(Hq):
                g = h // group
                # rebuild K and V for this sequence's valid tokens
                K = []
                V = []
                for t in range(n):
                    sk = _D(scales[0][b][g][t]) if scales is not None else Decimal(1)
                    sv = _D(scales[1][b][g][t]) if scales is not None else Decimal(1)
                    krow = []
                    vrow = []
                    for i in range(d):
                        acc_k = Decimal(0)
                        acc_v = Decimal(0)
                        for j in range(r):
                            acc_k += (sk * _D(L_K[b][g][t][j])) * _D(B_K[g][j][i])
                            acc_v += (sv * _D(L_V[b][g][t][j])) * _D(B_V[g][j][i])
                        krow.append(acc_k)
                        vrow.append(acc_v)
                    K.append(krow)
                    V.append(vrow)
                s = []
                for t in range(n):
                    acc = Decimal(0)
                    for i in range(d):
                        acc += _D(q[b][h][i]) * K[t][i]
                    s.append(alpha * acc)
                ex = [x.exp() for x in s]
                z = sum(ex, Decimal(0))
                o = []
                for i in range(d):
                    acc = Decimal(0)
                    for t in range(n):
                        acc += ex[t] * V[t][i]
                    o.append(acc / z)
                rows_b.append(o)
            out.append(rows_b)
    return out

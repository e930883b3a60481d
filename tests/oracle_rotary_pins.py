"""Pins for the rotated-key decode of the oracle (CPU only).

Each pin takes a function with the signature of oracle.decode_rotated and
checks it against something fixed independently of it: hand-derived closed
forms in 2 and 4 dimensions, the already-pinned unrotated decode (zero angles,
and explicitly rotated inputs built from 2x2 rotation blocks as dense
matrices), and the invariance of rotary scores under a common shift of all
positions.  The rotary definition: coordinates j and j + d/2 form a pair,
rotated by the angle whose cosine / sine are rope[p, j] / rope[p, d/2 + j];
key row t takes position t, the query position seq_len - 1.
"""
import numpy as np

import oracle
import workloads


def _small(seed, lt="bf16", lens=(37, 5, 1), d=16, r=8, G=2):
    kw = dict(B=len(lens), Hq=2 * G, Hkv=2, d=d, r=r, T=40, seq_lens=list(lens),
              factor_std=1.0 / np.sqrt(r), q_std=2.0)
    base = "int8" if lt == "i8" else "gqa_vlm"
    if lt != "i8":
        kw["latent_dtype"] = lt
    w = workloads.make(base, seed=seed, **kw)
    f = lambda a, t: oracle.as_float64(a, t)
    sc = None if w.scales is None else w.scales.astype(np.float64)
    return (f(w.q, w.q_dtype), f(w.L_K, w.latent_dtype), f(w.L_V, w.latent_dtype),
            f(w.B_K, w.factor_dtype), f(w.B_V, w.factor_dtype), w.seq_lens, sc)


def _exact_table(T, d, offset=0, base=10.0):
    """float64 rotary table from exact trigonometry (not rounded)."""
    j = np.arange(d // 2)
    ang = (np.arange(T)[:, None] + offset) * base ** (-2.0 * j / d)
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def pin_rot_zero_angles(dec):
    q, LK, LV, BK, BV, lens, sc = _small(1)
    T, d = LK.shape[2], q.shape[2]
    rope = np.concatenate([np.ones((T, d // 2)), np.zeros((T, d // 2))], axis=1)
    got = dec(q, LK, LV, BK, BV, lens, rope, scales=sc)
    ref = oracle.decode(q, LK, LV, BK, BV, lens, scales=sc)
    assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()


def pin_rot_closed_2d(dec):
    # d = 2, keys (0,1) at position 0 and (1,0) at position 1, values e0, e1,
    # query (1,0) at position 1 rotated by theta: scores sin(theta) and 1
    th = 0.7
    q = np.array([[[1.0, 0.0]]])
    LK = np.array([[[[0.0, 1.0], [1.0, 0.0]]]])
    LV = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    I = np.eye(2)[None]
    rope = np.array([[1.0, 0.0], [np.cos(th), np.sin(th)]])
    got = dec(q, LK, LV, I, I, np.array([2]), rope, softmax_scale=1.0)
    e = np.exp([np.sin(th), 1.0])
    want = e / e.sum()
    assert np.allclose(got[0, 0], want, rtol=0, atol=1e-15), (got, want)


def pin_rot_pairing_4d(dec):
    # d = 4: pairs (0,2) and (1,3).  q = e0 at position 1 (angles a, b), keys
    # e2 at position 0 and e1 at position 1: scores sin(a) and 0
    a, b = 0.4, 1.1
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    LK = np.array([[[[0.0, 0.0, 1.0, 0.0], [0.0, 1.0, 0.0, 0.0]]]])
    LV = np.array([[[[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]]]])
    I = np.eye(4)[None]
    rope = np.array([[1.0, 1.0, 0.0, 0.0],
                     [np.cos(a), np.cos(b), np.sin(a), np.sin(b)]])
    got = dec(q, LK, LV, I, I, np.array([2]), rope, softmax_scale=1.0)
    e = np.exp([np.sin(a), 0.0])
    want = np.array([e[0], e[1], 0.0, 0.0]) / e.sum()
    assert np.allclose(got[0, 0], want, rtol=0, atol=1e-15), (got, want)


def _rotation_matrix(row):
    h = row.shape[0] // 2
    c, s = np.diag(row[:h]), np.diag(row[h:])
    return np.block([[c, -s], [s, c]])


def pin_rot_matrix_form(dec):
    # rotate explicitly with dense rotation matrices, then run the pinned
    # unrotated decode on the rotated dense keys (identity factors)
    for lt in ("bf16", "i8"):
        q, LK, LV, BK, BV, lens, sc = _small(2, lt)
        Bsz, Hq, d = q.shape
        _, Hkv, T, r = LK.shape
        rope = workloads.rope_table(T, d, base=100.0).astype(np.float64)
        G = Hq // Hkv
        Kd = np.zeros((Bsz, Hkv, T, d))
        Vd = np.zeros((Bsz, Hkv, T, d))
        qr = np.zeros_like(q)
        for b in range(Bsz):
            n = int(lens[b])
            for g in range(Hkv):
                lk, lv = LK[b, g, :n], LV[b, g, :n]
                if sc is not None:
                    lk = lk * sc[0, b, g, :n, None]
                    lv = lv * sc[1, b, g, :n, None]
                for t in range(n):
                    Kd[b, g, t] = _rotation_matrix(rope[t]) @ (lk[t] @ BK[g])
                Vd[b, g, :n] = lv @ BV[g]
                for h in range(g * G, (g + 1) * G):
                    qr[b, h] = _rotation_matrix(rope[n - 1]) @ q[b, h]
        I = np.broadcast_to(np.eye(d), (Hkv, d, d))
        ref = oracle.decode(qr, Kd, Vd, I, I, lens, softmax_scale=1.0 / np.sqrt(d))
        got = dec(q, LK, LV, BK, BV, lens, rope, scales=sc)
        assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max(), lt


def pin_rot_shift(dec):
    # rotary scores depend on position differences only: a common shift of all
    # positions (exact trigonometry) leaves the output unchanged
    q, LK, LV, BK, BV, lens, sc = _small(3)
    T, d = LK.shape[2], q.shape[2]
    a = dec(q, LK, LV, BK, BV, lens, _exact_table(T, d, 0), scales=sc)
    b = dec(q, LK, LV, BK, BV, lens, _exact_table(T, d, 37), scales=sc)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


ALL_ROTARY_PINS = [pin_rot_zero_angles, pin_rot_closed_2d, pin_rot_pairing_4d,
                   pin_rot_matrix_form, pin_rot_shift]

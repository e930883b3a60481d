"""fp64 CPU oracle: single-token decode attention over a per-head low-rank KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and imports nothing from it.

What is computed, and where the pages define it
-----------------------------------------------
* WSVD page ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
  Execution of Low-Precision Vision-Language Models"), section 2.A (per-head
  SVD): each head's key projection is factored into two matrices of rank r,
  so the cache keeps, per token and head, a compact latent row, and each head
  is rebuilt from its own latent: K_h = L_Kh . B_Kh with L_Kh of shape T x r and
  B_Kh of shape r x d.  The same holds for V.
* AttentionPack page, section 2.A: a compressed cache times a decompression
  matrix approximates K (and V): K ~ K* . D_k*.  Same product, read per head.
* WSVD page, section 2.C: the decode kernel fuses this low-rank rebuild with
  the attention computation and Flash Decoding.  The fused kernel's result is
  by definition the result of rebuilding K and V and running ordinary
  single-query softmax attention, which is what this oracle does, in that
  order, in float64.
* WSVD page, sections 2.C and 4 (W8A8): low-precision latents.  Read here as
  symmetric int8 latents with one fp32 scale per (batch, kv-head, token),
  separate for K and V; dequantization is scale * integer.

Readings where the pages are silent (each is listed in the design notes):
  - query head h uses kv-head g = h // (Hq / Hkv) (consecutive groups);
  - softmax scale defaults to 1 / sqrt(d);
  - no positional rotation between rebuild and scoring in decode();
    decode_rotated() below adds one (its reading is stated there);
  - the current token is already in the cache: attend to rows [0, seq_len);
  - seq_len <= 0 has no defined result: the oracle raises ValueError.

Every function here is pinned by CPU tests against brute force in 40-digit
decimal arithmetic, closed forms, hand-derived fixtures, a library attention
routine, and invariants; none of the pins reuses this code.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = ["as_float64", "dequantize", "rebuild", "attend", "decode",
           "decode_rows", "decode_absorbed", "rotate", "decode_rotated", "decode_shared",
           "decode_modal", "decode_adaptive"]


def as_float64(a: np.ndarray, tag: str) -> np.ndarray:
    """Exact float64 values of a stored tensor.

    tag "f32" float32, "f16" float16, "i8" int8 (integer values) and "bf16"
    given as raw uint16 bit patterns: a bfloat16 is the top half of a binary32,
    so its value is the binary32 whose high 16 bits are those bits.  Every one
    of these types embeds exactly in binary64.
    """
    if tag == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if tag in ("f32", "f16", "i8"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(f"unknown dtype tag {tag!r}")


def dequantize(L: np.ndarray, scale: Optional[np.ndarray]) -> np.ndarray:
    """Latent rows as real values: scale[t] * L[t, :] for int8 rows, else L.

    L     [n, r] float64 (integer-valued for int8 latents)
    scale [n]    float64 or None
    """
    if scale is None:
        return L
    return L * scale[:, None]


def rebuild(L: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Explicit per-head rebuild of keys (or values): [n, r] @ [r, d] -> [n, d]."""
    return L @ B


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, alpha: float) -> np.ndarray:
    """Single-query softmax attention in float64.

    q [d], K [n, d], V [n, d]:  s = alpha * K q;  p = softmax(s);  return p^T V.
    """
    s = alpha * (K @ q)
    s = s - s.max()
    e = np.exp(s)
    p = e / e.sum()
    return p @ V


def _check_shapes(q, L_K, L_V, B_K, B_V, seq_lens, scales):
    if q.ndim != 3 or L_K.ndim != 4 or B_K.ndim != 3:
        raise ValueError("q [B,Hq,d], L [B,Hkv,T,r], B [Hkv,r,d] expected")
    Bsz, Hq, d = q.shape
    B2, Hkv, T, r = L_K.shape
    if L_V.shape != L_K.shape or B_K.shape != (Hkv, r, d) or B_V.shape != B_K.shape:
        raise ValueError("inconsistent shapes")
    if B2 != Bsz or Hq % Hkv:
        raise ValueError("batch mismatch or Hq not a multiple of Hkv")
    if np.asarray(seq_lens).shape != (Bsz,):
        raise ValueError("seq_lens must have shape [B]")
    if scales is not None and scales.shape != (2, Bsz, Hkv, T):
        raise ValueError("scales must have shape [2, B, Hkv, T]")
    return Bsz, Hq, Hkv, T, r, d


def decode_rows(q, L_K, L_V, B_K, B_V, seq_lens, rows: Iterable[Tuple[int, int]],
                scales=None, softmax_scale: Optional[float] = None) -> np.ndarray:
    """Output rows out[b, h, :] for the listed (b, h) pairs, float64 [len(rows), d].

    Inputs are float64 arrays (see as_float64); L_K/L_V hold integer values and
    `scales` is given when the latents are int8.  Only rows [0, seq_len_b) of a
    sequence are read.
    """
    Bsz, Hq, Hkv, T, r, d = _check_shapes(q, L_K, L_V, B_K, B_V, seq_lens, scales)
    group = Hq // Hkv
    alpha = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(d)
    rows = list(rows)
    out = np.empty((len(rows), d), dtype=np.float64)
    cache = {}
    for i, (b, h) in enumerate(rows):
        n = int(seq_lens[b])
        if n <= 0:
            raise ValueError(f"seq_len {n} for batch {b}: attention over no tokens")
        if n > T:
            raise ValueError(f"seq_len {n} exceeds the cache length {T}")
        g = h // group
        key = (b, g)
        if key not in cache:
            sK = scales[0, b, g, :n] if scales is not None else None
            sV = scales[1, b, g, :n] if scales is not None else None
            K = rebuild(dequantize(L_K[b, g, :n], sK), B_K[g])
            V = rebuild(dequantize(L_V[b, g, :n], sV), B_V[g])
            cache = {key: (K, V)}          # keep one (b, g) at a time
        K, V = cache[key]
        out[i] = attend(q[b, h], K, V, alpha)
    return out


def decode(q, L_K, L_V, B_K, B_V, seq_lens, scales=None,
           softmax_scale: Optional[float] = None) -> np.ndarray:
    """Every output row, float64 [B, Hq, d]."""
    Bsz, Hq = q.shape[0], q.shape[1]
    rows = [(b, h) for b in range(Bsz) for h in range(Hq)]
    return decode_rows(q, L_K, L_V, B_K, B_V, seq_lens, rows, scales,
                       softmax_scale).reshape(Bsz, Hq, -1)


def decode_absorbed(q, L_K, L_V, B_K, B_V, seq_lens, scales=None,
                    softmax_scale: Optional[float] = None) -> np.ndarray:
    """Same quantity through the factored route, float64 [B, Hq, d].

    q.(L_K[t] B_K)^T = (q B_K^T).L_K[t]^T and sum_t p_t (L_V[t] B_V) =
    (sum_t p_t L_V[t]) B_V, by associativity of the matrix product.  This route
    never forms K or V; the oracle keeps it only so tests can confirm, in
    float64, that the identity holds on the same inputs.
    """
    Bsz, Hq, Hkv, T, r, d = _check_shapes(q, L_K, L_V, B_K, B_V, seq_lens, scales)
    group = Hq // Hkv
    alpha = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(d)
    out = np.empty((Bsz, Hq, d), dtype=np.float64)
    for b in range(Bsz):
        n = int(seq_lens[b])
        if n <= 0 or n > T:
            raise ValueError(f"seq_len {n} out of range")
        for h in range(Hq):
            g = h // group
            sK = scales[0, b, g, :n] if scales is not None else None
            sV = scales[1, b, g, :n] if scales is not None else None
            qt = B_K[g] @ q[b, h]                      # [r]
            s = alpha * (dequantize(L_K[b, g, :n], sK) @ qt)
            e = np.exp(s - s.max())
            p = e / e.sum()
            vt = p @ dequantize(L_V[b, g, :n], sV)      # [r]
            out[b, h] = vt @ B_V[g]
    return out


# ---------------------------------------------------------------- rotated keys
#
# A position-dependent rotation between the rebuild and the score.  The pages
# do not name one; WSVD section 2.C rebuilds K on chip before scoring, which is
# the form a rotation needs (q . B_K^T no longer absorbs it).  Reading taken
# (listed in the design notes): the rotary embedding with rotate-half pairing,
# i.e. coordinates j and j + d/2 form a pair, and the caller supplies the
# per-position cosines and sines as a table; key row t is rotated with the
# table row of position t, the query with the row of its own position
# seq_len - 1 (it is the last token in the cache); values are not rotated.


def rotate(x: np.ndarray, row: np.ndarray) -> np.ndarray:
    """Rotate each pair (x[j], x[j + d/2]) by the angle whose cosine is
    row[j] and sine is row[d/2 + j]:  (a, b) -> (a cos - b sin, a sin + b cos).

    x [..., d] float64 (d even), row [..., d] float64 (cosines, then sines)."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = row[..., :h], row[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def decode_rotated(q, L_K, L_V, B_K, B_V, seq_lens, rope, scales=None,
                   softmax_scale: Optional[float] = None) -> np.ndarray:
    """Decode with rotated keys, float64 [B, Hq, d].

    rope [T, d] float64: row p = cosines of the d/2 angles at position p, then
    their sines.  For sequence b with n = seq_len_b: K[t] = rotate(L_K[t] B_K,
    rope[t]) for t < n, q' = rotate(q, rope[n - 1]), V[t] = L_V[t] B_V, and
    out = softmax(alpha K q') V.
    """
    Bsz, Hq, Hkv, T, r, d = _check_shapes(q, L_K, L_V, B_K, B_V, seq_lens, scales)
    if rope.shape != (T, d) or d % 2:
        raise ValueError("rope must be [T, d] with d even")
    group = Hq // Hkv
    alpha = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(d)
    out = np.empty((Bsz, Hq, d), dtype=np.float64)
    for b in range(Bsz):
        n = int(seq_lens[b])
        if n <= 0 or n > T:
            raise ValueError(f"seq_len {n} out of range")
        for g in range(Hkv):
            sK = scales[0, b, g, :n] if scales is not None else None
            sV = scales[1, b, g, :n] if scales is not None else None
            K = rotate(rebuild(dequantize(L_K[b, g, :n], sK), B_K[g]), rope[:n])
            V = rebuild(dequantize(L_V[b, g, :n], sV), B_V[g])
            for h in range(g * group, (g + 1) * group):
                out[b, h] = attend(rotate(q[b, h], rope[n - 1]), K, V, alpha)
    return out


# ------------------------------------------------------------ shared latent
#
# AttentionPack page, section 2.A (multi-head compression): the keys (values)
# of all heads are joined along the head axis and factored once, so the cache
# keeps one compressed row of R values per token, shared by the heads, and a
# decompression matrix of R x (H d) whose column block h rebuilds head h.
# Read here per latent stream: query head h attends to stream
# s = h // (Hq / S) and rebuilds its keys (values) with its own block
# B_K[h] (B_V[h]), R x d.  (S = 1 is the page's single shared cache.)


def decode_shared(q, L_K, L_V, B_K, B_V, seq_lens, scales=None,
                  softmax_scale: Optional[float] = None) -> np.ndarray:
    """Decode over shared latent streams with per-query-head factors,
    float64 [B, Hq, d].  L_K, L_V [B, S, T, R]; B_K, B_V [Hq, R, d]."""
    Bsz, Hq, d = q.shape
    _, S, T, R = L_K.shape
    if L_V.shape != L_K.shape or B_K.shape != (Hq, R, d) or B_V.shape != B_K.shape:
        raise ValueError("inconsistent shapes")
    if Hq % S:
        raise ValueError("Hq must be a multiple of the number of latent streams")
    group = Hq // S
    alpha = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(d)
    out = np.empty((Bsz, Hq, d), dtype=np.float64)
    for b in range(Bsz):
        n = int(seq_lens[b])
        if n <= 0 or n > T:
            raise ValueError(f"seq_len {n} out of range")
        for h in range(Hq):
            s_ = h // group
            sK = scales[0, b, s_, :n] if scales is not None else None
            sV = scales[1, b, s_, :n] if scales is not None else None
            K = rebuild(dequantize(L_K[b, s_, :n], sK), B_K[h])
            V = rebuild(dequantize(L_V[b, s_, :n], sV), B_V[h])
            out[b, h] = attend(q[b, h], K, V, alpha)
    return out


def decode_modal(q, L_K, L_V, B_K, B_V, seq_lens, image_tokens: int, scales=None,
                 softmax_scale: Optional[float] = None) -> np.ndarray:
    """Decode with one pair of factors for the image block and another for
    the text, float64 [B, Hq, d].

    AttentionPack page, section 2.A: visual and textual tokens are compressed
    separately, since their statistics differ.  Reading: every sequence
    starts with an image block of `image_tokens` tokens (the same count for
    all sequences, as in the gqa_vlm workload's 576-token block); token t of a
    sequence uses factor set 0 when t < image_tokens and set 1 otherwise, for
    both K and V.  B_K, B_V [2, Hkv, r, d]; other arguments as in decode().
    Keys and values are rebuilt per token with the token's set, then the
    ordinary softmax attention of attend() runs over all of them.
    """
    Bsz, Hq, d = q.shape
    _, Hkv, T, r = L_K.shape
    if B_K.shape != (2, Hkv, r, d) or B_V.shape != B_K.shape or L_V.shape != L_K.shape:
        raise ValueError("B_K, B_V [2, Hkv, r, d] and L [B, Hkv, T, r] expected")
    if image_tokens < 0:
        raise ValueError("image_tokens must be >= 0")
    group = Hq // Hkv
    alpha = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(d)
    out = np.empty((Bsz, Hq, d), dtype=np.float64)
    for b in range(Bsz):
        n = int(seq_lens[b])
        if n <= 0 or n > T:
            raise ValueError(f"seq_len {n} out of range")
        ni = min(int(image_tokens), n)
        for h in range(Hq):
            g = h // group
            sK = scales[0, b, g, :n] if scales is not None else None
            sV = scales[1, b, g, :n] if scales is not None else None
            Lk = dequantize(L_K[b, g, :n], sK)
            Lv = dequantize(L_V[b, g, :n], sV)
            K = np.concatenate([rebuild(Lk[:ni], B_K[0, g]), rebuild(Lk[ni:], B_K[1, g])])
            V = np.concatenate([rebuild(Lv[:ni], B_V[0, g]), rebuild(Lv[ni:], B_V[1, g])])
            out[b, h] = attend(q[b, h], K, V, alpha)
    return out


def decode_adaptive(q, L_K, L_V, B_K, B_V, seq_lens, importance, threshold: float,
                    low_rank: int, decay: float, scales=None,
                    softmax_scale: Optional[float] = None):
    """Decode with a per-token rank chosen by an importance score, and the
    score's moving-average update, float64: (out [B, Hq, d], importance').

    AttentionPack page, section 2.B (attention-aware decompression): a moving
    average of each token's accumulated attention marks the important
    tokens; those are rebuilt with the full rank, the others with a reduced
    rank.  Readings: the latent coordinates are ordered by importance (the
    leading singular directions first), so rank k keeps coordinates [0, k) of
    the token's latent row and rows [0, k) of the factors, for K and V alike;
    token t of sequence b, kv-head g uses the full rank r when
    importance[b, g, t] >= threshold and low_rank otherwise; after the step,
    for t < seq_len, importance'[b, g, t] = decay * importance[b, g, t] +
    (1 - decay) * a_t with a_t the attention weight of token t averaged over
    the query heads of kv-head g (entries t >= seq_len are unchanged).

    importance [B, Hkv, T]; 1 <= low_rank <= r; 0 <= decay <= 1.
    """
    Bsz, Hq, d = q.shape
    _, Hkv, T, r = L_K.shape
    _check_shapes(q, L_K, L_V, B_K, B_V, seq_lens, scales)
    if importance.shape != (Bsz, Hkv, T):
        raise ValueError("importance must be [B, Hkv, T]")
    if not 1 <= low_rank <= r:
        raise ValueError("low_rank must be in [1, r]")
    group = Hq // Hkv
    alpha = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(d)
    out = np.empty((Bsz, Hq, d), dtype=np.float64)
    imp = np.array(importance, dtype=np.float64, copy=True)
    for b in range(Bsz):
        n = int(seq_lens[b])
        if n <= 0 or n > T:
            raise ValueError(f"seq_len {n} out of range")
        for g in range(Hkv):
            sK = scales[0, b, g, :n] if scales is not None else None
            sV = scales[1, b, g, :n] if scales is not None else None
            Lk = dequantize(L_K[b, g, :n], sK)
            Lv = dequantize(L_V[b, g, :n], sV)
            full = importance[b, g, :n] >= threshold
            K = np.empty((n, d))
            V = np.empty((n, d))
            for t in range(n):
                k = r if full[t] else low_rank
                K[t] = Lk[t, :k] @ B_K[g, :k]
                V[t] = Lv[t, :k] @ B_V[g, :k]
            a = np.zeros(n)
            for h in range(g * group, (g + 1) * group):
                s_ = alpha * (K @ q[b, h])
                e = np.exp(s_ - s_.max())
                prob = e / e.sum()
                out[b, h] = prob @ V
                a += prob / group
            imp[b, g, :n] = decay * importance[b, g, :n] + (1.0 - decay) * a
    return out, imp

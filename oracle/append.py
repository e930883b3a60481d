"""fp64 CPU oracle for the append step: a new token's latent rows.

TEST INFRASTRUCTURE (same rules as the rest of oracle/).

WSVD page, section 2.A: each head's key (value) projection is factored per
head, W_Kh = A_Kh . B_Kh with rank r, so the cache row of a new token with
hidden state x is its latent x . A_Kh (r values), the compact row the decode
later reads.  Section 2.C (quantization of the low-rank path, W8A8): latents
may be stored as int8.

Readings (listed in the design notes):
  - A_K, A_V are given per kv-head as [Hkv, r, D]: row j holds the D weights
    of latent coordinate j (the transpose of A_Kh, like B_K's [r, d] rows);
  - int8: symmetric, one scale per (sequence, kv-head, token), separate for K
    and V: s = max_j |l_j| / 127 and code_j = round-half-even(l_j / s), so the
    largest entry maps to +-127; an all-zero row has s = 0 and codes 0;
  - a sequence whose position lies outside [0, T) is not written.
"""
from __future__ import annotations

import numpy as np

__all__ = ["project", "quantize_rows", "append"]


def project(x: np.ndarray, A: np.ndarray) -> np.ndarray:
    """Latent rows x . A_h^T for every head, float64 [B, Hkv, r].

    x [B, D] float64, A [Hkv, r, D] float64."""
    return np.einsum("bd,grd->bgr", x, A)


def quantize_rows(L: np.ndarray):
    """Symmetric per-row int8 codes and scales of float64 rows [..., r]:
    s = max |row| / 127, code = round-half-even(row / s) (numpy's rint)."""
    m = np.abs(L).max(axis=-1)
    s = m / 127.0
    safe = np.where(s > 0, s, 1.0)
    codes = np.where(s[..., None] > 0, np.rint(L / safe[..., None]), 0.0)
    return codes, s


def append(x, A_K, A_V, positions, T: int, quantized: bool):
    """Latent rows of one new token per sequence.

    Returns (rows, scales, written): rows [2, B, Hkv, r] float64 (K then V;
    int8 codes as integer values when quantized), scales [2, B, Hkv] float64
    (None unless quantized), written [B] bool (position inside [0, T))."""
    rows = np.stack([project(x, A_K), project(x, A_V)])
    written = (np.asarray(positions) >= 0) & (np.asarray(positions) < T)
    if not quantized:
        return rows, None, written
    codes, scales = quantize_rows(rows)
    return codes, scales, written

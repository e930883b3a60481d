"""CPU oracle for low-rank-KV decode attention (float64 NumPy + decimal brute force).

TEST INFRASTRUCTURE.  Only `tests/`, `__graft_entry__.smoke()` and the
benchmark's CPU-baseline leg may import anything under `oracle/`.  The product
path (the HIP library and its Python binding) never imports it and has no CPU
fallback.

Modules
  lowrank_decode  the plain definition: dequantize, rebuild K and V
                  explicitly, dense softmax attention, in float64; and the
                  same with keys and query rotated by position (decode_rotated),
                  over shared latent streams (decode_shared), with separate
                  factors for the image block and the text (decode_modal), and
                  with a per-token rank chosen by a moving-average importance
                  score that the step updates (decode_adaptive)
  brute           the same definition in 40-digit decimal, nested loops,
                  for tiny inputs
  append          a new token's latent rows (projection, int8 quantization)

Parity status: every function is pinned (see the CPU tests); none is
"parity unpinned".
"""
from .lowrank_decode import (as_float64, attend, decode, decode_absorbed,  # noqa: F401
                             decode_adaptive, decode_modal, decode_rotated, decode_rows,
                             decode_shared, dequantize, rebuild, rotate)
from . import append as append_step  # noqa: F401,E402

"""Python binding of liblrattn: decode attention over a per-head low-rank KV cache.

Thin ctypes layer over the C-ABI declared in include/lrattn.h and
include/lrattn_probe.h.  It only marshals arguments: it reads shapes and
dtypes from torch tensors, passes their device pointers and the current HIP
stream, and raises LrattnError on a nonzero status.  Every step of the
computation runs in the library's gfx950 kernels; there is no fallback, and
a missing library raises at first use.

    out = decode(q, L_K, L_V, B_K, B_V, seq_lens, scales=None, ...)

Shapes: q [B, Hq, d]; L_K, L_V [B, Hkv, T, r]; B_K, B_V [Hkv, r, d];
scales [2, B, Hkv, T] fp32 (int8 latents only); seq_lens [B] int32.  All on
the same GPU, contiguous.  See include/lrattn.h for the operation, supported
shapes and error behaviour.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

__all__ = [
    "LrattnError", "Params", "lib", "library_path", "version", "status_string",
    "params_for", "plan", "workspace_size", "partition_kernel", "decode", "partition",
    "combine", "Decoder", "decode_static", "STATIC_SCRATCH_BYTES", "PRE_ABSORB_SPLITS",
    "dense_params_for", "dense_decode", "DenseDecoder",
    "rebuild_plan", "rebuild_workspace_size", "rebuild_decode", "RebuildDecoder",
    "AppendParams", "append_workspace_size", "append", "Appender",
    "shared_params_for", "shared_workspace_size", "shared_decode", "SharedDecoder",
    "modal_params_for", "modal_workspace_size", "modal_decode", "ModalDecoder",
    "AdaptiveParams", "adaptive_workspace_size", "adaptive_kernel", "adaptive_decode",
    "AdaptiveDecoder",
    "probe_read", "probe_copy", "probe_clock", "probe_sink_floats", "declared_symbols",
    "F32", "BF16", "F16", "I8",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
F32, BF16, F16, I8 = 0, 1, 2, 3

# LRATTN_PRE_ABSORB_SPLITS (lrattn.h): from this many partitions per head the
# decode step absorbs the queries in a kernel of their own
PRE_ABSORB_SPLITS = 64

STATUS = {0: "LRATTN_OK", -1: "LRATTN_ERR_NULL", -2: "LRATTN_ERR_SHAPE",
          -3: "LRATTN_ERR_DTYPE", -4: "LRATTN_ERR_UNSUPPORTED", -5: "LRATTN_ERR_ALIGN",
          -6: "LRATTN_ERR_WORKSPACE", -7: "LRATTN_ERR_SPLITS", -8: "LRATTN_ERR_HIP"}


class LrattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class Params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("latent_dtype", ctypes.c_int32),
                ("factor_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("num_splits", ctypes.c_int32)]


class AppendParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("model_dim", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("factor_dtype", ctypes.c_int32), ("latent_dtype", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("LRATTN_LIBRARY", os.path.join(_PKG, "liblrattn.so"))


_LIB = None
_VP = ctypes.c_void_p
_PP = ctypes.POINTER(Params)


def lib() -> ctypes.CDLL:
    """The loaded liblrattn.so (built by rank_kv_cache_head_amd.build)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(
                f"liblrattn.so not found at {path}: build it with "
                "`python -m rank_kv_cache_head_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(path)
        L.lrattn_version.restype = ctypes.c_int
        L.lrattn_status_string.restype = ctypes.c_char_p
        L.lrattn_status_string.argtypes = [ctypes.c_int]
        L.lrattn_plan.argtypes = [_PP, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        L.lrattn_workspace_size.argtypes = [_PP, ctypes.POINTER(ctypes.c_size_t)]
        L.lrattn_dense_decode.argtypes = [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          ctypes.c_size_t, _VP]
        L.lrattn_rebuild_decode.argtypes = [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                            ctypes.c_size_t, _VP]
        L.lrattn_adaptive_decode.argtypes = [_PP, ctypes.POINTER(AdaptiveParams), _VP, _VP, _VP,
                                             _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                             _VP]
        L.lrattn_adaptive_workspace_size.argtypes = [_PP, ctypes.POINTER(AdaptiveParams),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        L.lrattn_modal_decode.argtypes = [_PP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          _VP, _VP, ctypes.c_size_t, _VP]
        L.lrattn_modal_workspace_size.argtypes = [_PP, ctypes.c_int32,
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.lrattn_rebuild_plan.argtypes = [_PP, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32)]
        L.lrattn_rebuild_workspace_size.argtypes = [_PP, ctypes.POINTER(ctypes.c_size_t)]
        L.lrattn_append.argtypes = [ctypes.POINTER(AppendParams), _VP, _VP, _VP, _VP, _VP, _VP,
                                    _VP, _VP, ctypes.c_size_t, _VP]
        L.lrattn_append_workspace_size.argtypes = [ctypes.POINTER(AppendParams),
                                                   ctypes.POINTER(ctypes.c_size_t)]
        L.lrattn_shared_decode.argtypes = [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                           ctypes.c_size_t, _VP]
        L.lrattn_shared_workspace_size.argtypes = [_PP, ctypes.POINTER(ctypes.c_size_t)]
        L.lrattn_decode_static.argtypes = [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
        L.lrattn_partition_kernel.argtypes = [_PP]
        L.lrattn_partition_kernel.restype = ctypes.c_char_p
        L.lrattn_adaptive_kernel.argtypes = [_PP, ctypes.POINTER(AdaptiveParams)]
        L.lrattn_adaptive_kernel.restype = ctypes.c_char_p
        L.lrattn_decode.argtypes = [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                    ctypes.c_size_t, _VP]
        L.lrattn_partition.argtypes = [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                       ctypes.c_size_t, _VP]
        L.lrattn_combine.argtypes = [_PP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]
        L.lrattn_probe_sink_floats.restype = ctypes.c_size_t
        L.lrattn_probe_read.argtypes = [_VP, ctypes.c_size_t, _VP, _VP]
        L.lrattn_probe_copy.argtypes = [_VP, _VP, ctypes.c_size_t, _VP]
        L.lrattn_probe_clock.argtypes = [_VP, _VP]
        for fn in ("lrattn_plan", "lrattn_workspace_size", "lrattn_decode",
                   "lrattn_decode_static", "lrattn_partition",
                   "lrattn_combine", "lrattn_dense_decode", "lrattn_rebuild_decode",
                   "lrattn_rebuild_plan", "lrattn_rebuild_workspace_size",
                   "lrattn_modal_decode", "lrattn_modal_workspace_size",
                   "lrattn_adaptive_decode", "lrattn_adaptive_workspace_size",
                   "lrattn_append", "lrattn_append_workspace_size",
                   "lrattn_shared_decode", "lrattn_shared_workspace_size",
                   "lrattn_probe_read",
                   "lrattn_probe_copy", "lrattn_probe_clock"):
            getattr(L, fn).restype = ctypes.c_int
        _LIB = L
    return _LIB


def declared_symbols():
    """Every function name declared in include/*.h (for export checks)."""
    names = []
    inc = os.path.join(_ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(lrattn_\w+)\s*\(", text, flags=re.M)
    return names


def version() -> int:
    return lib().lrattn_version()


def status_string(status: int) -> str:
    try:
        return lib().lrattn_status_string(int(status)).decode()
    except ImportError:
        return STATUS.get(status, "unknown")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LrattnError(status, where)


# ------------------------------------------------------------ torch glue

def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.int8: I8}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def params_for(q, L_K, B_K, *, out_dtype=None, softmax_scale=None, num_splits: int = 0) -> Params:
    """Parameter block for tensors q [B,Hq,d], L_K [B,Hkv,T,r], B_K [Hkv,r,d]."""
    import torch
    if q.dim() != 3 or L_K.dim() != 4 or B_K.dim() != 3:
        raise ValueError("q [B,Hq,d], L [B,Hkv,T,r], B [Hkv,r,d] expected")
    B, Hq, d = q.shape
    B2, Hkv, T, r = L_K.shape
    if B2 != B or tuple(B_K.shape) != (Hkv, r, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} L {tuple(L_K.shape)} "
                         f"B {tuple(B_K.shape)}")
    od = F32 if out_dtype in (None, torch.float32) else (BF16 if out_dtype == torch.bfloat16 else -1)
    return Params(B, Hq, Hkv, d, r, T, _dtype_code(q), _dtype_code(L_K), _dtype_code(B_K), od,
                  float(softmax_scale) if softmax_scale else 0.0, int(num_splits))


def partition_kernel(p: Params) -> str:
    """lrattn_partition_kernel: the partition kernel's name for these parameters."""
    _check(lib().lrattn_plan(ctypes.byref(p), None, None), "lrattn_partition_kernel")
    return lib().lrattn_partition_kernel(ctypes.byref(p)).decode()


def plan(p: Params) -> Tuple[int, int]:
    """(partitions per (b, kv-head), tokens per partition) the library will use."""
    n = ctypes.c_int32()
    s = ctypes.c_int32()
    _check(lib().lrattn_plan(ctypes.byref(p), ctypes.byref(n), ctypes.byref(s)), "lrattn_plan")
    return n.value, s.value


def workspace_size(p: Params) -> int:
    b = ctypes.c_size_t()
    _check(lib().lrattn_workspace_size(ctypes.byref(p), ctypes.byref(b)), "lrattn_workspace_size")
    return b.value


def _workspace(p: Params, workspace, device, need=None):
    import torch
    need = workspace_size(p) if need is None else need
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _check_shapes(p: Params, L_V, B_V, scales, seq_lens):
    if tuple(L_V.shape) != (p.batch, p.num_kv_heads, p.max_seq_len, p.rank):
        raise ValueError("L_V shape differs from L_K")
    if B_V is not None and tuple(B_V.shape) != (p.num_kv_heads, p.rank, p.head_dim):
        raise ValueError("B_V shape differs from B_K")
    if scales is not None and tuple(scales.shape) != (2, p.batch, p.num_kv_heads, p.max_seq_len):
        raise ValueError("scales must be [2, B, Hkv, T]")
    if tuple(seq_lens.shape) != (p.batch,):
        raise ValueError("seq_lens must be [B]")
    import torch
    if seq_lens.dtype != torch.int32 or (scales is not None and scales.dtype != torch.float32):
        raise TypeError("seq_lens must be int32 and scales float32")


def decode(q, L_K, L_V, B_K, B_V, seq_lens, scales=None, *, out=None, workspace=None,
           softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
    """lrattn_decode on torch tensors; returns `out` [B, Hq, d] (fp32 unless out_dtype)."""
    import torch
    p = params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                   num_splits=num_splits)
    _check_shapes(p, L_V, B_V, scales, seq_lens)
    if out is None:
        out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                          dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                          device=q.device)
    ws, ws_bytes = _workspace(p, workspace, q.device)
    st = lib().lrattn_decode(ctypes.byref(p), _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K), _ptr(B_V),
                             _ptr(scales), _ptr(seq_lens), _ptr(out), _ptr(ws), ws_bytes,
                             _stream(stream))
    _check(st, "lrattn_decode")
    return out


STATIC_SCRATCH_BYTES = 16 << 20   # LRATTN_STATIC_SCRATCH_BYTES


def decode_static(q, L_K, L_V, B_K, B_V, seq_lens, scales=None, *, out, softmax_scale=None,
                  num_splits: int = 0, stream=None):
    """lrattn_decode_static: the decode with its records in the library's
    static per-device buffer (no workspace; the call allocates nothing).
    `out` [B, Hq, d] (fp32 or bf16) is required and returned."""
    p = params_for(q, L_K, B_K, out_dtype=out.dtype, softmax_scale=softmax_scale,
                   num_splits=num_splits)
    _check_shapes(p, L_V, B_V, scales, seq_lens)
    if tuple(out.shape) != (p.batch, p.num_q_heads, p.head_dim):
        raise ValueError("out must be [B, Hq, d]")
    st = lib().lrattn_decode_static(ctypes.byref(p), _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K),
                                    _ptr(B_V), _ptr(scales), _ptr(seq_lens), _ptr(out),
                                    _stream(stream))
    _check(st, "lrattn_decode_static")
    return out


class AdaptiveParams(ctypes.Structure):
    """lrattn_adaptive: rank of the tokens below the importance threshold,
    the threshold, and the moving average's decay."""
    _fields_ = [("low_rank", ctypes.c_int32), ("threshold", ctypes.c_float),
                ("decay", ctypes.c_float)]


def adaptive_workspace_size(p: Params, ad: AdaptiveParams) -> int:
    b = ctypes.c_size_t()
    _check(lib().lrattn_adaptive_workspace_size(ctypes.byref(p), ctypes.byref(ad),
                                                ctypes.byref(b)),
           "lrattn_adaptive_workspace_size")
    return b.value


def adaptive_kernel(p: Params, ad: AdaptiveParams) -> str:
    """lrattn_adaptive_kernel: the adaptive-rank partition kernel's name."""
    adaptive_workspace_size(p, ad)  # raises on a rejected configuration
    return lib().lrattn_adaptive_kernel(ctypes.byref(p), ctypes.byref(ad)).decode()


def _check_importance(p: Params, importance):
    import torch
    if (tuple(importance.shape) != (p.batch, p.num_kv_heads, p.max_seq_len) or
            importance.dtype != torch.float32 or not importance.is_contiguous()):
        raise ValueError("importance must be contiguous float32 [B, Hkv, T]")


def adaptive_decode(q, L_K, L_V, B_K, B_V, seq_lens, importance, *, low_rank: int,
                    threshold: float, decay: float, scales=None, out=None, workspace=None,
                    softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
    """lrattn_adaptive_decode: tokens whose importance is below `threshold`
    are rebuilt at `low_rank`; `importance` [B, Hkv, T] is updated in place
    with the step's head-averaged attention (moving average, `decay`)."""
    import torch
    p = params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                   num_splits=num_splits)
    _check_shapes(p, L_V, B_V, scales, seq_lens)
    _check_importance(p, importance)
    ad = AdaptiveParams(int(low_rank), float(threshold), float(decay))
    if out is None:
        out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                          dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                          device=q.device)
    ws, ws_bytes = _workspace(p, workspace, q.device, adaptive_workspace_size(p, ad))
    st = lib().lrattn_adaptive_decode(ctypes.byref(p), ctypes.byref(ad), _ptr(q), _ptr(L_K),
                                      _ptr(L_V), _ptr(B_K), _ptr(B_V), _ptr(scales),
                                      _ptr(seq_lens), _ptr(importance), _ptr(out), _ptr(ws),
                                      ws_bytes, _stream(stream))
    _check(st, "lrattn_adaptive_decode")
    return out


class AdaptiveDecoder:
    """lrattn_adaptive_decode on fixed buffers, marshalled once (see Decoder)."""

    def __init__(self, q, L_K, L_V, B_K, B_V, seq_lens, importance, *, low_rank: int,
                 threshold: float, decay: float, scales=None, out=None, workspace=None,
                 softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
        import torch
        p = params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                       num_splits=num_splits)
        _check_shapes(p, L_V, B_V, scales, seq_lens)
        _check_importance(p, importance)
        ad = AdaptiveParams(int(low_rank), float(threshold), float(decay))
        if out is None:
            out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                              dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                              device=q.device)
        ws, ws_bytes = _workspace(p, workspace, q.device, adaptive_workspace_size(p, ad))
        self.params, self.adaptive, self.out, self.workspace = p, ad, out, ws
        self._keep = (q, L_K, L_V, B_K, B_V, seq_lens, importance, scales)
        self._fn = lib().lrattn_adaptive_decode
        self._args = (ctypes.byref(p), ctypes.byref(ad), _ptr(q), _ptr(L_K), _ptr(L_V),
                      _ptr(B_K), _ptr(B_V), _ptr(scales), _ptr(seq_lens), _ptr(importance),
                      _ptr(out), _ptr(ws), ws_bytes, _stream(stream))

    def __call__(self):
        _check(self._fn(*self._args), "lrattn_adaptive_decode")
        return self.out


def modal_params_for(q, L_K, B_K, *, out_dtype=None, softmax_scale=None,
                     num_splits: int = 0) -> Params:
    """Parameter block for two factor sets: B_K [2, Hkv, r, d] (image, text)."""
    if B_K.dim() != 4 or B_K.shape[0] != 2:
        raise ValueError("B_K [2, Hkv, r, d] expected (image set, text set)")
    return params_for(q, L_K, B_K[0], out_dtype=out_dtype, softmax_scale=softmax_scale,
                      num_splits=num_splits)


def modal_workspace_size(p: Params, image_tokens: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().lrattn_modal_workspace_size(ctypes.byref(p), int(image_tokens), ctypes.byref(b)),
           "lrattn_modal_workspace_size")
    return b.value


def _check_modal(p: Params, B_K, B_V):
    if tuple(B_V.shape) != tuple(B_K.shape) or not (B_K.is_contiguous() and B_V.is_contiguous()):
        raise ValueError("B_K, B_V must both be contiguous [2, Hkv, r, d]")


def modal_decode(q, L_K, L_V, B_K, B_V, seq_lens, image_tokens: int, scales=None, *, out=None,
                 workspace=None, softmax_scale=None, num_splits: int = 0, out_dtype=None,
                 stream=None):
    """lrattn_modal_decode: factor set 0 for the first image_tokens tokens of
    every sequence, set 1 for the rest; B_K, B_V [2, Hkv, r, d]."""
    import torch
    p = modal_params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                         num_splits=num_splits)
    _check_shapes(p, L_V, B_V[0], scales, seq_lens)
    _check_modal(p, B_K, B_V)
    if out is None:
        out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                          dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                          device=q.device)
    ws, ws_bytes = _workspace(p, workspace, q.device, modal_workspace_size(p, image_tokens))
    st = lib().lrattn_modal_decode(ctypes.byref(p), int(image_tokens), _ptr(q), _ptr(L_K),
                                   _ptr(L_V), _ptr(B_K), _ptr(B_V), _ptr(scales),
                                   _ptr(seq_lens), _ptr(out), _ptr(ws), ws_bytes,
                                   _stream(stream))
    _check(st, "lrattn_modal_decode")
    return out


class ModalDecoder:
    """lrattn_modal_decode on fixed buffers, marshalled once (see Decoder)."""

    def __init__(self, q, L_K, L_V, B_K, B_V, seq_lens, image_tokens: int, scales=None, *,
                 out=None, workspace=None, softmax_scale=None, num_splits: int = 0,
                 out_dtype=None, stream=None):
        import torch
        p = modal_params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                             num_splits=num_splits)
        _check_shapes(p, L_V, B_V[0], scales, seq_lens)
        _check_modal(p, B_K, B_V)
        if out is None:
            out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                              dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                              device=q.device)
        ws, ws_bytes = _workspace(p, workspace, q.device, modal_workspace_size(p, image_tokens))
        self.params, self.out, self.workspace = p, out, ws
        self._keep = (q, L_K, L_V, B_K, B_V, seq_lens, scales)
        self._fn = lib().lrattn_modal_decode
        self._args = (ctypes.byref(p), int(image_tokens), _ptr(q), _ptr(L_K), _ptr(L_V),
                      _ptr(B_K), _ptr(B_V), _ptr(scales), _ptr(seq_lens), _ptr(out), _ptr(ws),
                      ws_bytes, _stream(stream))

    def __call__(self):
        _check(self._fn(*self._args), "lrattn_modal_decode")
        return self.out


def dense_params_for(q, K, *, out_dtype=None, softmax_scale=None, num_splits: int = 0) -> Params:
    """Parameter block for the dense baseline: q [B,Hq,d], K [B,Hkv,T,d] (rank = d)."""
    import torch
    if q.dim() != 3 or K.dim() != 4 or K.shape[0] != q.shape[0] or K.shape[3] != q.shape[2]:
        raise ValueError("q [B,Hq,d], K [B,Hkv,T,d] expected")
    B, Hq, d = q.shape
    _, Hkv, T, _ = K.shape
    od = F32 if out_dtype in (None, torch.float32) else (BF16 if out_dtype == torch.bfloat16 else -1)
    qd = _dtype_code(q)
    return Params(B, Hq, Hkv, d, d, T, qd, _dtype_code(K), qd, od,
                  float(softmax_scale) if softmax_scale else 0.0, int(num_splits))


def dense_decode(q, K, V, seq_lens, scales=None, *, out=None, workspace=None,
                 softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
    """lrattn_dense_decode: the same decode over an uncompressed cache K, V [B,Hkv,T,d]."""
    import torch
    p = dense_params_for(q, K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                         num_splits=num_splits)
    _check_shapes(p, V, None, scales, seq_lens)
    if out is None:
        out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                          dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                          device=q.device)
    ws, ws_bytes = _workspace(p, workspace, q.device)
    st = lib().lrattn_dense_decode(ctypes.byref(p), _ptr(q), _ptr(K), _ptr(V), _ptr(scales),
                                   _ptr(seq_lens), _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lrattn_dense_decode")
    return out


def _check_rope(p: Params, rope):
    import torch
    if rope is not None and (tuple(rope.shape) != (p.max_seq_len, p.head_dim) or
                             rope.dtype != torch.float32):
        raise ValueError("rope must be float32 [T, d]")


def rebuild_plan(p: Params) -> Tuple[int, int]:
    """(partitions, tokens per partition) of lrattn_rebuild_decode."""
    n = ctypes.c_int32()
    s = ctypes.c_int32()
    _check(lib().lrattn_rebuild_plan(ctypes.byref(p), ctypes.byref(n), ctypes.byref(s)),
           "lrattn_rebuild_plan")
    return n.value, s.value


def rebuild_workspace_size(p: Params) -> int:
    b = ctypes.c_size_t()
    _check(lib().lrattn_rebuild_workspace_size(ctypes.byref(p), ctypes.byref(b)),
           "lrattn_rebuild_workspace_size")
    return b.value


def rebuild_decode(q, L_K, L_V, B_K, B_V, seq_lens, rope=None, *, out=None, workspace=None,
                   softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
    """lrattn_rebuild_decode: keys rebuilt on chip, rotated by position when
    `rope` ([T, d] float32: cosines then sines per position) is given."""
    import torch
    p = params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                   num_splits=num_splits)
    _check_shapes(p, L_V, B_V, None, seq_lens)
    _check_rope(p, rope)
    if out is None:
        out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                          dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                          device=q.device)
    ws, ws_bytes = _workspace(p, workspace, q.device, rebuild_workspace_size(p))
    st = lib().lrattn_rebuild_decode(ctypes.byref(p), _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K),
                                     _ptr(B_V), _ptr(rope), _ptr(seq_lens), _ptr(out), _ptr(ws),
                                     ws_bytes, _stream(stream))
    _check(st, "lrattn_rebuild_decode")
    return out


def shared_params_for(q, L_K, B_K, *, out_dtype=None, softmax_scale=None,
                      num_splits: int = 0) -> Params:
    """Parameter block for shared latent streams: q [B,Hq,d], L [B,S,T,r],
    B_K [Hq,r,d] (one factor block per query head)."""
    import torch
    if q.dim() != 3 or L_K.dim() != 4 or B_K.dim() != 3:
        raise ValueError("q [B,Hq,d], L [B,S,T,r], B [Hq,r,d] expected")
    B, Hq, d = q.shape
    B2, S, T, r = L_K.shape
    if B2 != B or tuple(B_K.shape) != (Hq, r, d):
        raise ValueError("shape mismatch")
    od = F32 if out_dtype in (None, torch.float32) else (BF16 if out_dtype == torch.bfloat16 else -1)
    return Params(B, Hq, S, d, r, T, _dtype_code(q), _dtype_code(L_K), _dtype_code(B_K), od,
                  float(softmax_scale) if softmax_scale else 0.0, int(num_splits))


def shared_workspace_size(p: Params) -> int:
    b = ctypes.c_size_t()
    _check(lib().lrattn_shared_workspace_size(ctypes.byref(p), ctypes.byref(b)),
           "lrattn_shared_workspace_size")
    return b.value


def shared_decode(q, L_K, L_V, B_K, B_V, seq_lens, scales=None, *, out=None, workspace=None,
                  softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
    """lrattn_shared_decode: shared latent streams, per-query-head factors."""
    import torch
    p = shared_params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                          num_splits=num_splits)
    if tuple(L_V.shape) != tuple(L_K.shape) or tuple(B_V.shape) != tuple(B_K.shape):
        raise ValueError("L_V / B_V shapes differ from L_K / B_K")
    if tuple(seq_lens.shape) != (p.batch,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32 [B]")
    if out is None:
        out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                          dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                          device=q.device)
    need = shared_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().lrattn_shared_decode(ctypes.byref(p), _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K),
                                    _ptr(B_V), _ptr(scales), _ptr(seq_lens), _ptr(out),
                                    _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "lrattn_shared_decode")
    return out


def append_workspace_size(p: "AppendParams") -> int:
    b = ctypes.c_size_t()
    _check(lib().lrattn_append_workspace_size(ctypes.byref(p), ctypes.byref(b)),
           "lrattn_append_workspace_size")
    return b.value


def append(x, A_K, A_V, positions, L_K, L_V, scales=None, *, workspace=None, stream=None):
    """lrattn_append: write each sequence's new latent rows (x . A_h^T) into
    L_K / L_V (and int8 scales) at positions[b]; returns (L_K, L_V)."""
    import torch
    if x.dim() != 2 or A_K.dim() != 3 or L_K.dim() != 4:
        raise ValueError("x [B,D], A [Hkv,r,D], L [B,Hkv,T,r] expected")
    B, D = x.shape
    Hkv, r, D2 = A_K.shape
    if (D2 != D or tuple(A_V.shape) != tuple(A_K.shape) or L_K.shape[0] != B or
            L_K.shape[1] != Hkv or L_K.shape[3] != r or L_V.shape != L_K.shape):
        raise ValueError("shape mismatch")
    if tuple(positions.shape) != (B,) or positions.dtype != torch.int32:
        raise ValueError("positions must be int32 [B]")
    if scales is not None and (tuple(scales.shape) != (2, B, Hkv, L_K.shape[2]) or
                               scales.dtype != torch.float32):
        raise ValueError("scales must be float32 [2, B, Hkv, T]")
    p = AppendParams(B, Hkv, D, r, L_K.shape[2], _dtype_code(x), _dtype_code(A_K),
                     _dtype_code(L_K))
    need = append_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().lrattn_append(ctypes.byref(p), _ptr(x), _ptr(A_K), _ptr(A_V), _ptr(positions),
                             _ptr(L_K), _ptr(L_V), _ptr(scales), _ptr(workspace), ws_bytes,
                             _stream(stream))
    _check(st, "lrattn_append")
    return L_K, L_V


class Appender:
    """lrattn_append on fixed buffers: arguments validated and marshalled
    once, each call passes the same pointers and stream to the library.  The
    tensors must stay alive and keep their storage while the object is used."""

    def __init__(self, x, A_K, A_V, positions, L_K, L_V, scales=None, *, workspace=None,
                 stream=None):
        import torch
        append(x, A_K, A_V, positions, L_K, L_V, scales, workspace=workspace, stream=stream)
        p = AppendParams(x.shape[0], A_K.shape[0], x.shape[1], A_K.shape[1], L_K.shape[2],
                         _dtype_code(x), _dtype_code(A_K), _dtype_code(L_K))
        if workspace is None:
            workspace = torch.empty(append_workspace_size(p), dtype=torch.uint8, device=x.device)
        self.params, self.workspace = p, workspace
        self._keep = (x, A_K, A_V, positions, L_K, L_V, scales)
        self._args = (ctypes.byref(p), _ptr(x), _ptr(A_K), _ptr(A_V), _ptr(positions),
                      _ptr(L_K), _ptr(L_V), _ptr(scales), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _stream(stream))

    def __call__(self):
        _check(lib().lrattn_append(*self._args), "lrattn_append")


def partition(q, L_K, L_V, B_K, seq_lens, scales=None, *, workspace=None, softmax_scale=None,
              num_splits: int = 0, stream=None):
    """lrattn_partition alone; returns the workspace tensor holding the partials."""
    p = params_for(q, L_K, B_K, softmax_scale=softmax_scale, num_splits=num_splits)
    _check_shapes(p, L_V, None, scales, seq_lens)
    ws, ws_bytes = _workspace(p, workspace, q.device)
    st = lib().lrattn_partition(ctypes.byref(p), _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K),
                                _ptr(scales), _ptr(seq_lens), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lrattn_partition")
    return ws


def combine(p: Params, B_V, seq_lens, workspace, *, out=None, stream=None):
    """lrattn_combine alone, on the workspace a matching partition() call filled."""
    import torch
    if out is None:
        out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                          dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                          device=B_V.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().lrattn_combine(ctypes.byref(p), _ptr(B_V), _ptr(seq_lens), _ptr(out),
                              _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "lrattn_combine")
    return out


def probe_sink_floats() -> int:
    return lib().lrattn_probe_sink_floats()


def probe_read(src, sink, stream=None) -> None:
    """Stream-read every byte of `src` (HBM bandwidth probe)."""
    nbytes = src.numel() * src.element_size()
    _check(lib().lrattn_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "lrattn_probe_read")


def probe_clock(out, stream=None) -> None:
    """lrattn_probe_clock: enqueue a shader-clock sample into `out` (a
    contiguous int64 tensor of 2 values): shader cycles and 100 MHz ticks
    over ~5 us; GHz = out[0] / out[1] / 10."""
    import torch
    if out.dtype != torch.int64 or out.numel() < 2 or not out.is_contiguous():
        raise ValueError("out must be a contiguous int64 tensor of at least 2 values")
    _check(lib().lrattn_probe_clock(_ptr(out), _stream(stream)), "lrattn_probe_clock")


def probe_copy(dst, src, stream=None) -> None:
    """Copy `src` into `dst` (same byte size) with 16-byte loads and stores."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _check(lib().lrattn_probe_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)),
           "lrattn_probe_copy")


class Decoder:
    """lrattn_decode / lrattn_partition / lrattn_combine on fixed buffers.

    Arguments are validated and marshalled once; each call then passes the
    same pointers and stream straight to the library (for loops that reuse
    buffers, e.g. a decode loop or a benchmark).  The tensors must stay alive
    and keep their storage while the object is used.
    """

    def __init__(self, q, L_K, L_V, B_K, B_V, seq_lens, scales=None, *, out=None,
                 workspace=None, softmax_scale=None, num_splits: int = 0, out_dtype=None,
                 stream=None):
        import torch
        p = params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                       num_splits=num_splits)
        _check_shapes(p, L_V, B_V, scales, seq_lens)
        if out is None:
            out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                              dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                              device=q.device)
        ws, ws_bytes = _workspace(p, workspace, q.device)
        self.params, self.out, self.workspace = p, out, ws
        self.plan = plan(p)
        self._keep = (q, L_K, L_V, B_K, B_V, seq_lens, scales)
        st = _stream(stream)
        pp = ctypes.byref(p)
        L = lib()
        self._decode = (L.lrattn_decode, (pp, _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K), _ptr(B_V),
                                          _ptr(scales), _ptr(seq_lens), _ptr(out), _ptr(ws),
                                          ws_bytes, st))
        self._partition = (L.lrattn_partition, (pp, _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K),
                                                _ptr(scales), _ptr(seq_lens), _ptr(ws), ws_bytes,
                                                st))
        self._combine = (L.lrattn_combine, (pp, _ptr(B_V), _ptr(seq_lens), _ptr(out), _ptr(ws),
                                            ws_bytes, st))

    def __call__(self):
        fn, args = self._decode
        _check(fn(*args), "lrattn_decode")
        return self.out

    def partition(self):
        fn, args = self._partition
        _check(fn(*args), "lrattn_partition")

    def combine(self):
        fn, args = self._combine
        _check(fn(*args), "lrattn_combine")
        return self.out


class SharedDecoder:
    """lrattn_shared_decode on fixed buffers, marshalled once (see Decoder)."""

    def __init__(self, q, L_K, L_V, B_K, B_V, seq_lens, scales=None, *, out=None,
                 workspace=None, softmax_scale=None, num_splits: int = 0, out_dtype=None,
                 stream=None):
        import torch
        p = shared_params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                              num_splits=num_splits)
        if tuple(L_V.shape) != tuple(L_K.shape) or tuple(B_V.shape) != tuple(B_K.shape):
            raise ValueError("L_V / B_V shapes differ from L_K / B_K")
        if tuple(seq_lens.shape) != (p.batch,) or seq_lens.dtype != torch.int32:
            raise ValueError("seq_lens must be int32 [B]")
        if out is None:
            out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                              dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                              device=q.device)
        ws, ws_bytes = _workspace(p, workspace, q.device, shared_workspace_size(p))
        self.params, self.out, self.workspace = p, out, ws
        self._keep = (q, L_K, L_V, B_K, B_V, seq_lens, scales)
        self._fn = lib().lrattn_shared_decode
        self._args = (ctypes.byref(p), _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K), _ptr(B_V),
                      _ptr(scales), _ptr(seq_lens), _ptr(out), _ptr(ws), ws_bytes,
                      _stream(stream))

    def __call__(self):
        _check(self._fn(*self._args), "lrattn_shared_decode")
        return self.out


class DenseDecoder:
    """lrattn_dense_decode on fixed buffers, marshalled once (see Decoder)."""

    def __init__(self, q, K, V, seq_lens, scales=None, *, out=None, workspace=None,
                 softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
        import torch
        p = dense_params_for(q, K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                             num_splits=num_splits)
        _check_shapes(p, V, None, scales, seq_lens)
        if out is None:
            out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                              dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                              device=q.device)
        ws, ws_bytes = _workspace(p, workspace, q.device)
        self.params, self.out, self.workspace = p, out, ws
        self.plan = plan(p)
        self._keep = (q, K, V, seq_lens, scales)
        self._fn = lib().lrattn_dense_decode
        self._args = (ctypes.byref(p), _ptr(q), _ptr(K), _ptr(V), _ptr(scales), _ptr(seq_lens),
                      _ptr(out), _ptr(ws), ws_bytes, _stream(stream))

    def __call__(self):
        _check(self._fn(*self._args), "lrattn_dense_decode")
        return self.out


class RebuildDecoder:
    """lrattn_rebuild_decode on fixed buffers, marshalled once (see Decoder)."""

    def __init__(self, q, L_K, L_V, B_K, B_V, seq_lens, rope=None, *, out=None, workspace=None,
                 softmax_scale=None, num_splits: int = 0, out_dtype=None, stream=None):
        import torch
        p = params_for(q, L_K, B_K, out_dtype=out_dtype, softmax_scale=softmax_scale,
                       num_splits=num_splits)
        _check_shapes(p, L_V, B_V, None, seq_lens)
        _check_rope(p, rope)
        if out is None:
            out = torch.empty((p.batch, p.num_q_heads, p.head_dim),
                              dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                              device=q.device)
        ws, ws_bytes = _workspace(p, workspace, q.device, rebuild_workspace_size(p))
        self.params, self.out, self.workspace = p, out, ws
        self.plan = rebuild_plan(p)
        self._keep = (q, L_K, L_V, B_K, B_V, seq_lens, rope)
        self._fn = lib().lrattn_rebuild_decode
        self._args = (ctypes.byref(p), _ptr(q), _ptr(L_K), _ptr(L_V), _ptr(B_K), _ptr(B_V),
                      _ptr(rope), _ptr(seq_lens), _ptr(out), _ptr(ws), ws_bytes, _stream(stream))

    def __call__(self):
        _check(self._fn(*self._args), "lrattn_rebuild_decode")
        return self.out

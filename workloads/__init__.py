"""Seeded synthetic inputs for low-rank-KV decode attention.

This module only draws random numbers and rounds them to their storage type.
It holds none of the attention arithmetic: both the fp64 oracle and the HIP
path consume what it produces, and neither is imported here.

Storage conventions (what every consumer receives):

  dtype tag  numpy storage         meaning
  "f32"      float32               IEEE binary32
  "bf16"     uint16 (raw bits)     bfloat16, rounded to nearest-even from fp32
  "f16"      float16               IEEE binary16
  "i8"       int8                  signed integer latents (dequantized by a scale)

Tensor shapes (row-major, contiguous):

  q        [B, Hq, d]
  L_K, L_V [B, Hkv, T, r]      per-token, per-kv-head latent rows
  B_K, B_V [Hkv, r, d]         per-kv-head factors
  scales   [2, B, Hkv, T]      fp32, index 0 = K, 1 = V; only for "i8" latents
  seq_lens [B] int32           valid tokens of each sequence; rows t >= seq_len
                               are padding (zero, or NaN when asked for)

The five named workloads follow the shapes of the pages' workloads: a per-head
rank-r latent per token and an r x d factor per head (WSVD page, section 2.A),
a 576-token image block ahead of the text tokens (the LLaVA-1.5 visual sequence
length on the SVD-Prune page, lay summary), and an int8 latent with a per-token
scale (WSVD page, section 2.C, W8A8).

Random streams: numpy PCG64, one SeedSequence child per tensor, spawned in the
fixed order q, L_K, L_V, B_K, B_V, scales, seq_lens.  The latent and scale
tensors spawn one grandchild per (b, kv-head) block, so any block can be drawn
alone and blocks can be drawn in parallel threads with identical results.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "CONFIG_ORDER", "SPECS", "make", "bf16_bits_from_f32", "rope_table",
    "make_append",
    "storage_dtype", "fingerprint",
]

# name -> shape/dtype/distribution recipe.  Variances follow N(mean, variance).
SPECS: Dict[str, dict] = {
    # Tiny: fp32 everywhere; entries N(0,1), factors scaled by 1/sqrt(r).
    "tiny": dict(B=1, Hq=4, Hkv=4, d=64, r=16, T=256,
                 q_dtype="f32", latent_dtype="f32", factor_dtype="f32",
                 q_std=1.0, latent_std=1.0, factor_std=1.0 / math.sqrt(16),
                 lengths="full", seed=1),
    # 7B-LLM-like decode: bf16; latents N(0,1), factors N(0,1/r), q N(0,1).
    "llm7b": dict(B=8, Hq=32, Hkv=32, d=128, r=32, T=4096,
                  q_dtype="bf16", latent_dtype="bf16", factor_dtype="bf16",
                  q_std=1.0, latent_std=1.0, factor_std=1.0 / math.sqrt(32),
                  lengths="full", seed=2),
    # GQA VLM long prompt: 32 q heads on 8 kv heads; 576-token image block with
    # variance 4 (std 2) ahead of text latents N(0,1); factors N(0,1/r).
    "gqa_vlm": dict(B=16, Hq=32, Hkv=8, d=128, r=64, T=16384,
                    q_dtype="bf16", latent_dtype="bf16", factor_dtype="bf16",
                    q_std=1.0, latent_std=1.0, factor_std=1.0 / math.sqrt(64),
                    image_tokens=576, image_std=2.0,
                    lengths="full", seed=3),
    # Quantized latents: int8 uniform on [-127, 127], fp32 scale per
    # (batch, kv-head, token) drawn U(0.005, 0.02), separate for K and V.
    "int8": dict(B=32, Hq=32, Hkv=32, d=128, r=32, T=8192,
                 q_dtype="bf16", latent_dtype="i8", factor_dtype="bf16",
                 q_std=1.0, factor_std=1.0 / math.sqrt(32),
                 scale_lo=0.005, scale_hi=0.02,
                 lengths="full", seed=4),
    # Ragged long context: lengths uniform on [1024, 131072], padded to 131072.
    "ragged": dict(B=4, Hq=40, Hkv=40, d=128, r=48, T=131072,
                   q_dtype="bf16", latent_dtype="bf16", factor_dtype="bf16",
                   q_std=1.0, latent_std=1.0, factor_std=1.0 / math.sqrt(48),
                   lengths="uniform", len_lo=1024, len_hi=131072, seed=5),
}
CONFIG_ORDER = ["tiny", "llm7b", "gqa_vlm", "int8", "ragged"]

# Partitions per (sequence, kv-head) a workload names for its launch: the
# ragged long-context workload asks for split-K across at least 256
# partitions per head (over T = 131072, 512 tokens each).  Others: 0, the
# library's default plan.
SPLITS = {"ragged": 256}

_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16, "i8": np.int8}
_ESIZE = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1}


def storage_dtype(tag: str):
    return _STORAGE[tag]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as raw uint16 bits.

    NaN inputs stay NaN (a quiet NaN pattern); finite values that round past
    the largest bfloat16 become infinity, as nearest-even rounding does.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def _to_storage(x32: np.ndarray, tag: str) -> np.ndarray:
    if tag == "f32":
        return x32.astype(np.float32, copy=False)
    if tag == "bf16":
        return bf16_bits_from_f32(x32)
    if tag == "f16":
        return x32.astype(np.float16)
    raise ValueError(f"no float storage for {tag!r}")


def _nan_storage(tag: str):
    return {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0),
            "f16": np.float16(np.nan)}[tag]


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rank: int
    max_seq_len: int
    q_dtype: str
    latent_dtype: str
    factor_dtype: str
    q: np.ndarray
    L_K: np.ndarray
    L_V: np.ndarray
    B_K: np.ndarray
    B_V: np.ndarray
    scales: Optional[np.ndarray]
    seq_lens: np.ndarray
    seed: int
    softmax_scale: Optional[float] = None

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def latent_bytes_per_row(self) -> int:
        return self.rank * _ESIZE[self.latent_dtype]

    def algorithmic_bytes(self) -> dict:
        """Bytes a decode step must move at minimum, by tensor.

        Valid latent rows (K and V), their int8 scales, q, both factors and an
        fp32 output.  Padding rows past seq_len are never needed.
        """
        valid = int(np.clip(self.seq_lens.astype(np.int64), 0, self.max_seq_len).sum())
        rows = valid * self.num_kv_heads
        lat = 2 * rows * self.latent_bytes_per_row
        sc = 2 * rows * 4 if self.latent_dtype == "i8" else 0
        qb = self.q.nbytes
        fb = self.B_K.nbytes + self.B_V.nbytes
        ob = self.batch * self.num_q_heads * self.head_dim * 4
        return dict(latents=lat, scales=sc, q=qb, factors=fb, out=ob,
                    total=lat + sc + qb + fb + ob, valid_tokens=valid)


def _normal_block(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seq))
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make(name: str, seed: Optional[int] = None, *, pad: str = "zero",
         threads: Optional[int] = None, **overrides) -> Workload:
    """Draw one named workload.

    name      one of CONFIG_ORDER
    seed      defaults to the workload's own seed (tiny 1 ... ragged 5)
    pad       "zero" or "nan": value stored in latent rows (and int8 scales)
              past each sequence's length.  Those rows are padding that a
              correct decode never reads.
    overrides shape keys B, Hq, Hkv, d, r, T; "seq_lens" (explicit list);
              any distribution key of SPECS.  Structure is kept: the image
              block stays at the front, lengths keep their distribution
              (clipped to T).
    """
    if name not in SPECS:
        raise KeyError(f"unknown workload {name!r}; choose from {CONFIG_ORDER}")
    spec = dict(SPECS[name])
    explicit_lens = overrides.pop("seq_lens", None)
    for k, v in overrides.items():
        if k not in spec:
            raise KeyError(f"unknown override {k!r} for {name}")
        spec[k] = v
    if seed is None:
        seed = spec["seed"]
    B, Hq, Hkv, d, r, T = (int(spec[k]) for k in ("B", "Hq", "Hkv", "d", "r", "T"))
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    qt, lt, ft = spec["q_dtype"], spec["latent_dtype"], spec["factor_dtype"]
    if pad not in ("zero", "nan"):
        raise ValueError("pad must be 'zero' or 'nan'")

    ss = np.random.SeedSequence(seed)
    s_q, s_lk, s_lv, s_bk, s_bv, s_sc, s_len = ss.spawn(7)

    # sequence lengths first: the latent draw depends on them (padding)
    if explicit_lens is not None:
        seq_lens = np.asarray(explicit_lens, dtype=np.int32).reshape(B)
    elif spec["lengths"] == "full":
        seq_lens = np.full(B, T, dtype=np.int32)
    else:
        g = np.random.Generator(np.random.PCG64(s_len))
        lo = min(int(spec["len_lo"]), T)
        hi = min(int(spec["len_hi"]), T)
        seq_lens = g.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)

    q = _to_storage(_normal_block(s_q, (B, Hq, d), spec["q_std"]), qt)
    B_K = _to_storage(_normal_block(s_bk, (Hkv, r, d), spec["factor_std"]), ft)
    B_V = _to_storage(_normal_block(s_bv, (Hkv, r, d), spec["factor_std"]), ft)

    L_K = np.empty((B, Hkv, T, r), dtype=_STORAGE[lt])
    L_V = np.empty((B, Hkv, T, r), dtype=_STORAGE[lt])
    scales = np.empty((2, B, Hkv, T), dtype=np.float32) if lt == "i8" else None
    kid = s_lk.spawn(B * Hkv)
    vid = s_lv.spawn(B * Hkv)
    sid = s_sc.spawn(B * Hkv)
    n_img = min(int(spec.get("image_tokens", 0)), T)

    def fill(idx: int) -> None:
        b, g = divmod(idx, Hkv)
        n = int(np.clip(seq_lens[b], 0, T))
        for dst, child in ((L_K, kid[idx]), (L_V, vid[idx])):
            if lt == "i8":
                gen = np.random.Generator(np.random.PCG64(child))
                dst[b, g, :n] = gen.integers(-127, 128, size=(n, r), dtype=np.int8)
                dst[b, g, n:] = 0
                continue
            x = _normal_block(child, (n, r), spec["latent_std"])
            if n_img:
                m = min(n_img, n)
                x[:m] *= np.float32(spec["image_std"] / spec["latent_std"])
            dst[b, g, :n] = _to_storage(x, lt)
            dst[b, g, n:] = _nan_storage(lt) if pad == "nan" else 0
        if scales is not None:
            gen = np.random.Generator(np.random.PCG64(sid[idx]))
            s = gen.uniform(spec["scale_lo"], spec["scale_hi"], size=(2, n))
            scales[:, b, g, :n] = s.astype(np.float32)
            scales[:, b, g, n:] = np.nan if pad == "nan" else 0.0

    nthr = threads or _threads()
    if nthr > 1 and B * Hkv > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, range(B * Hkv)))
    else:
        for i in range(B * Hkv):
            fill(i)

    return Workload(name=name, batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=d, rank=r, max_seq_len=T, q_dtype=qt,
                    latent_dtype=lt, factor_dtype=ft, q=q, L_K=L_K, L_V=L_V,
                    B_K=B_K, B_V=B_V, scales=scales, seq_lens=seq_lens,
                    seed=int(seed))


def fingerprint(w: Workload) -> Dict[str, str]:
    """SHA-256 of every tensor's bytes (short hex), for determinism checks."""
    out = {}
    for k in ("q", "L_K", "L_V", "B_K", "B_V", "scales", "seq_lens"):
        a = getattr(w, k)
        if a is None:
            continue
        out[k] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
    return out


def rope_table(T: int, d: int, base: float = 10000.0, offset: int = 0) -> np.ndarray:
    """Rotary cosine/sine table, float32 [T, d]: row p holds cos((p + offset)
    w_j) for j < d/2, then sin((p + offset) w_j), with w_j = base^(-2j/d).
    Angles and trigonometry in float64, rounded once to float32.  (An input of
    the rotated-key decode, supplied by the caller like any cache tensor.)"""
    j = np.arange(d // 2, dtype=np.float64)
    w = base ** (-2.0 * j / d)
    ang = (np.arange(T, dtype=np.float64)[:, None] + offset) * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_append(seed: int, B: int, Hkv: int, D: int, r: int, x_dtype: str = "bf16",
                x_std: float = 1.0) -> Dict[str, np.ndarray]:
    """Inputs of the append step: hidden states x [B, D] ~ N(0, x_std^2) and
    per-head projections A_K, A_V [Hkv, r, D] ~ N(0, 1/D) (so latents are
    about N(0, x_std^2)), drawn in float32 and rounded to x_dtype storage
    (bf16 as raw uint16 bits).  Child streams of SeedSequence(seed) in the
    order x, A_K, A_V."""
    sx, sk, sv = np.random.SeedSequence(seed).spawn(3)
    x = _normal_block(sx, (B, D), x_std)
    AK = _normal_block(sk, (Hkv, r, D), 1.0 / np.sqrt(D))
    AV = _normal_block(sv, (Hkv, r, D), 1.0 / np.sqrt(D))
    return dict(x=_to_storage(x, x_dtype), A_K=_to_storage(AK, x_dtype),
                A_V=_to_storage(AV, x_dtype), dtype=x_dtype)

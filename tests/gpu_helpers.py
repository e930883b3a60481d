"""Shared helpers for the GPU tests: move a drawn workload to the device, run
the library through its C-ABI binding, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads

TOL = {"f32": 1e-5, "bf16": 2e-3, "f16": 2e-3, "i8": 2e-3}


def say(*a):
    """Progress line flushed before each GPU step, so a failing run names its case."""
    print("[gpu]", *a, flush=True, file=sys.stderr)


def tensor(a: np.ndarray, tag: str, device="cuda"):
    import torch
    if tag == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_device(w: workloads.Workload, device="cuda"):
    import torch
    return dict(
        q=tensor(w.q, w.q_dtype, device),
        L_K=tensor(w.L_K, w.latent_dtype, device),
        L_V=tensor(w.L_V, w.latent_dtype, device),
        B_K=tensor(w.B_K, w.factor_dtype, device),
        B_V=tensor(w.B_V, w.factor_dtype, device),
        scales=None if w.scales is None else torch.from_numpy(w.scales).to(device),
        seq_lens=torch.from_numpy(w.seq_lens.astype(np.int32)).to(device),
    )


def f64_args(w: workloads.Workload):
    q = oracle.as_float64(w.q, w.q_dtype)
    LK = oracle.as_float64(w.L_K, w.latent_dtype)
    LV = oracle.as_float64(w.L_V, w.latent_dtype)
    BK = oracle.as_float64(w.B_K, w.factor_dtype)
    BV = oracle.as_float64(w.B_V, w.factor_dtype)
    sc = None if w.scales is None else w.scales.astype(np.float64)
    return q, LK, LV, BK, BV, w.seq_lens, sc


def oracle_all_rows(w: workloads.Workload) -> np.ndarray:
    """The oracle's whole output [B, Hq, d], one (sequence, kv-head) at a time:
    each step converts only that pair's valid latent rows to float64 and
    rebuilds K and V once for the group's query heads, so a full-size
    workload (2 GB of ragged latents) stays within a few hundred MB."""
    q = oracle.as_float64(w.q, w.q_dtype)
    BK = oracle.as_float64(w.B_K, w.factor_dtype)
    BV = oracle.as_float64(w.B_V, w.factor_dtype)
    G = w.group
    out = np.empty((w.batch, w.num_q_heads, w.head_dim))
    for b in range(w.batch):
        n = int(w.seq_lens[b])
        for g in range(w.num_kv_heads):
            LK = oracle.as_float64(w.L_K[b:b + 1, g:g + 1, :n], w.latent_dtype)
            LV = oracle.as_float64(w.L_V[b:b + 1, g:g + 1, :n], w.latent_dtype)
            sc = None
            if w.scales is not None:
                sc = w.scales[:, b:b + 1, g:g + 1, :n].astype(np.float64)
            out[b, g * G:(g + 1) * G] = oracle.decode_rows(
                q[b:b + 1, g * G:(g + 1) * G], LK, LV, BK[g:g + 1], BV[g:g + 1], np.array([n]),
                [(0, h) for h in range(G)], scales=sc, softmax_scale=w.softmax_scale)
    return out


def rel_rowmax(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((num / den).max())


def run_decode(w, dev=None, **kw):
    import torch
    import rank_kv_cache_head_amd as lr
    dev = dev or to_device(w)
    out = lr.decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"],
                    dev["scales"], softmax_scale=w.softmax_scale, **kw)
    torch.cuda.synchronize()
    return out

#!/usr/bin/env python3
"""Decode-attention benchmark over a per-head low-rank KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config gqa_vlm]

One step = one lrattn_decode call (partition kernel + combine kernel) over
one batch: every query head of every sequence attends to its whole cached
context once, i.e. one decode token per sequence for one attention layer.
Inputs are seeded synthetic tensors with the workload's shapes and value
distributions, resident in HBM before timing starts.

Printed: one JSON line.  `value` = decode tokens/s = B * K / (wall time of K
steps), bracketed by device synchronization.  `roofline` describes the
dominant (partition) kernel: algorithmic bytes per launch / mean launch time
measured with HIP events on the launch stream.  `cpu_baseline` times the fp64
CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X published HBM3E bandwidth
ROTATE_BYTES = 1 << 30       # rotate input copies so the 256 MB MALL cannot hold them
WORKLOAD_TEXT = {
    "tiny": "tiny: B=1 H=4 d=64 r=16 T=256 fp32",
    "llm7b": "7B-LLM-like decode: B=8 H=32 d=128 r=32 T=4096 bf16",
    "gqa_vlm": "GQA VLM long prompt: B=16 Hq=32 Hkv=8 d=128 r=64 T=16384 (576 image + text) bf16",
    "int8": "int8 latents: B=32 H=32 d=128 r=32 T=8192, fp32 per-token scales, bf16 q/factors",
    "ragged": "ragged long context: B=4 H=40 d=128 r=48 T<=131072 bf16",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="gqa_vlm",
                    choices=["tiny", "llm7b", "gqa_vlm", "int8", "ragged"])
    ap.add_argument("--num-splits", type=int, default=0,
                    help="0 = the workload's own (ragged: 256), else the library heuristic")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe", action="store_true",
                    help="also run the HBM read/copy probe kernels (calibration)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-cache baseline (same workload, K and V of d columns)")
    ap.add_argument("--no-rebuild", action="store_true",
                    help="skip the rebuilt-key (and rotated-key) mode timing")
    ap.add_argument("--no-append", action="store_true",
                    help="skip the append-step timing")
    ap.add_argument("--no-adaptive", action="store_true",
                    help="skip the attention-aware adaptive-rank timing")
    ap.add_argument("--no-modal", action="store_true",
                    help="skip the separate image/text factor timing")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the shared-latent (one stream for all heads) timing")
    return ap.parse_args()


def device_tensors(w, torch, copies):
    import numpy as np

    def t(a, tag):
        if tag == "bf16":
            x = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            x = torch.from_numpy(np.ascontiguousarray(a))
        return x.cuda()

    base = dict(q=t(w.q, w.q_dtype), B_K=t(w.B_K, w.factor_dtype), B_V=t(w.B_V, w.factor_dtype),
                seq_lens=torch.from_numpy(w.seq_lens.astype(np.int32)).cuda())
    sets = []
    lk = t(w.L_K, w.latent_dtype)
    lv = t(w.L_V, w.latent_dtype)
    sc = None if w.scales is None else torch.from_numpy(w.scales).cuda()
    for i in range(copies):
        if i == 0:
            sets.append((lk, lv, sc))
        else:
            sets.append((lk.clone(), lv.clone(), None if sc is None else sc.clone()))
    return base, sets


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in ("lrattn_kernels.hip", "lrattn_internal.hpp", "lrattn_device.hpp"):
        with open(os.path.join(ROOT, "rank_kv_cache_head_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(config: str, per_launch_alg: float):
    """HBM bytes per partition launch from committed rocprofv3 counter runs.

    Null when no counter file exists for this workload or the kernel source has
    changed since the counters were taken.
    """
    path = os.path.join(ROOT, "profiles", f"partition_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, gpu_out, seconds: float):
    """Time the fp64 oracle on whole sequences of the workload, cycling through
    the batch until `seconds` have passed (at least one sequence).  The first
    pass is also checked against the GPU output."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count(), "?"
    q = oracle.as_float64(w.q, w.q_dtype)
    BK = oracle.as_float64(w.B_K, w.factor_dtype)
    BV = oracle.as_float64(w.B_V, w.factor_dtype)
    G = w.group
    done = 0
    err = 0.0
    t0 = time.perf_counter()
    while True:
        b = done % w.batch
        n = int(w.seq_lens[b])
        for g in range(w.num_kv_heads):
            LK = oracle.as_float64(w.L_K[b:b + 1, g:g + 1, :n], w.latent_dtype)
            LV = oracle.as_float64(w.L_V[b:b + 1, g:g + 1, :n], w.latent_dtype)
            sc = None if w.scales is None else w.scales[:, b:b + 1, g:g + 1, :n].astype(np.float64)
            rows = [(0, h) for h in range(G)]
            ref = oracle.decode_rows(q[b:b + 1, g * G:(g + 1) * G], LK, LV, BK[g:g + 1],
                                     BV[g:g + 1], np.array([n]), rows, scales=sc)
            if done < w.batch:
                got = gpu_out[b, g * G:(g + 1) * G]
                e = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
                err = max(err, float(e.max()))
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{done} sequence decodes (all {w.num_q_heads} heads each, cycling over "
                       f"the {w.batch} sequences), fp64 NumPy rebuild-then-attend, {dt:.1f} s, "
                       f"BLAS {blas}",
                seconds=dt, max_rel_err_vs_gpu=err, checked_sequences=min(done, w.batch))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path is "
              "single-GPU, sharding across GPUs is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import workloads
    import rank_kv_cache_head_amd as lr

    lr.lib()  # fail loudly if the library is missing
    if args.num_splits == 0:
        args.num_splits = workloads.SPLITS.get(args.config, 0)
    t_gen = time.perf_counter()
    w = workloads.make(args.config)
    ab = w.algorithmic_bytes()
    gen_s = time.perf_counter() - t_gen
    lat_bytes = ab["latents"] + ab["scales"]
    copies = max(1, min(8, math.ceil(ROTATE_BYTES / max(1, lat_bytes))))
    base, sets = device_tensors(w, torch, copies)
    p = lr.params_for(base["q"], sets[0][0], base["B_K"], num_splits=args.num_splits)
    P, S = lr.plan(p)
    ws = torch.empty(lr.workspace_size(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")

    decs = [lr.Decoder(base["q"], lk, lv, base["B_K"], base["B_V"], base["seq_lens"], sc,
                       out=out, workspace=ws, num_splits=args.num_splits)
            for lk, lv, sc in sets]

    def step(i):
        decs[i % copies]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K whole decode steps, back to back
    K = args.steps
    e_beg, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_beg.record()
    for i in range(K):
        step(i)
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = e_beg.elapsed_time(e_end)
    gpu_out = out.cpu().numpy().astype(np.float64)

    # ---- the dominant kernel (partition) alone: K launches back to back
    # between two HIP events on the stream they are launched on (the average
    # launch duration), then K launches each between its own pair of events
    # (an isolated launch, which adds the launch latency)
    for i in range(min(args.warmup, 5)):
        decs[i % copies].partition()
    torch.cuda.synchronize()
    r_beg, r_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r_beg.record()
    for i in range(K):
        decs[i % copies].partition()
    r_end.record()
    torch.cuda.synchronize()
    launch_mean_s = r_beg.elapsed_time(r_end) / K / 1e3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        decs[i % copies].partition()
        ev[i][1].record()
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])

    # algorithmic bytes of one partition launch: valid latent rows (K and V),
    # their int8 scales, q and B_K
    part_bytes = ab["latents"] + ab["scales"] + ab["q"] + w.B_K.nbytes
    achieved = part_bytes / launch_mean_s / 1e9
    traffic = load_traffic(args.config, part_bytes)

    ms_per_step = wall / K * 1e3
    line = {
        "metric": "decode attention tokens/s per GPU + achieved HBM GB/s vs ~8 TB/s peak",
        "value": w.batch * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, workload shapes and distributions)",
        "config": {
            "workload": WORKLOAD_TEXT[args.config],
            "name": args.config,
            "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "rank": w.rank, "max_seq_len": w.max_seq_len,
            "valid_tokens": ab["valid_tokens"], "storage": w.latent_dtype,
            "num_splits": P, "split_tokens": S, "input_copies_rotated": copies,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel": lr.partition_kernel(p),
            "mean_launch_us": launch_mean_s * 1e6,
            "isolated_launch_us": float(launch_ms.mean()) * 1e3,
            "min_isolated_launch_us": float(launch_ms.min()) * 1e3,
            "algorithmic_bytes_per_launch": part_bytes,
        },
        "step_algorithmic_GBps": ab["total"] / (ms_per_step / 1e3) / 1e9,
        "timed_region_event_ms": region_ms,
        "input_generation_s": gen_s,
    }
    if not args.no_dense:
        line["dense_baseline"] = dense_baseline(w, torch, lr, args, ms_per_step)
    if not args.no_rebuild:
        line["rebuilt_keys"] = rebuilt_keys(w, torch, lr, args, base, sets, ms_per_step)
    if not args.no_append:
        line["append_step"] = append_step(w, torch, lr, args)
    if not args.no_shared:
        line["shared_latent"] = shared_latent(w, torch, lr, args, ms_per_step)
    if not args.no_modal:
        line["modal_factors"] = modal_factors(w, torch, lr, args, base, sets, ms_per_step)
    if not args.no_adaptive:
        line["adaptive_rank"] = adaptive_rank(w, torch, lr, args, base, sets, ms_per_step)
    if args.probe:
        line["probe"] = run_probe(torch, lr)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, gpu_out, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def dense_baseline(w, torch, lr, args, compressed_ms):
    """The same workload over an uncompressed cache: K, V [B, Hkv, T, d] in
    the latent storage type (random values drawn on the device; the content
    does not change the work), timed like the main loop.  None when such rows
    exceed what the kernels take (d * sizeof > 256 bytes)."""
    esz = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1}[w.latent_dtype]
    d = w.head_dim
    if d * esz > 256:
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + d)
    shape = (w.batch, w.num_kv_heads, w.max_seq_len, d)

    def draw():
        if w.latent_dtype == "i8":
            return torch.randint(-127, 128, shape, generator=g, device="cuda", dtype=torch.int8)
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.latent_dtype]
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dt)

    import numpy as np
    q = torch.randn((w.batch, w.num_q_heads, d), generator=g, device="cuda").to(
        torch.float32 if w.q_dtype == "f32" else
        torch.float16 if w.q_dtype == "f16" else torch.bfloat16)
    seq = torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    sc = None if w.scales is None else torch.from_numpy(w.scales).cuda()
    per_copy = 2 * math.prod(shape) * esz
    copies = max(1, min(4, math.ceil(ROTATE_BYTES / per_copy)))
    out = torch.empty((w.batch, w.num_q_heads, d), dtype=torch.float32, device="cuda")
    decs, keep = [], []
    for _ in range(copies):
        K, V = draw(), draw()
        keep.append((K, V))
        decs.append(lr.DenseDecoder(q, K, V, seq, sc, out=out, num_splits=args.num_splits))
    for i in range(args.warmup):
        decs[i % copies]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        decs[i % copies]()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    valid = int(w.seq_lens.sum())
    alg = valid * w.num_kv_heads * (2 * d * esz + (8 if w.latent_dtype == "i8" else 0))
    P, S = decs[0].plan
    res = dict(ms_per_step=ms, tokens_per_s=w.batch / (ms / 1e3),
               cache_bytes_per_step=alg, cache_GBps=alg / (ms / 1e3) / 1e9,
               kernel=lr.partition_kernel(decs[0].params), num_splits=P,
               speedup_of_factored=ms / compressed_ms)
    del decs, keep
    torch.cuda.empty_cache()
    return res


def rebuilt_keys(w, torch, lr, args, base, sets, absorbed_ms):
    """The same step with keys rebuilt on chip (lrattn_rebuild_decode), without
    and with a rotary table, on the same inputs.  None where the mode does not
    apply (it takes bf16 inputs, d in {64, 128}, r in {32, 64})."""
    G = w.num_q_heads // w.num_kv_heads
    if not (w.q_dtype == w.latent_dtype == w.factor_dtype == "bf16" and
            w.head_dim in (64, 128) and w.rank in (32, 64) and G in (1, 2, 4, 8)):
        return None
    import workloads
    rope = torch.from_numpy(workloads.rope_table(w.max_seq_len, w.head_dim)).cuda()
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    res = {}
    for name, tab in (("unrotated", None), ("rotated", rope)):
        decs = [lr.RebuildDecoder(base["q"], lk, lv, base["B_K"], base["B_V"], base["seq_lens"],
                                  tab, out=out, num_splits=args.num_splits)
                for lk, lv, _ in sets]
        n = len(decs)
        for i in range(args.warmup):
            decs[i % n]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            decs[i % n]()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        # per step: the latent rows read (HBM) and the rebuild's matrix-core
        # work, 2 r d flops per valid (token, kv-head)
        lat = w.algorithmic_bytes()["latents"]
        units = int(w.seq_lens.sum()) * w.num_kv_heads
        res[name] = dict(ms_per_step=ms, tokens_per_s=w.batch / (ms / 1e3),
                         vs_absorbed=ms / absorbed_ms,
                         latent_GBps=lat / (ms / 1e3) / 1e9,
                         frac_of_8TBps=lat / (ms / 1e3) / 8e12,
                         rebuild_TFLOPs=2.0 * w.rank * w.head_dim * units / (ms / 1e3) / 1e12)
    res["kernel"] = "partition_rebuild_kernel"
    res["num_splits"], res["split_tokens"] = lr.rebuild_plan(decs[0].params)
    return res


def append_step(w, torch, lr, args):
    """The append step of one decode token per sequence at the workload's
    shape: hidden width D = Hq * d (bf16 x and projections A_K, A_V
    [Hkv, r, D]) into the workload's latent type.  Timed over K calls."""
    import workloads
    D = w.num_q_heads * w.head_dim
    if D % 128 or w.batch > 64:
        return None
    inp = workloads.make_append(77, w.batch, w.num_kv_heads, D, w.rank, "bf16")
    import numpy as np

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    x, AK, AV = t(inp["x"]), t(inp["A_K"]), t(inp["A_V"])
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
           "i8": torch.int8}[w.latent_dtype]
    T = 64
    LK = torch.zeros((w.batch, w.num_kv_heads, T, w.rank), dtype=tdt, device="cuda")
    LV = torch.zeros_like(LK)
    sc = (torch.zeros((2, w.batch, w.num_kv_heads, T), device="cuda")
          if w.latent_dtype == "i8" else None)
    pos = torch.arange(w.batch, dtype=torch.int32, device="cuda") % T
    p = lr.AppendParams(w.batch, w.num_kv_heads, D, w.rank, T, lr.BF16, lr.BF16,
                        {"f32": lr.F32, "bf16": lr.BF16, "f16": lr.F16, "i8": lr.I8}[w.latent_dtype])
    ws = torch.empty(lr.append_workspace_size(p), dtype=torch.uint8, device="cuda")
    run = lr.Appender(x, AK, AV, pos, LK, LV, sc, workspace=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    esz = LK.element_size()
    alg = (AK.nbytes + AV.nbytes + x.nbytes +
           2 * w.batch * w.num_kv_heads * w.rank * esz + (0 if sc is None else 2 * w.batch * w.num_kv_heads * 4))
    return dict(us_per_call=us, model_dim=D, bytes_per_call=alg, GBps=alg / (us / 1e6) / 1e9,
                frac_of_8TBps=alg / (us / 1e6) / 8e12,
                kernels=("append_direct_kernel" if w.latent_dtype != "i8" and
                         w.num_kv_heads * 2 * (w.rank // 16) >= 192
                         else "append_partial_kernel + append_finish_kernel"))


def adaptive_rank(w, torch, lr, args, base, sets, plain_ms):
    """The same step with attention-aware rank (AttentionPack's adaptive
    decompression): tokens whose importance score is below 0.5 keep r/2
    latent coordinates; the step writes its logits and updates the scores
    (decay 0.9).  Scores drawn U(0, 1) on the device.  None where the shape
    has no adaptive kernel."""
    G = w.num_q_heads // w.num_kv_heads
    ok = {"bf16": w.rank in (32, 48, 64), "i8": w.rank == 32 and G in (1, 4),
          "f32": w.rank == 16 and G == 1}.get(w.latent_dtype, False)
    if not ok:
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(2026)
    imp = torch.rand((w.batch, w.num_kv_heads, w.max_seq_len), generator=g, device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    decs = [lr.AdaptiveDecoder(base["q"], lk, lv, base["B_K"], base["B_V"], base["seq_lens"],
                               imp, low_rank=w.rank // 2, threshold=0.5, decay=0.9, scales=sc,
                               out=out, num_splits=args.num_splits)
            for lk, lv, sc in sets]
    n = len(decs)
    for i in range(args.warmup):
        decs[i % n]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        decs[i % n]()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    valid = int(w.seq_lens.sum())
    # added traffic per valid token: importance read (partition), logits
    # written and read, importance read and written (update)
    extra = valid * (w.num_kv_heads * 4 + 2 * w.num_q_heads * 4 + w.num_kv_heads * 8)
    moved = w.algorithmic_bytes()["total"] + extra
    return dict(ms_per_step=ms, tokens_per_s=w.batch / (ms / 1e3), low_rank=w.rank // 2,
                vs_plain=ms / plain_ms, added_bytes_per_step=extra,
                step_GBps=moved / (ms / 1e3) / 1e9, frac_of_8TBps=moved / (ms / 1e3) / 8e12,
                kernel="partition_kernel (adaptive) + combine + importance_kernel")


def modal_factors(w, torch, lr, args, base, sets, one_set_ms):
    """The same step with separate factors for the workload's image block and
    its text (AttentionPack's modal separation): the image tokens and the
    text in partitions of their own, one latent-space sum per set in the
    combine.  None for workloads without an image block; the second factor
    set is drawn on the device (its values do not change the work)."""
    import workloads
    ni = int(workloads.SPECS[w.name].get("image_tokens", 0))
    if ni <= 0:
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(2025)
    BK = torch.stack([base["B_K"], (torch.randn(base["B_K"].shape, generator=g, device="cuda") *
                                    base["B_K"].float().std()).to(base["B_K"].dtype)])
    BV = torch.stack([base["B_V"], (torch.randn(base["B_V"].shape, generator=g, device="cuda") *
                                    base["B_V"].float().std()).to(base["B_V"].dtype)])
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    decs = [lr.ModalDecoder(base["q"], lk, lv, BK, BV, base["seq_lens"], ni, sc, out=out,
                            num_splits=args.num_splits)
            for lk, lv, sc in sets]
    n = len(decs)
    for i in range(args.warmup):
        decs[i % n]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        decs[i % n]()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    moved = w.algorithmic_bytes()["total"] + BK.nbytes // 2 + BV.nbytes // 2
    return dict(ms_per_step=ms, tokens_per_s=w.batch / (ms / 1e3), image_tokens=ni,
                vs_one_set=ms / one_set_ms,
                step_GBps=moved / (ms / 1e3) / 1e9, frac_of_8TBps=moved / (ms / 1e3) / 8e12,
                records=lr.modal_workspace_size(decs[0].params, ni))


def shared_latent(w, torch, lr, args, grouped_ms):
    """The workload's batch, query heads and lengths over one latent stream of
    R = 128 bf16 values per token shared by all heads, each head with its own
    factor blocks (AttentionPack's multi-head compression), timed like the
    main loop.  Random values drawn on the device."""
    if w.latent_dtype == "i8" or w.num_q_heads < 8:
        return None
    R, d, Hq = 128, w.head_dim, w.num_q_heads
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    shp = (w.batch, 1, w.max_seq_len, R)
    LK = torch.randn(shp, generator=g, device="cuda").to(torch.bfloat16)
    LV = torch.randn(shp, generator=g, device="cuda").to(torch.bfloat16)
    BK = (torch.randn((Hq, R, d), generator=g, device="cuda") / math.sqrt(R)).to(torch.bfloat16)
    BV = (torch.randn((Hq, R, d), generator=g, device="cuda") / math.sqrt(R)).to(torch.bfloat16)
    q = torch.randn((w.batch, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    import numpy as np
    sl = torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    p = lr.shared_params_for(q, LK, BK, num_splits=args.num_splits)
    ws = torch.empty(lr.shared_workspace_size(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, Hq, d), device="cuda")
    run = lambda: lr.shared_decode(q, LK, LV, BK, BV, sl, out=out, workspace=ws,
                                   num_splits=args.num_splits)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    valid = int(w.seq_lens.sum())
    lat = valid * 2 * R * 2
    res = dict(ms_per_step=ms, tokens_per_s=w.batch / (ms / 1e3), rank=R, streams=1,
               latent_bytes_per_step=lat, latent_GBps=lat / (ms / 1e3) / 1e9,
               frac_of_8TBps=lat / (ms / 1e3) / 8e12,
               heads_per_pass=min(64, 16 * -(-Hq // 16)) if Hq >= 32 else 8, vs_grouped=ms / grouped_ms)
    del LK, LV
    torch.cuda.empty_cache()
    return res


def run_probe(torch, lr):
    """Attainable streaming read/copy bandwidth (1 GiB buffers, rotated)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(2)
    sink = torch.empty(lr.probe_sink_floats(), dtype=torch.float32, device="cuda")
    res = {}
    for name, fn, moved in (("read", lambda: lr.probe_read(a, sink), n),
                            ("copy", lambda: lr.probe_copy(b, a), 2 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_GBps"] = moved * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
    return res


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Decode-attention benchmark over a per-head low-rank KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config ragged]

One step = one lrattn_decode call (partition kernel + combine kernel) over
one batch: every query head of every sequence attends to its whole cached
context once, i.e. one decode token per sequence for one attention layer.
Inputs are seeded synthetic tensors with the workload's shapes and value
distributions, resident in HBM before timing starts.  The headline workload
is the largest, ragged long context (4 sequences x 40 heads, lengths up to
131072, 256 partitions per head); the other workloads are timed the same way
and reported under `other_workloads`.  Every workload's decode runs exactly K
timed and W untimed steps; the side legs (dense cache, rebuilt keys, append,
shared stream, modal factors, adaptive rank) run at least `leg_steps` and
`leg_warmup` of each.

Printed: one JSON line.  `value` = decode tokens/s = B * K / (wall time of K
steps), bracketed by device synchronization.  `roofline` describes the
dominant (partition) kernel: algorithmic bytes per launch / mean launch time
measured with HIP events on the launch stream (with 64 or more partitions
per head the timed partition step also holds the small query-absorption
kernel launched ahead of it; `roofline.launch` names both), the counted HBM
traffic of a launch from the committed rocprofv3 counter record (and its
GB/s at the launch time measured here), and the read probe's attainable
GB/s.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
workload.
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
LEG_MIN_STEPS = 100          # timed calls of every sub-measurement, at least
LEG_MIN_WARMUP = 20          # untimed calls before them, at least
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
    ap.add_argument("--config", default="ragged",
                    choices=["tiny", "llm7b", "gqa_vlm", "int8", "ragged"],
                    help="headline workload (default: ragged, the largest: 4 x 40 heads over "
                         "up to 131072 tokens, 256 partitions per head)")
    ap.add_argument("--also", default="gqa_vlm,int8,llm7b,tiny",
                    help="comma-separated workloads also timed (plain decode step and "
                         "partition kernel), reported under other_workloads; '' for none")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="0 = the workload's own (ragged: 256), else the library heuristic")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the HBM read/copy probe kernels (attainable bandwidth)")
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


def lr_pre_absorb_splits() -> int:
    import rank_kv_cache_head_amd as lr
    return lr.PRE_ABSORB_SPLITS


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in ("lrattn_kernels.hip", "lrattn_internal.hpp", "lrattn_device.hpp"):
        with open(os.path.join(ROOT, "rank_kv_cache_head_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(config: str):
    """The partition launch's HBM traffic record from the committed rocprofv3
    counter runs (FETCH_SIZE, then WRITE_SIZE, each calibrated against a
    probe copy of known size): (bytes per launch, record file), or None when
    no record exists for this workload or the kernel source has changed since
    the counters were taken."""
    rel = os.path.join("profiles", f"partition_{config}_traffic.json")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch"), rel, rec.get("kernel_sha")


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
                e = float((np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())
                err = max(err, e) if np.isfinite(e) else float("inf")  # a NaN row must show
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{done} sequence decodes (all {w.num_q_heads} heads each, cycling over "
                       f"the {w.batch} sequences), fp64 NumPy rebuild-then-attend, {dt:.1f} s, "
                       f"BLAS {blas}",
                seconds=dt, max_rel_err_vs_gpu=err, checked_sequences=min(done, w.batch))


class Measured:
    """One workload's decode step, timed: K steps back to back (wall clock and
    HIP events), then the partition kernel alone (K launches between two HIP
    events on the stream they are launched on, and K isolated launches)."""

    def __init__(self, name, torch, lr, args, splits, steps, warmup):
        import numpy as np
        import workloads
        t_gen = time.perf_counter()
        w = workloads.make(name)
        self.w = w
        self.ab = ab = w.algorithmic_bytes()
        self.gen_s = time.perf_counter() - t_gen
        lat_bytes = ab["latents"] + ab["scales"]
        # rotate input copies so the 256 MB MALL cannot serve a step from cache
        self.copies = copies = max(1, min(8, math.ceil(ROTATE_BYTES / max(1, lat_bytes))))
        self.base, self.sets = base, sets = device_tensors(w, torch, copies)
        self.p = p = lr.params_for(base["q"], sets[0][0], base["B_K"], num_splits=splits)
        self.P, self.S = lr.plan(p)
        ws = torch.empty(lr.workspace_size(p), dtype=torch.uint8, device="cuda")
        self.out = out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32,
                                     device="cuda")
        decs = [lr.Decoder(base["q"], lk, lv, base["B_K"], base["B_V"], base["seq_lens"], sc,
                           out=out, workspace=ws, num_splits=splits)
                for lk, lv, sc in sets]

        for i in range(warmup):
            decs[i % copies]()
        torch.cuda.synchronize()
        e_beg, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e_beg.record()
        for i in range(steps):
            decs[i % copies]()
        e_end.record()
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - t0
        self.region_ms = e_beg.elapsed_time(e_end)
        self.gpu_out = out.cpu().numpy().astype(np.float64)

        for i in range(min(warmup, 5)):
            decs[i % copies].partition()
        torch.cuda.synchronize()
        r_beg, r_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r_beg.record()
        for i in range(steps):
            decs[i % copies].partition()
        r_end.record()
        torch.cuda.synchronize()
        self.launch_mean_s = r_beg.elapsed_time(r_end) / steps / 1e3
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            decs[i % copies].partition()
            ev[i][1].record()
        torch.cuda.synchronize()
        self.launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
        self.ms_per_step = self.wall / steps * 1e3
        # algorithmic bytes of one partition launch: valid latent rows (K and
        # V), their int8 scales, q and B_K
        self.part_bytes = ab["latents"] + ab["scales"] + ab["q"] + w.B_K.nbytes
        self.kernel = lr.partition_kernel(p)
        del decs

    def roofline(self):
        achieved = self.part_bytes / self.launch_mean_s / 1e9
        tr = load_traffic(self.w.name)
        res = {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None if tr is None else tr[0],
            "kernel": self.kernel,
            # with many partitions per head the timed partition step is two
            # launches: the query absorption, then the partition kernel
            "launch": (f"absorb_heads_kernel + {self.kernel}" if self.P >= lr_pre_absorb_splits()
                       else self.kernel),
            "mean_launch_us": self.launch_mean_s * 1e6,
            "isolated_launch_us": float(self.launch_ms.mean()) * 1e3,
            "min_isolated_launch_us": float(self.launch_ms.min()) * 1e3,
            "algorithmic_bytes_per_launch": self.part_bytes,
        }
        if tr is not None:
            # counter bandwidth: the counted HBM bytes of one launch over the
            # mean launch time measured here
            res["counter_GBps"] = tr[0] / self.launch_mean_s / 1e9
            res["traffic_over_algorithmic"] = tr[0] / self.part_bytes
            res["traffic_source"] = f"{tr[1]} (kernel source {tr[2]})"
        return res

    def summary(self):
        w = self.w
        return dict(workload=WORKLOAD_TEXT[w.name], ms_per_step=self.ms_per_step,
                    tokens_per_s=w.batch / (self.ms_per_step / 1e3),
                    step_algorithmic_GBps=self.ab["total"] / (self.ms_per_step / 1e3) / 1e9,
                    num_splits=self.P, split_tokens=self.S, roofline=self.roofline())

    def release(self, torch):
        self.base = self.sets = self.out = None
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path is "
              "single-GPU, sharding across GPUs is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    import rank_kv_cache_head_amd as lr

    lr.lib()  # fail loudly if the library is missing
    splits = args.num_splits or workloads.SPLITS.get(args.config, 0)
    K = args.steps
    m = Measured(args.config, torch, lr, args, splits, K, args.warmup)
    w, ab = m.w, m.ab
    line = {
        "metric": "decode attention tokens/s per GPU + achieved HBM GB/s vs ~8 TB/s peak",
        "value": w.batch * K / m.wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": m.ms_per_step,
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
            "seq_lens": [int(x) for x in w.seq_lens],
            "valid_tokens": ab["valid_tokens"], "storage": w.latent_dtype,
            "num_splits": m.P, "split_tokens": m.S, "input_copies_rotated": m.copies,
        },
        "roofline": m.roofline(),
        "step_algorithmic_GBps": ab["total"] / (m.ms_per_step / 1e3) / 1e9,
        "timed_region_event_ms": m.region_ms,
        "input_generation_s": m.gen_s,
    }
    # the other workloads' decode, before the legs below allocate their
    # large buffers; gqa_vlm's inputs stay resident for the legs that do
    # not apply to the headline workload (rebuilt keys need r 32 or 64,
    # separate image/text factors need an image block)
    # The side legs below (dense cache, rebuilt keys, append, shared stream,
    # modal factors, adaptive rank) are sub-measurements: each runs at least
    # LEG_MIN_STEPS timed calls after LEG_MIN_WARMUP untimed ones, so that a
    # short run (--steps 20 --warmup 5) still times them past their ramp-up
    # (the matrix-core-heavy rebuilt-key legs lower the shader clock over
    # their first launches); the decode of every workload uses K and W.
    la = argparse.Namespace(**vars(args))
    la.steps, la.warmup = max(args.steps, LEG_MIN_STEPS), max(args.warmup, LEG_MIN_WARMUP)
    line["leg_steps"], line["leg_warmup"] = la.steps, la.warmup
    others = [x for x in args.also.split(",") if x and x != args.config]
    aux = {}
    if others:
        line["other_workloads"] = {}
        for name in others:
            o = Measured(name, torch, lr, args, workloads.SPLITS.get(name, 0), K, args.warmup)
            line["other_workloads"][name] = o.summary()
            if name == "gqa_vlm":
                aux[name] = o
            else:
                o.release(torch)
    if not args.no_probe:
        sizes = [m.part_bytes] + [o["roofline"]["algorithmic_bytes_per_launch"]
                                  for o in line.get("other_workloads", {}).values()
                                  if o["roofline"]["algorithmic_bytes_per_launch"] >= (1 << 26)]
        line["probe"] = run_probe(torch, lr, sizes)
        by = line["probe"]["read_GBps_by_bytes"]
        # the read probe at the same byte count: what a streaming kernel of
        # this size attains on this device
        line["roofline"]["attainable_read_GBps"] = by[str(m.part_bytes)]
        line["roofline"]["frac_of_attainable"] = line["roofline"]["achieved"] / by[str(m.part_bytes)]
        for o in line.get("other_workloads", {}).values():
            key = str(o["roofline"]["algorithmic_bytes_per_launch"])
            if key in by:
                o["roofline"]["attainable_read_GBps"] = by[key]
                o["roofline"]["frac_of_attainable"] = o["roofline"]["achieved"] / by[key]

    def leg(fn, *extra, vlm_first=False):
        """A leg on the headline workload, else on gqa_vlm when the
        headline workload has no such mode (tagged with the workload).
        vlm_first: gqa_vlm first (AttentionPack's variants are methods for
        vision-language models; the gqa_vlm workload is that setting)."""
        order = [m] + list(aux.values())
        if vlm_first:
            order = list(aux.values()) + [m]
        for mm in order:
            sp = args.num_splits or workloads.SPLITS.get(mm.w.name, 0)
            res = fn(mm.w, torch, lr, la, sp, *[e(mm) for e in extra])
            if res is not None:
                res["workload"] = mm.w.name
                return res
        return None

    base_sets = (lambda mm: mm.base, lambda mm: mm.sets)
    step_ms = lambda mm: mm.ms_per_step  # noqa: E731
    if not args.no_dense:
        line["dense_baseline"] = leg(dense_baseline, step_ms)
    if not args.no_rebuild:
        line["rebuilt_keys"] = leg(rebuilt_keys, *base_sets, step_ms)
    if not args.no_append:
        line["append_step"] = leg(lambda w_, t_, l_, a_, sp_: append_step(w_, t_, l_, a_))
    if not args.no_shared:
        line["shared_latent"] = leg(shared_latent, step_ms, vlm_first=True)
    if not args.no_modal:
        line["modal_factors"] = leg(modal_factors, *base_sets, step_ms, vlm_first=True)
    if not args.no_adaptive:
        line["adaptive_rank"] = leg(adaptive_rank, *base_sets, step_ms, vlm_first=True)
        line["adaptive_rank_r128"] = leg(adaptive_rank_wide, vlm_first=True)
    gpu_out = m.gpu_out
    m.release(torch)
    for o in aux.values():
        o.release(torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, gpu_out, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def dense_baseline(w, torch, lr, args, splits, compressed_ms):
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
        decs.append(lr.DenseDecoder(q, K, V, seq, sc, out=out, num_splits=splits))
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


def rebuilt_keys(w, torch, lr, args, splits, base, sets, absorbed_ms):
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
                                  tab, out=out, num_splits=splits)
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
                         rebuild_TFLOPs=2.0 * w.rank * w.head_dim * units / (ms / 1e3) / 1e12,
                         clock_GHz=sample_clock(torch, lr, lambda i: decs[i % n](), args.steps))
    res["kernel"] = "partition_rebuild_kernel"
    res["num_splits"], res["split_tokens"] = lr.rebuild_plan(decs[0].params)
    return res


def sample_clock(torch, lr, launch, steps, every=5):
    """Shader clock while a leg runs: `steps` more launches back to back
    (untimed) with a clock sample (lrattn_probe_clock) after every `every`-th;
    min / mean / max GHz and the samples in launch order."""
    n = max(1, steps // every)
    out = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    for i in range(n * every):
        launch(i)
        if (i + 1) % every == 0:
            lr.probe_clock(out[2 * ((i + 1) // every - 1):])
    torch.cuda.synchronize()
    o = out.cpu().tolist()
    ghz = [o[2 * j] / o[2 * j + 1] / 10.0 for j in range(n) if o[2 * j + 1] > 0]
    if not ghz:
        return None
    return dict(min=min(ghz), mean=sum(ghz) / len(ghz), max=max(ghz),
                samples=[round(x, 3) for x in ghz])


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


def adaptive_rank(w, torch, lr, args, splits, base, sets, plain_ms):
    """The same step with attention-aware rank (AttentionPack's adaptive
    decompression): tokens whose importance score is below 0.5 keep r/2
    latent coordinates; the step writes its logits and updates the scores.
    Scores drawn U(0, 1) on the device; decay 1.0, so the update runs in
    full but leaves the scores, and with them the half of the rows at low
    rank, the same from step to step (with decay < 1 the scores would sink
    below the threshold within a few steps: a step's attention weights are
    ~1/T each).  None where the shape has no adaptive kernel."""
    G = w.num_q_heads // w.num_kv_heads
    ok = {"bf16": w.rank in (32, 48, 64, 128), "i8": w.rank == 32 and G in (1, 4),
          "f32": w.rank == 16 and G == 1}.get(w.latent_dtype, False)
    if not ok:
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(2026)
    imp = torch.rand((w.batch, w.num_kv_heads, w.max_seq_len), generator=g, device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    decs = [lr.AdaptiveDecoder(base["q"], lk, lv, base["B_K"], base["B_V"], base["seq_lens"],
                               imp, low_rank=w.rank // 2, threshold=0.5, decay=1.0, scales=sc,
                               out=out, num_splits=splits)
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
    kern = lr.adaptive_kernel(decs[0].params, decs[0].adaptive)
    return dict(ms_per_step=ms, tokens_per_s=w.batch / (ms / 1e3), low_rank=w.rank // 2,
                vs_plain=ms / plain_ms, added_bytes_per_step=extra,
                step_GBps=moved / (ms / 1e3) / 1e9, frac_of_8TBps=moved / (ms / 1e3) / 8e12,
                kernel=f"{kern} (adaptive) + combine_kernel + importance_kernel")


def adaptive_rank_wide(w, torch, lr, args, splits):
    """Attention-aware rank where a dropped half row is a whole HBM line: the
    workload's batch, heads and lengths with r = 128 bf16 latents (256-byte
    rows, two 128-byte lines), low rank 64, scores U(0, 1) against threshold
    0.5 (half the rows drop their second line; decay 1.0 keeps that half
    from step to step, see adaptive_rank), timed against the plain
    decode of the same r = 128 cache.  Random values drawn on the device;
    copies rotated over more than 1 GiB as in the main loop.  None for
    workloads whose queries are not bf16."""
    if not (w.q_dtype == w.factor_dtype == "bf16"):
        return None
    import numpy as np
    R, d = 128, w.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(2027)
    shp = (w.batch, w.num_kv_heads, w.max_seq_len, R)
    LK = torch.randn(shp, generator=g, device="cuda").to(torch.bfloat16)
    LV = torch.randn(shp, generator=g, device="cuda").to(torch.bfloat16)
    copies = max(1, -(-ROTATE_BYTES // (2 * LK.nbytes)))
    lats = [(LK, LV)] + [(LK.clone(), LV.clone()) for _ in range(copies - 1)]
    BK = (torch.randn((w.num_kv_heads, R, d), generator=g, device="cuda") / R ** 0.5).to(torch.bfloat16)
    BV = (torch.randn((w.num_kv_heads, R, d), generator=g, device="cuda") / R ** 0.5).to(torch.bfloat16)
    q = torch.randn((w.batch, w.num_q_heads, d), generator=g, device="cuda").to(torch.bfloat16)
    sl = torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    imp = torch.rand((w.batch, w.num_kv_heads, w.max_seq_len), generator=g, device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, d), dtype=torch.float32, device="cuda")

    def timed(decs):
        for i in range(args.warmup):
            decs[i % copies]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            decs[i % copies]()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    plain = [lr.Decoder(q, lk, lv, BK, BV, sl, out=out, num_splits=splits) for lk, lv in lats]
    plain_ms = timed(plain)
    del plain
    ad = [lr.AdaptiveDecoder(q, lk, lv, BK, BV, sl, imp, low_rank=R // 2, threshold=0.5,
                             decay=1.0, out=out, num_splits=splits) for lk, lv in lats]
    ad_ms = timed(ad)
    kern = lr.adaptive_kernel(ad[0].params, ad[0].adaptive)
    del ad, lats, LK, LV
    torch.cuda.empty_cache()
    valid = int(w.seq_lens.sum())
    lat = valid * w.num_kv_heads * 2 * R * 2
    return dict(rank=R, low_rank=R // 2, plain_ms_per_step=plain_ms, ms_per_step=ad_ms,
                vs_plain=ad_ms / plain_ms, latent_bytes_plain=lat,
                latent_lines_dropped=lat // 4,
                kernel=f"{kern} (adaptive) + combine_kernel + importance_kernel",
                input_copies_rotated=copies)


def modal_factors(w, torch, lr, args, splits, base, sets, one_set_ms):
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
                            num_splits=splits)
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


def shared_latent(w, torch, lr, args, splits, grouped_ms):
    """The workload's batch, query heads and lengths over one latent stream of
    R = 128 bf16 values per token shared by all heads, each head with its own
    factor blocks (AttentionPack's multi-head compression), timed like the
    main loop: calls marshalled once (SharedDecoder), and copies of the
    stream rotated so that more than 1 GiB is read between two reads of one
    copy (the 256 MB MALL cannot serve a repeat).  Random values drawn on
    the device."""
    if w.latent_dtype == "i8" or w.num_q_heads < 8:
        return None
    R, d, Hq = 128, w.head_dim, w.num_q_heads
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    shp = (w.batch, 1, w.max_seq_len, R)
    LK = torch.randn(shp, generator=g, device="cuda").to(torch.bfloat16)
    LV = torch.randn(shp, generator=g, device="cuda").to(torch.bfloat16)
    copies = max(1, -(-ROTATE_BYTES // (2 * LK.nbytes)))
    lats = [(LK, LV)] + [(LK.clone(), LV.clone()) for _ in range(copies - 1)]
    BK = (torch.randn((Hq, R, d), generator=g, device="cuda") / math.sqrt(R)).to(torch.bfloat16)
    BV = (torch.randn((Hq, R, d), generator=g, device="cuda") / math.sqrt(R)).to(torch.bfloat16)
    q = torch.randn((w.batch, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    import numpy as np
    sl = torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    p = lr.shared_params_for(q, LK, BK, num_splits=splits)
    ws = torch.empty(lr.shared_workspace_size(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, Hq, d), device="cuda")
    decs = [lr.SharedDecoder(q, lk, lv, BK, BV, sl, out=out, workspace=ws, num_splits=splits)
            for lk, lv in lats]
    for i in range(args.warmup):
        decs[i % copies]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        decs[i % copies]()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    valid = int(w.seq_lens.sum())
    lat = valid * 2 * R * 2
    res = dict(ms_per_step=ms, tokens_per_s=w.batch / (ms / 1e3), rank=R, streams=1,
               latent_bytes_per_step=lat, latent_GBps=lat / (ms / 1e3) / 1e9,
               frac_of_8TBps=lat / (ms / 1e3) / 8e12,
               heads_per_pass=min(64, 16 * -(-Hq // 16)) if Hq >= 32 else 8, vs_grouped=ms / grouped_ms,
               input_copies_rotated=copies)
    del LK, LV, lats, decs
    torch.cuda.empty_cache()
    return res


def run_probe(torch, lr, sizes=()):
    """Attainable streaming read/copy bandwidth over 1 GiB buffers, and the
    read bandwidth at each byte count in `sizes` (a partition launch's
    algorithmic bytes), reading ceil(1 GiB / n) buffers in turn so the
    256 MB MALL cannot serve a repeat."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(2)
    sink = torch.empty(lr.probe_sink_floats(), dtype=torch.float32, device="cuda")

    def rate(fn, moved, reps):
        for _ in range(3):
            fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return moved * reps / (e0.elapsed_time(e1) / 1e3) / 1e9

    res = {"read_GBps": rate(lambda i: lr.probe_read(a, sink), n, 10),
           "copy_GBps": rate(lambda i: lr.probe_copy(b, a), 2 * n, 10)}
    del a, b
    torch.cuda.empty_cache()
    by = {}
    for size in sizes:
        m = size // 4096 * 4096
        k = max(1, -(-n // m))
        bufs = [torch.empty(m, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(k)]
        by[str(size)] = rate(lambda i: lr.probe_read(bufs[i % k], sink), m, 50)
        del bufs
        torch.cuda.empty_cache()
    res["read_GBps_by_bytes"] = by
    return res


if __name__ == "__main__":
    main()

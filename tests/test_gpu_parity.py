"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Gate: max over output rows of ||gpu - oracle||_inf / ||oracle||_inf <= 2e-3
for bf16/fp16/int8 inputs and <= 1e-5 for fp32 inputs, with fp32 output.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, f64_args, oracle_all_rows, rel_rowmax, run_decode, say, tensor,
                         to_device)
import oracle

pytestmark = pytest.mark.gpu

SMALL = {
    # reduced sizes the oracle finishes in seconds; several partitions and a
    # ragged tail in every case
    "tiny": dict(),
    "llm7b": dict(B=2, Hq=4, Hkv=4, T=1500, seq_lens=[1500, 1037]),
    "gqa_vlm": dict(B=2, Hq=8, Hkv=2, T=2000, seq_lens=[2000, 1234]),
    "int8": dict(B=2, Hq=4, Hkv=4, T=1800, seq_lens=[1800, 999]),
    "ragged": dict(B=3, Hq=2, Hkv=2, T=6000, len_lo=1024, len_hi=6000),
}


def _full_oracle(w):
    args = f64_args(w)
    return oracle.decode(*args[:6], scales=args[6], softmax_scale=w.softmax_scale)


@pytest.mark.parametrize("splits", [0, 1, 3, 7])
@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_small_config(name, splits):
    w = workloads.make(name, **SMALL[name])
    say(f"small {name} splits={splits} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"T={w.max_seq_len} r={w.rank} lens={list(w.seq_lens)}")
    got = run_decode(w, num_splits=splits).cpu().numpy()
    ref = _full_oracle(w)
    err = rel_rowmax(got, ref)
    say(f"  err {err:.3e}")
    assert err <= TOL[w.latent_dtype], err


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_full_size(name):
    """Full-size workload in the launch configuration the benchmark times (the
    workload's own split count: 256 partitions per head for ragged, else the
    default plan).  Every output row is compared with the fp64 oracle, and
    the decode is repeated twice more on the same inputs: the split-K
    records and their fixed-order merge must give the same bits each time."""
    say(f"full {name}: drawing inputs")
    w = workloads.make(name)
    dev = to_device(w)
    splits = workloads.SPLITS.get(name, 0)
    say(f"full {name}: decode B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"T={w.max_seq_len} r={w.rank} splits={splits} lens={list(w.seq_lens)}")
    got = run_decode(w, dev, num_splits=splits).cpu().numpy()
    assert np.isfinite(got).all()
    for rep in range(2):
        say(f"full {name}: repeat {rep + 1}")
        again = run_decode(w, dev, num_splits=splits).cpu().numpy()
        assert np.array_equal(again, got), f"repeat {rep + 1} differs"
    say(f"full {name}: oracle over all {w.batch * w.num_q_heads} rows")
    ref = oracle_all_rows(w)
    err = rel_rowmax(got, ref)
    say(f"  err {err:.3e}")
    assert err <= TOL[w.latent_dtype], err


@pytest.mark.parametrize("name", ["ragged", "int8", "gqa_vlm"])
def test_nan_padding_never_read(name):
    kw = dict(SMALL[name])
    a = workloads.make(name, pad="zero", **kw)
    b = workloads.make(name, pad="nan", **kw)
    say(f"nan padding {name} lens={list(a.seq_lens)}")
    oa = run_decode(a).cpu().numpy()
    ob = run_decode(b).cpu().numpy()
    assert np.isfinite(ob).all()
    assert np.array_equal(oa, ob)


@pytest.mark.parametrize("name", ["gqa_vlm", "int8", "ragged"])
def test_bitwise_deterministic(name):
    w = workloads.make(name, **SMALL[name])
    dev = to_device(w)
    say(f"determinism {name}")
    first = run_decode(w, dev).cpu().numpy()
    for _ in range(9):
        assert np.array_equal(run_decode(w, dev).cpu().numpy(), first)


def test_split_count_invariance():
    w = workloads.make("gqa_vlm", B=1, Hq=4, Hkv=1, T=3000, seq_lens=[2999])
    dev = to_device(w)
    ref = _full_oracle(w)
    outs = []
    for splits in (1, 2, 5, 11, 64, 3000):
        say(f"split invariance splits={splits}")
        o = run_decode(w, dev, num_splits=splits).cpu().numpy()
        assert rel_rowmax(o, ref) <= 2e-3
        outs.append(o)
    for o in outs[1:]:
        assert rel_rowmax(o, outs[0]) <= 1e-5


def test_lengths_on_partition_boundaries():
    import rank_kv_cache_head_amd as lr
    T = 1024
    w0 = workloads.make("llm7b", B=1, Hq=2, Hkv=2, T=T)
    dev0 = to_device(w0)
    p = lr.params_for(dev0["q"], dev0["L_K"], dev0["B_K"], num_splits=8)
    P, S = lr.plan(p)
    assert S == 128
    lens = [1, 2, S - 1, S, S + 1, 2 * S, 3 * S - 1, T - 1, T]
    w = workloads.make("llm7b", B=len(lens), Hq=2, Hkv=2, T=T, seq_lens=lens)
    say(f"partition boundaries S={S} lens={lens}")
    got = run_decode(w, num_splits=8).cpu().numpy()
    ref = _full_oracle(w)
    assert rel_rowmax(got, ref) <= 2e-3


def test_single_token_cache():
    w = workloads.make("gqa_vlm", B=3, Hq=8, Hkv=2, T=1)
    say("T=1 cache")
    got = run_decode(w).cpu().numpy()
    assert rel_rowmax(got, _full_oracle(w)) <= 2e-3


def test_zero_negative_and_overlong_lengths():
    import torch
    w = workloads.make("llm7b", B=4, Hq=2, Hkv=2, T=300, seq_lens=[300, 300, 300, 300])
    dev = to_device(w)
    dev["seq_lens"] = torch.tensor([0, -5, 1000, 150], dtype=torch.int32, device="cuda")
    say("zero / negative / overlong lengths")
    got = run_decode(w, dev).cpu().numpy()
    assert (got[0] == 0).all() and (got[1] == 0).all()
    w2 = workloads.make("llm7b", B=4, Hq=2, Hkv=2, T=300, seq_lens=[300, 300, 300, 150])
    ref = _full_oracle(w2)
    assert rel_rowmax(got[2:], ref[2:]) <= 2e-3


def test_bf16_output():
    import torch
    w = workloads.make("gqa_vlm", **SMALL["gqa_vlm"])
    say("bf16 output")
    out = run_decode(w, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    got = out.float().cpu().numpy()
    # bf16 rounding of the output alone costs up to 2^-9 of each value
    assert rel_rowmax(got, _full_oracle(w)) <= 2e-3 + 2.0 ** -8


def test_explicit_softmax_scale():
    w = workloads.make("llm7b", B=2, Hq=2, Hkv=2, T=700)
    w.softmax_scale = 0.02
    say("explicit softmax scale")
    got = run_decode(w).cpu().numpy()
    assert rel_rowmax(got, _full_oracle(w)) <= 2e-3


def _matrix():
    cases = []
    for lt in ("f32", "bf16", "f16", "i8"):
        esz = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1}[lt]
        for r in (16, 32, 48, 64, 128):
            if r * esz > 256:
                continue
            for G in (1, 2, 4, 8):
                cases.append((lt, r, G, 128))
    cases += [("bf16", 32, 1, 64), ("bf16", 64, 4, 256), ("f32", 16, 2, 256), ("i8", 64, 8, 64),
              ("bf16", 48, 2, 64), ("bf16", 16, 1, 64), ("bf16", 128, 2, 256), ("f16", 48, 4, 256)]
    return cases


@pytest.mark.parametrize("lt,r,G,d", _matrix())
def test_instantiation_matrix(lt, r, G, d):
    base = "int8" if lt == "i8" else "tiny"
    fdt = "f32" if lt == "f32" else ("f16" if lt == "f16" else "bf16")
    kw = dict(B=2, Hq=2 * G, Hkv=2, d=d, r=r, T=700, seq_lens=[700, 333],
              q_dtype=fdt, factor_dtype=fdt, factor_std=1.0 / np.sqrt(r))
    if lt != "i8":
        kw["latent_dtype"] = lt
    w = workloads.make(base, seed=100 + r + G, **kw)
    say(f"matrix latent={lt} r={r} G={G} d={d}")
    got = run_decode(w, num_splits=3).cpu().numpy()
    err = rel_rowmax(got, _full_oracle(w))
    assert err <= TOL[lt], err


@pytest.mark.parametrize("lt,r,G", [("bf16", 48, 1), ("bf16", 32, 2), ("bf16", 48, 8),
                                    ("f32", 16, 1), ("f16", 64, 4), ("i8", 32, 1),
                                    ("i8", 64, 8), ("bf16", 128, 1)])
@pytest.mark.parametrize("T,splits", [(2000, 16), (2000, 37), (2000, 64), (16384, 64),
                                      (16640, 65), (8192, 256)])
def test_many_short_partitions(lt, r, G, T, splits):
    """Many short partitions per sequence on the VALU partition kernel (the
    long-context workload takes 256), on short and long rows (256 splits of
    8192 tokens: 32-token partitions; 64 and 65 splits of 16384 and 16640
    tokens: 256-token partitions, an even and an odd count of them).
    Lengths end inside, at and one past a run of two and of four partitions,
    one token into a partition, at one token, and at zero (a zero row, the
    other rows unchanged); the result matches the oracle and repeats bit for
    bit."""
    import torch
    S = -(-T // splits)
    lens = [T, 4 * S, 4 * S + 1, 4 * S - 1, 2 * S, 2 * S + 1, 1, S + 1, 3 * S + 5]
    base = "int8" if lt == "i8" else "tiny"
    fdt = "f32" if lt == "f32" else ("f16" if lt == "f16" else "bf16")
    kw = dict(B=len(lens), Hq=2 * G, Hkv=2, d=128, r=r, T=T, seq_lens=lens,
              q_dtype=fdt, factor_dtype=fdt, factor_std=1.0 / np.sqrt(r))
    if lt != "i8":
        kw["latent_dtype"] = lt
    w = workloads.make(base, seed=1500 + r + G + splits, **kw)
    dev = to_device(w)
    say(f"many short partitions latent={lt} r={r} G={G} T={T} splits={splits} lens={lens}")
    got = run_decode(w, dev, num_splits=splits).cpu().numpy()
    assert rel_rowmax(got, _full_oracle(w)) <= TOL[lt]
    again = run_decode(w, dev, num_splits=splits).cpu().numpy()
    assert np.array_equal(got, again)
    # a sequence of length 0 gives a zero row
    dev["seq_lens"] = torch.tensor([0] + lens[1:], dtype=torch.int32, device="cuda")
    z = run_decode(w, dev, num_splits=splits).cpu().numpy()
    assert (z[0] == 0).all() and np.array_equal(z[1:], got[1:])


@pytest.mark.parametrize("r,d,fdt", [(128, 256, "f32"), (128, 64, "f32"), (48, 64, "bf16"),
                                     (16, 64, "f32"), (128, 128, "f16"), (48, 256, "f32")])
def test_combine_projection_tiles(r, d, fdt):
    """The combine's projection reads B_V in 16-byte pieces, a column chunk of
    every NG-th row per thread: bf16 latents with fp32 / fp16 / bf16 factors
    cover two batches of pieces (r 128, d 256, fp32), a row count that does
    not fill the last row group (r 48 or 16 with 16 or 32 row groups), and
    one batch of 16 pieces."""
    kw = dict(B=2, Hq=2, Hkv=2, d=d, r=r, T=500, seq_lens=[500, 131], latent_dtype="bf16",
              q_dtype=fdt, factor_dtype=fdt, factor_std=1.0 / np.sqrt(r))
    w = workloads.make("tiny", seed=700 + r + d, **kw)
    say(f"combine projection r={r} d={d} factors={fdt}")
    got = run_decode(w, num_splits=3).cpu().numpy()
    assert rel_rowmax(got, _full_oracle(w)) <= TOL["bf16"]


@pytest.mark.parametrize("r,G", [(32, 4), (32, 8), (64, 4), (64, 8), (128, 4), (128, 8)])
def test_matrix_core_scores_exact_inputs(r, G):
    """bf16 latents with 4 or 8 heads per kv-head are scored on the matrix
    cores, with q~ split exactly into three bf16 terms.  Scores are then fp32
    sums of exact products, as on the VALU path, so the result must agree with
    the oracle to fp32 accumulation accuracy: far inside the bf16 gate, and
    tight enough that a q~ rounded to one or two bf16 terms fails.  Lengths
    cover empty, partial and full 16-token tiles; q_std = 4 spreads the logits
    so the reference max moves within partitions."""
    lens = [1, 15, 16, 17, 33, 200, 511, 700]
    w = workloads.make("gqa_vlm", seed=300 + r + G, B=len(lens), Hq=2 * G, Hkv=2, r=r, T=700,
                       seq_lens=lens, q_std=4.0, factor_std=1.0 / np.sqrt(r))
    dev = to_device(w)
    ref = _full_oracle(w)
    for splits in (1, 3, 0, 700):
        say(f"matrix-core scores r={r} G={G} splits={splits}")
        got = run_decode(w, dev, num_splits=splits).cpu().numpy()
        err = rel_rowmax(got, ref)
        say(f"  err {err:.3e}")
        assert err <= 2e-5, err


@pytest.mark.parametrize("qdt,fdt", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16"),
                                     ("bf16", "f16"), ("f32", "f32"), ("f16", "f32")])
@pytest.mark.parametrize("G,d", [(4, 64), (4, 256), (1, 128), (8, 128)])
def test_absorption_formats(qdt, fdt, G, d):
    """q . B_K^T runs on the matrix cores when q and B_K share a 2-byte
    format and on the VALU otherwise; both keep exact products and fp32
    sums, so every pairing must match the oracle to fp32 accuracy.  d = 64
    leaves half of the 32-wide k-steps of a chunk empty, d = 256 takes two
    chunks; G = 1 runs the VALU partition kernel, G = 4 and 8 the
    matrix-core one."""
    lens = [300, 17, 1]
    w = workloads.make("gqa_vlm", seed=400 + G + d, B=len(lens), Hq=2 * G, Hkv=2, d=d, r=64,
                       T=300, seq_lens=lens, q_dtype=qdt, factor_dtype=fdt,
                       factor_std=1.0 / np.sqrt(64))
    say(f"absorption q={qdt} factors={fdt} G={G} d={d}")
    got = run_decode(w, num_splits=2).cpu().numpy()
    err = rel_rowmax(got, _full_oracle(w))
    say(f"  err {err:.3e}")
    assert err <= 2e-5, err


def _dense_case(lt, d, G, seed):
    """A dense cache drawn like the factored one with r = d; the oracle runs
    it with identity factors (K = L . I)."""
    base = "int8" if lt == "i8" else "gqa_vlm"
    lens = [500, 129, 16, 1]
    kw = dict(B=len(lens), Hq=2 * G, Hkv=2, d=d, r=d, T=500, seq_lens=lens,
              factor_std=1.0 / np.sqrt(d))
    if lt != "i8":
        kw["latent_dtype"] = lt
    return workloads.make(base, seed=seed, **kw)


def _dense_oracle(w):
    q, K, V, _, _, lens, sc = f64_args(w)
    eye = np.broadcast_to(np.eye(w.head_dim), (w.num_kv_heads, w.head_dim, w.head_dim))
    return oracle.decode(q, K, V, eye, eye, lens, scales=sc, softmax_scale=w.softmax_scale)


@pytest.mark.parametrize("lt,d,G", [("bf16", 128, 4), ("bf16", 128, 1), ("bf16", 64, 8),
                                    ("f16", 128, 2), ("f32", 64, 4), ("i8", 128, 1),
                                    ("i8", 64, 4)])
def test_dense_decode_matches_oracle(lt, d, G):
    """The dense baseline is exact attention over the uncompressed cache
    (20 splits: one partition per wave on the VALU kernel)."""
    import rank_kv_cache_head_amd as lr
    w = _dense_case(lt, d, G, seed=500 + d + G)
    dev = to_device(w)
    say(f"dense {lt} d={d} G={G} lens={list(w.seq_lens)}")
    for splits in (0, 3, 20):
        got = lr.dense_decode(dev["q"], dev["L_K"], dev["L_V"], dev["seq_lens"], dev["scales"],
                              softmax_scale=w.softmax_scale, num_splits=splits)
        import torch
        torch.cuda.synchronize()
        err = rel_rowmax(got.cpu().numpy(), _dense_oracle(w))
        say(f"  splits={splits} err {err:.3e}")
        assert err <= 2e-5, err


@pytest.mark.parametrize("lt,G", [("bf16", 4), ("bf16", 1), ("i8", 2)])
def test_dense_equals_factored_with_identity_factors(lt, G):
    """With B_K = B_V = I the factored path computes the dense result in the
    same order: absorbing q into I and projecting through I add only exact
    zeros, so the two outputs are bitwise equal."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = _dense_case(lt, 128, G, seed=600 + G)
    dev = to_device(w)
    eye = torch.eye(128, dtype=dev["q"].dtype, device="cuda").expand(2, 128, 128).contiguous()
    say(f"dense == factored(I) {lt} G={G}")
    a = lr.dense_decode(dev["q"], dev["L_K"], dev["L_V"], dev["seq_lens"], dev["scales"],
                        num_splits=3)
    b = lr.decode(dev["q"], dev["L_K"], dev["L_V"], eye, eye, dev["seq_lens"], dev["scales"],
                  num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _rebuild_case(r, G, d, seed, lens=(700, 333, 17, 16, 1), T=700, pad="zero"):
    return workloads.make("gqa_vlm", seed=seed, pad=pad, B=len(lens), Hq=2 * G, Hkv=2, d=d, r=r,
                          T=T, seq_lens=list(lens), q_std=2.0, factor_std=1.0 / np.sqrt(r))


def _rope(w, base=500.0):
    import torch
    tab = workloads.rope_table(w.max_seq_len, w.head_dim, base=base)
    return tab, torch.from_numpy(tab).cuda()


@pytest.mark.parametrize("r,G,d", [(64, 4, 128), (32, 1, 128), (64, 8, 64), (32, 2, 64),
                                   (64, 1, 128), (32, 8, 128)])
@pytest.mark.parametrize("rotate", [False, True])
def test_rebuild_decode_matches_oracle(r, G, d, rotate):
    """Keys rebuilt on the matrix cores (exact products, fp32 sums), rotated
    in fp32, scored with both operands split exactly into bf16 terms: the
    result must match the oracle to fp32 accuracy, with and without rotation,
    at every split count, including one-token partitions."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = _rebuild_case(r, G, d, seed=700 + r + G + d + rotate)
    dev = to_device(w)
    args = f64_args(w)
    if rotate:
        tab, rope = _rope(w)
        ref = oracle.decode_rotated(*args[:6], tab.astype(np.float64), softmax_scale=w.softmax_scale)
    else:
        rope = None
        ref = _full_oracle(w)
    for splits in (1, 3, 0, 700):
        say(f"rebuild r={r} G={G} d={d} rotate={rotate} splits={splits}")
        got = lr.rebuild_decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"],
                                dev["seq_lens"], rope, softmax_scale=w.softmax_scale,
                                num_splits=splits)
        torch.cuda.synchronize()
        err = rel_rowmax(got.cpu().numpy(), ref)
        say(f"  err {err:.3e}")
        assert err <= 2e-5, err


def test_rebuild_equals_absorbed_without_rotation():
    """Absorbed and rebuilt keys are the same quantity (associativity): the
    two kernels agree to fp32 accuracy on the GPU."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = _rebuild_case(64, 4, 128, seed=801)
    dev = to_device(w)
    say("rebuilt == absorbed")
    a = lr.rebuild_decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"],
                          dev["seq_lens"])
    b = run_decode(w, dev)
    torch.cuda.synchronize()
    assert rel_rowmax(a.cpu().numpy(), b.cpu().numpy().astype(np.float64)) <= 2e-5


def test_rebuild_nan_padding_and_determinism():
    import torch
    import rank_kv_cache_head_amd as lr
    wz = _rebuild_case(64, 4, 128, seed=802, lens=(500, 77, 3), T=512)
    wn = _rebuild_case(64, 4, 128, seed=802, lens=(500, 77, 3), T=512, pad="nan")
    _, rope = _rope(wz)
    say("rebuild NaN padding")
    outs = []
    for w in (wz, wn, wz):
        dev = to_device(w)
        o = lr.rebuild_decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"],
                              dev["seq_lens"], rope)
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy())
    assert np.isfinite(outs[1]).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_rebuild_full_size_rotated():
    """gqa_vlm at full size with rotation, default plan; every sequence
    checked against the oracle (one sequence at a time in float64)."""
    import torch
    import rank_kv_cache_head_amd as lr
    say("rebuild full gqa_vlm: drawing inputs")
    w = workloads.make("gqa_vlm")
    dev = to_device(w)
    tab, rope = _rope(w, base=10000.0)
    say("rebuild full gqa_vlm: decode")
    got = lr.rebuild_decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"],
                            dev["seq_lens"], rope).cpu().numpy()
    assert np.isfinite(got).all()
    f = oracle.as_float64
    tab64 = tab.astype(np.float64)
    err = 0.0
    for b in range(w.batch):
        sel = [b]
        ref = oracle.decode_rotated(f(w.q[sel], w.q_dtype), f(w.L_K[sel], w.latent_dtype),
                                    f(w.L_V[sel], w.latent_dtype), f(w.B_K, w.factor_dtype),
                                    f(w.B_V, w.factor_dtype), w.seq_lens[sel], tab64)
        err = max(err, rel_rowmax(got[sel], ref))
    say(f"  err {err:.3e}")
    assert err <= 2e-5, err


@pytest.mark.parametrize("lt,S,Hq,r,d", [("bf16", 1, 32, 64, 128), ("bf16", 1, 12, 48, 128),
                                         ("f16", 2, 16, 32, 64), ("i8", 1, 40, 32, 128),
                                         ("f32", 1, 8, 16, 64), ("bf16", 3, 3, 32, 128),
                                         # q~ from factor rows read in two rounds
                                         ("bf16", 1, 8, 64, 256), ("f32", 1, 4, 32, 128),
                                         # one pass per tile (bf16, r 32/64/128, >= 32 heads)
                                         ("bf16", 1, 32, 128, 128), ("bf16", 2, 64, 32, 64),
                                         ("bf16", 1, 64, 64, 128),
                                         # 3 and 4 blocks of 16 heads per workgroup, full
                                         # or with a partial last block or group
                                         ("bf16", 1, 40, 64, 128), ("bf16", 2, 100, 32, 64),
                                         ("bf16", 1, 48, 128, 128), ("bf16", 1, 80, 128, 64)])
def test_shared_decode_matches_oracle(lt, S, Hq, r, d):
    """Shared latent streams (AttentionPack's multi-head compression) with a
    factor block per query head: q~ per head, then partitions over head
    groups of up to 8 reading the same stream, or (bf16, at least 32 heads
    per stream) one pass per tile for up to 64 heads (2, 3 or 4 blocks of
    16); combine with each head's B_V."""
    import torch
    import rank_kv_cache_head_amd as lr
    base = "int8" if lt == "i8" else "gqa_vlm"
    lens = [300, 97, 16, 1]
    kw = dict(B=len(lens), Hq=Hq, Hkv=Hq, d=d, r=r, T=300, seq_lens=lens,
              factor_std=1.0 / np.sqrt(r))
    if lt != "i8":
        kw["latent_dtype"] = lt
    if lt == "f32":
        kw.update(q_dtype="f32", factor_dtype="f32")
    w = workloads.make(base, seed=1100 + Hq + r, **kw)
    dev = to_device(w)
    LK = dev["L_K"][:, :S].contiguous()
    LV = dev["L_V"][:, :S].contiguous()
    sc = None if dev["scales"] is None else dev["scales"][:, :, :S].contiguous()
    f = oracle.as_float64
    ref = oracle.decode_shared(f(w.q, w.q_dtype), f(w.L_K, w.latent_dtype)[:, :S],
                               f(w.L_V, w.latent_dtype)[:, :S], f(w.B_K, w.factor_dtype),
                               f(w.B_V, w.factor_dtype), w.seq_lens,
                               scales=None if w.scales is None else w.scales[:, :, :S].astype(np.float64),
                               softmax_scale=w.softmax_scale)
    for splits in (0, 3):
        say(f"shared {lt} S={S} Hq={Hq} r={r} d={d} splits={splits}")
        got = lr.shared_decode(dev["q"], LK, LV, dev["B_K"], dev["B_V"], dev["seq_lens"], sc,
                               softmax_scale=w.softmax_scale, num_splits=splits)
        torch.cuda.synchronize()
        err = rel_rowmax(got.cpu().numpy(), ref)
        say(f"  err {err:.3e}")
        assert err <= 2e-5, err


@pytest.mark.parametrize("Hq", [32, 48])
def test_shared_one_pass_edges(Hq):
    """The one-pass shared kernel (32 or 48 heads per stream: 2 or 3 blocks
    of 16 per workgroup): an empty sequence gives a zero row, NaN padding
    past each length is never read, and the result repeats bit for bit."""
    import torch
    import rank_kv_cache_head_amd as lr
    kw = dict(B=3, Hq=Hq, Hkv=Hq, d=128, r=64, T=600, seq_lens=[600, 0, 77],
              factor_std=0.125)
    wz = workloads.make("gqa_vlm", seed=1300, pad="zero", **kw)
    wn = workloads.make("gqa_vlm", seed=1300, pad="nan", **kw)
    outs = []
    for w in (wz, wn, wz):
        dev = to_device(w)
        say("shared one pass edges")
        o = lr.shared_decode(dev["q"], dev["L_K"][:, :1].contiguous(),
                             dev["L_V"][:, :1].contiguous(), dev["B_K"], dev["B_V"],
                             dev["seq_lens"])
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy())
    assert np.isfinite(outs[1]).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert (outs[0][1] == 0).all()
    f = oracle.as_float64
    sel = [0, 2]
    ref = oracle.decode_shared(f(wz.q[sel], wz.q_dtype), f(wz.L_K[sel], wz.latent_dtype)[:, :1],
                               f(wz.L_V[sel], wz.latent_dtype)[:, :1], f(wz.B_K, wz.factor_dtype),
                               f(wz.B_V, wz.factor_dtype), wz.seq_lens[sel])
    assert rel_rowmax(outs[0][sel], ref) <= 2e-5


def test_shared_full_size_gqa_vlm():
    """The benchmark's shared-stream shape at full size: gqa_vlm's batch,
    heads and lengths over one stream of R = 128 bf16 latents shared by all
    32 heads (one pass per tile), each head with its own factor blocks;
    every sequence against the oracle (one at a time in float64)."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = workloads.make("gqa_vlm", Hkv=1, r=128, factor_std=1.0 / np.sqrt(128))
    wf = workloads.make("gqa_vlm", seed=1400, B=1, Hkv=w.num_q_heads, r=128, T=16,
                        seq_lens=[16], factor_std=1.0 / np.sqrt(128))
    say("shared full gqa_vlm: inputs")
    dev = to_device(w)
    BK, BV = tensor(wf.B_K, wf.factor_dtype), tensor(wf.B_V, wf.factor_dtype)
    say("shared full gqa_vlm: decode")
    got = lr.shared_decode(dev["q"], dev["L_K"], dev["L_V"], BK, BV, dev["seq_lens"],
                           softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.isfinite(got).all()
    f = oracle.as_float64
    BK64, BV64 = f(wf.B_K, wf.factor_dtype), f(wf.B_V, wf.factor_dtype)
    err = 0.0
    for b in range(w.batch):
        sel = [b]
        ref = oracle.decode_shared(f(w.q[sel], w.q_dtype), f(w.L_K[sel], w.latent_dtype),
                                   f(w.L_V[sel], w.latent_dtype), BK64, BV64, w.seq_lens[sel],
                                   softmax_scale=w.softmax_scale)
        err = max(err, rel_rowmax(got[sel], ref))
    say(f"  err {err:.3e}")
    assert err <= 2e-5, err


def test_shared_equals_per_head_cache():
    """A stream shared by G heads gives the result of a per-head cache that
    repeats the stream's latents for each head (same factors)."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = workloads.make("gqa_vlm", seed=1200, B=2, Hq=16, Hkv=16, d=128, r=64, T=256,
                       seq_lens=[256, 100], factor_std=0.125)
    dev = to_device(w)
    LK1, LV1 = dev["L_K"][:, :1].contiguous(), dev["L_V"][:, :1].contiguous()
    say("shared == per-head replicated")
    a = lr.shared_decode(dev["q"], LK1, LV1, dev["B_K"], dev["B_V"], dev["seq_lens"])
    b = lr.decode(dev["q"], LK1.expand(2, 16, 256, 64).contiguous(),
                  LV1.expand(2, 16, 256, 64).contiguous(), dev["B_K"], dev["B_V"],
                  dev["seq_lens"])
    torch.cuda.synchronize()
    assert rel_rowmax(a.cpu().numpy(), b.cpu().numpy().astype(np.float64)) <= 2e-5


def test_shared_decoder_object_equals_function():
    """SharedDecoder (arguments marshalled once, as the benchmark times it)
    gives the bits of shared_decode on the same inputs, call after call, on
    the one-pass shape (32 heads, one stream of rank 128)."""
    import torch
    import rank_kv_cache_head_amd as lr
    g = torch.Generator(device="cuda")
    g.manual_seed(1300)
    B, Hq, T, R, d = 2, 32, 700, 128, 128
    LK = torch.randn((B, 1, T, R), generator=g, device="cuda").to(torch.bfloat16)
    LV = torch.randn((B, 1, T, R), generator=g, device="cuda").to(torch.bfloat16)
    BK = (torch.randn((Hq, R, d), generator=g, device="cuda") / R ** 0.5).to(torch.bfloat16)
    BV = (torch.randn((Hq, R, d), generator=g, device="cuda") / R ** 0.5).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    sl = torch.tensor([700, 333], dtype=torch.int32, device="cuda")
    say("SharedDecoder == shared_decode")
    ref = lr.shared_decode(q, LK, LV, BK, BV, sl).clone()
    dec = lr.SharedDecoder(q, LK, LV, BK, BV, sl)
    for _ in range(3):
        out = dec()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_guard_bands_untouched():
    import torch
    import rank_kv_cache_head_amd as lr
    w = workloads.make("ragged", **SMALL["ragged"])
    dev = to_device(w)
    p = lr.params_for(dev["q"], dev["L_K"], dev["B_K"])
    need = lr.workspace_size(p)
    n_out = w.batch * w.num_q_heads * w.head_dim
    guard = 4096
    out_buf = torch.full((n_out + 2 * guard,), 1234.5, dtype=torch.float32, device="cuda")
    ws_buf = torch.full((need // 4 + 2 * guard,), -777.25, dtype=torch.float32, device="cuda")
    out = out_buf[guard:guard + n_out].view(w.batch, w.num_q_heads, w.head_dim)
    ws = ws_buf[guard:guard + need // 4]
    say("guard bands")
    lr.decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"],
              dev["scales"], out=out, workspace=ws)
    torch.cuda.synchronize()
    ob = out_buf.cpu().numpy()
    wb = ws_buf.cpu().numpy()
    assert (ob[:guard] == 1234.5).all() and (ob[guard + n_out:] == 1234.5).all()
    assert (wb[:guard] == -777.25).all() and (wb[guard + need // 4:] == -777.25).all()
    assert rel_rowmax(out.cpu().numpy(), _full_oracle(w)) <= 2e-3


@pytest.mark.parametrize("name,splits", [("int8", 5), ("int8", 100), ("gqa_vlm", 80)])
def test_partition_then_combine_equals_decode(name, splits):
    """lrattn_partition then lrattn_combine give lrattn_decode's bits, also
    with the queries absorbed ahead of the partition kernel (64 or more
    partitions per head)."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = workloads.make(name, **SMALL[name])
    dev = to_device(w)
    say(f"partition + combine {name} splits={splits}")
    ref = run_decode(w, dev, num_splits=splits).cpu().numpy()
    ws = lr.partition(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["seq_lens"],
                      dev["scales"], num_splits=splits)
    p = lr.params_for(dev["q"], dev["L_K"], dev["B_K"], num_splits=splits)
    assert (lr.plan(p)[0] >= lr.PRE_ABSORB_SPLITS) == (splits >= 64)
    out = lr.combine(p, dev["B_V"], dev["seq_lens"], ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
    assert rel_rowmax(out.cpu().numpy(), _full_oracle(w)) <= TOL[w.latent_dtype]


@pytest.mark.parametrize("base,kw", [
    # fp32 factors at d = 256: 64 pieces per factor row, four load rounds
    ("gqa_vlm", dict(B=2, Hq=2, Hkv=2, r=128, d=256, T=700, seq_lens=[700, 333],
                     q_dtype="f32", factor_dtype="f32")),
    # 2-byte factors at r = 16, d = 64: 128 pieces, half a round
    ("tiny", dict(B=2, T=256, seq_lens=[256, 100], q_dtype="bf16", factor_dtype="bf16")),
    # fp16 query and factors, 4 heads per kv-head, d = 64: 8 pieces per row
    ("gqa_vlm", dict(B=2, Hq=8, Hkv=2, r=32, d=64, T=900, seq_lens=[900, 45],
                     q_dtype="f16", factor_dtype="f16")),
    # the ragged workload's shape family: r = 48, one head per kv-head
    ("ragged", dict(B=3, Hq=3, Hkv=3, T=2000, seq_lens=[2000, 1500, 64])),
])
def test_queries_absorbed_ahead(base, kw):
    """With 64 or more partitions per head the queries are absorbed once per
    query head by a kernel of their own; its factor-piece geometry depends
    on r, d and the factor type.  Compared with the oracle at 100 splits."""
    w = workloads.make(base, **kw)
    say(f"absorbed ahead {base} {kw}")
    got = run_decode(w, num_splits=100).cpu().numpy()
    err = rel_rowmax(got, _full_oracle(w))
    say(f"  err {err:.3e}")
    assert err <= TOL[w.latent_dtype], err


def test_side_stream():
    import torch
    w = workloads.make("gqa_vlm", **SMALL["gqa_vlm"])
    dev = to_device(w)
    ref = run_decode(w, dev).cpu().numpy()
    s = torch.cuda.Stream()
    say("side stream")
    import rank_kv_cache_head_amd as lr
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = lr.decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"],
                        dev["seq_lens"], dev["scales"])
    s.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


def test_host_errors_through_binding():
    import torch
    import rank_kv_cache_head_amd as lr
    w = workloads.make("llm7b", B=1, Hq=2, Hkv=2, T=64)
    dev = to_device(w)
    say("binding errors")
    big = torch.empty(dev["q"].numel() + 8, dtype=torch.bfloat16, device="cuda")
    q_mis = big[1:1 + dev["q"].numel()].view_as(dev["q"])
    with pytest.raises(lr.LrattnError) as e:
        lr.decode(q_mis, dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"])
    assert e.value.status == -5
    with pytest.raises(lr.LrattnError) as e:
        lr.decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"],
                  num_splits=65)
    assert e.value.status == -7
    with pytest.raises(ValueError):
        lr.decode(dev["q"].cpu(), dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"])


def test_probe_copy_and_read():
    import torch
    import rank_kv_cache_head_amd as lr
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 22,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    say("probe copy/read")
    lr.probe_copy(dst, src)
    sink = torch.empty(lr.probe_sink_floats(), dtype=torch.float32, device="cuda")
    lr.probe_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_probe_clock():
    """The shader-clock sample reads a plausible clock (the part runs at up
    to 2.4 GHz) over its ~5 us spin of the 100 MHz real-time counter."""
    import torch
    import rank_kv_cache_head_amd as lr
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    say("probe clock")
    lr.probe_clock(out)
    lr.probe_clock(out[2:])
    torch.cuda.synchronize()
    o = out.cpu().tolist()
    for j in range(2):
        assert 400 <= o[2 * j + 1] <= 5000, o
        assert 0.3 <= o[2 * j] / o[2 * j + 1] / 10.0 <= 3.5, o


def test_back_to_back_inputs_share_a_workspace():
    """Two different inputs decoded back to back on one workspace, no host
    sync in between: each result must come from its own call's partials."""
    import torch
    import rank_kv_cache_head_amd as lr
    wa = workloads.make("gqa_vlm", seed=21, **SMALL["gqa_vlm"])
    wb = workloads.make("gqa_vlm", seed=22, **SMALL["gqa_vlm"])
    da, db = to_device(wa), to_device(wb)
    p = lr.params_for(da["q"], da["L_K"], da["B_K"], num_splits=5)
    ws = torch.empty(lr.workspace_size(p), dtype=torch.uint8, device="cuda")
    say("back-to-back inputs on one workspace")
    outs = []
    for _ in range(3):
        for d in (da, db):
            outs.append(lr.decode(d["q"], d["L_K"], d["L_V"], d["B_K"], d["B_V"], d["seq_lens"],
                                  workspace=ws, num_splits=5))
    torch.cuda.synchronize()
    ra, rb = _full_oracle(wa), _full_oracle(wb)
    for i, o in enumerate(outs):
        assert rel_rowmax(o.cpu().numpy(), ra if i % 2 == 0 else rb) <= 2e-3, i


def test_graph_capture_replay():
    """lrattn_decode captured in a HIP graph and replayed with new inputs
    copied into the captured buffers; every replay must equal eager decode."""
    import torch
    import rank_kv_cache_head_amd as lr
    w0 = workloads.make("int8", seed=31, **SMALL["int8"])
    d0 = to_device(w0)
    dec = lr.Decoder(d0["q"], d0["L_K"], d0["L_V"], d0["B_K"], d0["B_V"], d0["seq_lens"],
                     d0["scales"], num_splits=3)
    torch.cuda.synchronize()
    say("graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dec()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        # decode() launches on the current (capturing) stream
        lr.decode(d0["q"], d0["L_K"], d0["L_V"], d0["B_K"], d0["B_V"], d0["seq_lens"],
                  d0["scales"], out=dec.out, workspace=dec.workspace, num_splits=3)
    torch.cuda.synchronize()
    for seed in (32, 33, 34):
        w = workloads.make("int8", seed=seed, **SMALL["int8"])
        d = to_device(w)
        for k in ("q", "L_K", "L_V", "B_K", "B_V", "scales", "seq_lens"):
            d0[k].copy_(d[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = dec.out.cpu().numpy().copy()
        eager = lr.decode(d["q"], d["L_K"], d["L_V"], d["B_K"], d["B_V"], d["seq_lens"],
                          d["scales"], num_splits=3)
        torch.cuda.synchronize()
        assert np.array_equal(got, eager.cpu().numpy()), seed
        assert rel_rowmax(got, _full_oracle(w)) <= 2e-3

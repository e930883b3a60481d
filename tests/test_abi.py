"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any device work.

Every call below is made with arguments the host layer must reject, so no
kernel is ever launched here (there is no GPU in the CPU suite).  Pointers are
fake, never dereferenced: validation looks only at their values.
"""
import ctypes
import math

import pytest

import rank_kv_cache_head_amd as lr

ALIGNED = 0x10000          # a fake, 16-byte aligned device address
MISALIGNED = 0x10004


def params(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, rank=64, max_seq_len=1000,
                q_dtype=lr.BF16, latent_dtype=lr.BF16, factor_dtype=lr.BF16, out_dtype=lr.F32,
                softmax_scale=0.0, num_splits=0)
    base.update(kw)
    return lr.Params(**base)


def decode_status(p, q=ALIGNED, lk=ALIGNED, lv=ALIGNED, bk=ALIGNED, bv=ALIGNED, scales=None,
                  seq=ALIGNED, out=ALIGNED, ws=ALIGNED, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = 0        # too small: a fully valid call would otherwise launch
    return lr.lib().lrattn_decode(ctypes.byref(p), q, lk, lv, bk, bv, scales, seq, out, ws,
                                  ws_bytes, None)


def test_library_loads_and_exports_everything_declared():
    L = lr.lib()
    names = lr.declared_symbols()
    assert {"lrattn_decode", "lrattn_workspace_size", "lrattn_status_string", "lrattn_plan",
            "lrattn_partition_kernel",
            "lrattn_partition", "lrattn_combine", "lrattn_probe_read", "lrattn_probe_copy",
            "lrattn_probe_sink_floats", "lrattn_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared but not exported"
    assert lr.version() == 10000


def test_status_strings():
    for code in range(-8, 1):
        assert lr.status_string(code) and lr.status_string(code) != "unknown status"
    assert lr.status_string(-99) == "unknown status"


def test_workspace_size_formula():
    p = params(num_splits=7)
    P, S = lr.plan(p)
    assert S == math.ceil(1000 / 7) and P == math.ceil(1000 / S)
    records = 2 * 8 * P * (64 + 4) * 4
    assert lr.workspace_size(p) == (records + 255) // 256 * 256


def test_workspace_size_with_absorbed_queries():
    """From LRATTN_PRE_ABSORB_SPLITS partitions per head the workspace also
    holds the absorbed queries [B, Hq, r] fp32 after the records."""
    assert lr.PRE_ABSORB_SPLITS == 64
    for splits, extra in ((63, False), (64, True), (200, True)):
        p = params(num_splits=splits, max_seq_len=1024)
        P, _ = lr.plan(p)
        records = (2 * 8 * P * (64 + 4) * 4 + 255) // 256 * 256
        qt = (2 * 8 * 64 * 4 + 255) // 256 * 256 if P >= 64 else 0
        assert (P >= 64) == extra, (splits, P)
        assert lr.workspace_size(p) == records + qt, splits


@pytest.mark.parametrize("kw,exp_P,exp_S", [
    # the five workloads' shapes and storage types
    (dict(batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64, rank=16, max_seq_len=256,
          q_dtype=lr.F32, latent_dtype=lr.F32, factor_dtype=lr.F32), 1, 256),
    (dict(batch=8, num_q_heads=32, num_kv_heads=32, rank=32, max_seq_len=4096), 4, 1024),
    (dict(batch=16, num_q_heads=32, num_kv_heads=8, rank=64, max_seq_len=16384), 4, 4096),
    (dict(batch=32, num_q_heads=32, num_kv_heads=32, rank=32, max_seq_len=8192,
          latent_dtype=lr.I8), 4, 2048),
    (dict(batch=4, num_q_heads=40, num_kv_heads=40, rank=48, max_seq_len=131072), 128, 1024),
    # few (b, kv-head) pairs: split finer to keep >= 512 workgroups
    (dict(batch=1, num_q_heads=8, num_kv_heads=8, rank=64, max_seq_len=65536), 64, 1024),
])
def test_default_plan(kw, exp_P, exp_S):
    P, S = lr.plan(params(**kw))
    T = kw["max_seq_len"]
    assert (P, S) == (exp_P, exp_S)
    assert P * S >= T and (P - 1) * S < T


def test_plan_explicit_splits():
    for splits in (1, 2, 3, 256, 1000):
        P, S = lr.plan(params(num_splits=splits))
        assert P <= splits and P * S >= 1000 and (P - 1) * S < 1000


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), -2), (dict(num_q_heads=-1), -2), (dict(num_q_heads=7), -2),
    (dict(max_seq_len=0), -2), (dict(rank=0), -2),
    (dict(q_dtype=lr.I8), -3), (dict(latent_dtype=9), -3), (dict(factor_dtype=lr.I8), -3),
    (dict(out_dtype=lr.F16), -3),
    (dict(head_dim=96), -4), (dict(rank=24), -4), (dict(rank=128, latent_dtype=lr.F32), -4),
    (dict(num_q_heads=6, num_kv_heads=2), -4), (dict(num_q_heads=32, num_kv_heads=2), -4),
    (dict(batch=70000), -4),
    (dict(num_splits=-1), -7), (dict(num_splits=1001), -7),
    (dict(softmax_scale=float("nan")), -2),
])
def test_param_errors(kw, status):
    p = params(**kw)
    b = ctypes.c_size_t(12345)
    assert lr.lib().lrattn_workspace_size(ctypes.byref(p), ctypes.byref(b)) == status
    assert b.value == 12345  # untouched on error
    assert decode_status(p) == status


def test_pointer_errors():
    p = params()
    assert lr.lib().lrattn_workspace_size(None, None) == -1
    assert decode_status(p, q=None) == -1
    assert decode_status(p, lv=None) == -1
    assert decode_status(p, bv=None) == -1
    assert decode_status(p, seq=None) == -1
    assert decode_status(p, out=None) == -1
    assert decode_status(p, scales=ALIGNED) == -1                       # scales with bf16 latents
    assert decode_status(params(latent_dtype=lr.I8, rank=32)) == -1     # int8 without scales
    assert decode_status(p, q=MISALIGNED) == -5
    assert decode_status(p, bk=MISALIGNED) == -5
    assert decode_status(p, out=MISALIGNED) == -5
    assert decode_status(p, ws=MISALIGNED) == -5
    assert decode_status(params(latent_dtype=lr.I8, rank=32), scales=MISALIGNED) == -5
    assert decode_status(p, ws=None) == -6
    need = lr.workspace_size(p)
    assert decode_status(p, ws_bytes=need - 1) == -6


def test_partition_and_combine_validate_too():
    p = params()
    L = lr.lib()
    assert L.lrattn_partition(ctypes.byref(p), None, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED,
                              ALIGNED, 1 << 30, None) == -1
    assert L.lrattn_partition(ctypes.byref(p), ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED,
                              ALIGNED, 0, None) == -6
    assert L.lrattn_combine(ctypes.byref(p), ALIGNED, ALIGNED, None, ALIGNED, 1 << 30, None) == -1
    assert L.lrattn_combine(ctypes.byref(p), ALIGNED, ALIGNED, ALIGNED, ALIGNED, 0, None) == -6


def test_probe_validation():
    L = lr.lib()
    assert lr.probe_sink_floats() >= 1024
    assert L.lrattn_probe_read(None, 16, ALIGNED, None) == -1
    assert L.lrattn_probe_read(ALIGNED, 15, ALIGNED, None) == -2
    assert L.lrattn_probe_read(ALIGNED, 0, ALIGNED, None) == -2
    assert L.lrattn_probe_copy(ALIGNED, MISALIGNED, 32, None) == -5
    assert L.lrattn_probe_clock(None, None) == -1
    assert L.lrattn_probe_clock(MISALIGNED, None) == -5


def test_supported_matrix_plans():
    # every compiled (latent dtype, rank, group) combination is accepted
    for lt, esz in ((lr.F32, 4), (lr.BF16, 2), (lr.F16, 2), (lr.I8, 1)):
        for r in (16, 32, 48, 64, 128):
            for G in (1, 2, 4, 8):
                for d in (64, 128, 256):
                    p = params(latent_dtype=lt, rank=r, num_q_heads=2 * G, num_kv_heads=2,
                               head_dim=d)
                    b = ctypes.c_size_t()
                    st = lr.lib().lrattn_workspace_size(ctypes.byref(p), ctypes.byref(b))
                    assert st == (0 if r * esz <= 256 else -4), (lt, r, G, d)


def test_partition_kernel_names():
    # bf16 latents, r a multiple of 32, 4 or 8 heads per kv-head: matrix-core scores
    for r in (16, 32, 48, 64, 128):
        for G in (1, 2, 4, 8):
            p = params(rank=r, num_q_heads=2 * G, num_kv_heads=2)
            want = "partition_mfma_kernel" if r % 32 == 0 and G >= 4 else "partition_kernel"
            assert lr.partition_kernel(p) == want, (r, G)
    for lt in (lr.F32, lr.F16, lr.I8):
        assert lr.partition_kernel(params(latent_dtype=lt, rank=32)) == "partition_kernel"
    assert lr.lib().lrattn_partition_kernel(ctypes.byref(params(head_dim=96))) is None
    assert lr.lib().lrattn_partition_kernel(None) is None
    with pytest.raises(lr.LrattnError):
        lr.partition_kernel(params(rank=24))


def test_dense_decode_validates_on_host():
    L = lr.lib()
    p = params(rank=128)  # rank == head_dim
    def call(p, q=ALIGNED, k=ALIGNED, v=ALIGNED, sc=None, seq=ALIGNED, out=ALIGNED, ws=ALIGNED,
             ws_bytes=0):
        return L.lrattn_dense_decode(ctypes.byref(p), q, k, v, sc, seq, out, ws, ws_bytes, None)
    assert call(params(rank=64)) == -2          # rank must equal head_dim
    assert call(p, k=None) == -1
    assert call(p, out=None) == -1
    assert call(p, sc=ALIGNED) == -1            # scales with bf16 K/V
    assert call(params(rank=128, latent_dtype=lr.I8)) == -1
    assert call(p, v=MISALIGNED) == -5
    assert call(p, ws=None) == -6
    assert call(p, ws_bytes=lr.workspace_size(p) - 1) == -6
    assert call(params(rank=128, latent_dtype=lr.F32)) == -4   # 512-byte rows
    assert L.lrattn_dense_decode(None, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, ALIGNED, ALIGNED,
                                 1 << 30, None) == -1


def test_rebuild_decode_validates_on_host():
    L = lr.lib()
    def call(p, q=ALIGNED, lk=ALIGNED, lv=ALIGNED, bk=ALIGNED, bv=ALIGNED, rope=None,
             seq=ALIGNED, out=ALIGNED, ws=ALIGNED, ws_bytes=0):
        return L.lrattn_rebuild_decode(ctypes.byref(p), q, lk, lv, bk, bv, rope, seq, out, ws,
                                       ws_bytes, None)
    p = params()                                       # bf16, d 128, r 64, G 4
    assert call(params(rank=48)) == -4                 # r not in {32, 64}
    assert call(params(head_dim=256)) == -4
    assert call(params(latent_dtype=lr.F16)) == -4     # bf16 only
    assert call(params(q_dtype=lr.F32)) == -4
    assert call(params(factor_dtype=lr.F16)) == -4
    assert call(params(latent_dtype=lr.I8, rank=32)) == -4
    assert call(p, lk=None) == -1
    assert call(p, bv=None) == -1
    assert call(p, rope=MISALIGNED) == -5
    assert call(p, q=MISALIGNED) == -5
    assert call(p, ws=None) == -6
    assert call(p, rope=ALIGNED, ws_bytes=lr.rebuild_workspace_size(p) - 1) == -6
    assert call(params(max_seq_len=1 << 22), rope=ALIGNED) == -4   # T * d * 4 >= 2^31


def test_rebuild_plan():
    """One wave per sequence partition, four sequences per workgroup: the
    default plan gives about 512 workgroups of whole 32-token steps."""
    for kw, want in [(dict(batch=16, num_q_heads=32, num_kv_heads=8, rank=64, max_seq_len=16384),
                      (16, 1024)),                # 8 kv-heads x 4 quads x 16 partitions
                     (dict(batch=8, num_q_heads=32, num_kv_heads=32, rank=32, max_seq_len=4096),
                      (8, 512)),                  # 32 x 2 x 8
                     (dict(batch=5, num_q_heads=8, num_kv_heads=2, rank=64, max_seq_len=700),
                      (6, 128)),                  # floor of 128 tokens
                     (dict(batch=5, num_q_heads=8, num_kv_heads=2, rank=64, max_seq_len=700,
                           num_splits=3), (3, 234))]:   # explicit splits as given
        p = params(**kw)
        P, S = lr.rebuild_plan(p)
        assert (P, S) == want, (kw, P, S)
        rec = p.batch * p.num_q_heads * P * (p.rank + 4) * 4   # records, rounded to 256 bytes
        assert lr.rebuild_workspace_size(p) == (rec + 255) // 256 * 256
    with pytest.raises(lr.LrattnError):
        lr.rebuild_plan(params(latent_dtype=lr.I8, rank=32))


def test_append_validates_on_host():
    L = lr.lib()
    def ap(**kw):
        base = dict(batch=8, num_kv_heads=32, model_dim=4096, rank=32, max_seq_len=4096,
                    x_dtype=lr.BF16, factor_dtype=lr.BF16, latent_dtype=lr.BF16)
        base.update(kw)
        return lr.AppendParams(**base)
    def call(p, x=ALIGNED, ak=ALIGNED, av=ALIGNED, pos=ALIGNED, lk=ALIGNED, lv=ALIGNED, sc=None,
             ws=ALIGNED, ws_bytes=0):
        return L.lrattn_append(ctypes.byref(p), x, ak, av, pos, lk, lv, sc, ws, ws_bytes, None)
    assert L.lrattn_append(None, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None,
                           ALIGNED, 1 << 30, None) == -1
    need = lr.append_workspace_size(ap())
    assert 0 < need <= 4 << 20
    assert call(ap(), ws=None, ws_bytes=need) == -6
    assert call(ap(), ws=MISALIGNED, ws_bytes=need) == -5
    assert call(ap(), ws_bytes=need - 1) == -6
    assert call(ap(batch=0)) == -2
    assert call(ap(x_dtype=lr.F32, factor_dtype=lr.F32)) == -3
    assert call(ap(factor_dtype=lr.F16)) == -3
    assert call(ap(latent_dtype=7)) == -3
    assert call(ap(rank=24)) == -4
    assert call(ap(batch=65)) == -4
    assert call(ap(model_dim=4000)) == -4
    assert call(ap(), x=None) == -1
    assert call(ap(), sc=ALIGNED) == -1                    # scales with bf16 latents
    assert call(ap(latent_dtype=lr.I8)) == -1              # int8 without scales
    assert call(ap(), lv=MISALIGNED) == -5
    assert call(ap(latent_dtype=lr.I8), sc=MISALIGNED) == -5


def test_shared_decode_validates_on_host():
    L = lr.lib()
    def call(p, ws=ALIGNED, ws_bytes=0, **kw):
        a = dict(q=ALIGNED, lk=ALIGNED, lv=ALIGNED, bk=ALIGNED, bv=ALIGNED, sc=None, seq=ALIGNED,
                 out=ALIGNED)
        a.update(kw)
        return L.lrattn_shared_decode(ctypes.byref(p), a["q"], a["lk"], a["lv"], a["bk"], a["bv"],
                                      a["sc"], a["seq"], a["out"], ws, ws_bytes, None)
    one = params(num_q_heads=32, num_kv_heads=1)        # one stream shared by 32 heads
    need = lr.shared_workspace_size(one)
    P, _ = lr.plan(params(num_q_heads=32, num_kv_heads=4))   # grouped in 8s: 4 groups
    assert need >= 2 * 32 * P * 68 * 4 + 2 * 32 * 64 * 4
    assert call(params(num_q_heads=30, num_kv_heads=4)) == -2
    assert call(params(num_q_heads=12, num_kv_heads=1), ws_bytes=0) == -6   # group of 4s
    assert call(params(num_q_heads=6, num_kv_heads=2, rank=24)) == -4
    assert call(one, bk=None) == -1
    assert call(one, bv=MISALIGNED) == -5
    assert call(one, ws=None, ws_bytes=need) == -6
    assert call(one, ws_bytes=need - 1) == -6


def test_modal_decode_validates_on_host():
    L = lr.lib()
    def call(p, ni=576, q=ALIGNED, lk=ALIGNED, lv=ALIGNED, bk=ALIGNED, bv=ALIGNED, sc=None,
             seq=ALIGNED, out=ALIGNED, ws=ALIGNED, ws_bytes=0):
        return L.lrattn_modal_decode(ctypes.byref(p), ni, q, lk, lv, bk, bv, sc, seq, out, ws,
                                     ws_bytes, None)
    p = params()                                       # bf16, d 128, r 64, G 4, T 1000
    assert call(params(head_dim=256)) == -4            # d in {64, 128}
    assert call(params(rank=128)) == -4                # r <= 64
    assert call(p, ni=-1) == -2
    assert call(p, lk=None) == -1
    assert call(p, bv=None) == -1
    assert call(p, bk=MISALIGNED) == -5
    assert call(p, ws=None) == -6
    assert call(p, ws_bytes=lr.modal_workspace_size(p, 576) - 1) == -6


def test_modal_plan_records():
    """Image tokens and text are split apart, each in parts of at most the
    decode plan's S: the workspace holds P_img + P_txt records per head."""
    p = params(max_seq_len=1000)
    P, S = lr.plan(p)
    rec = lambda n: (p.batch * p.num_q_heads * n * (p.rank + 4) * 4 + 255) // 256 * 256
    for ni in (0, 1, 576, 999, 1000, 5000):
        nic = min(ni, 1000)
        want = -(-nic // S) + -(-(1000 - nic) // S)
        assert lr.modal_workspace_size(p, ni) == rec(want), ni


def test_adaptive_decode_validates_on_host():
    L = lr.lib()
    def call(p, ad=None, q=ALIGNED, lk=ALIGNED, lv=ALIGNED, bk=ALIGNED, bv=ALIGNED, sc=None,
             seq=ALIGNED, imp=ALIGNED, out=ALIGNED, ws=ALIGNED, ws_bytes=0):
        ad = ad or lr.AdaptiveParams(16, 0.5, 0.9)
        return L.lrattn_adaptive_decode(ctypes.byref(p), ctypes.byref(ad), q, lk, lv, bk, bv,
                                        sc, seq, imp, out, ws, ws_bytes, None)
    p = params()                                       # bf16, d 128, r 64, G 4
    assert call(params(latent_dtype=lr.F16)) == -4     # bf16, int8 (r 32), fp32 (r 16)
    assert call(params(rank=16)) == -4                 # bf16: r in {32, 48, 64, 128}
    assert call(params(rank=128, latent_dtype=lr.I8)) == -4
    assert call(p, ad=lr.AdaptiveParams(0, 0.5, 0.9)) == -2       # low_rank in [1, r]
    assert call(p, ad=lr.AdaptiveParams(65, 0.5, 0.9)) == -2
    assert call(p, ad=lr.AdaptiveParams(8, 0.5, 1.5)) == -2       # decay in [0, 1]
    assert call(p, ad=lr.AdaptiveParams(8, float("nan"), 0.5)) == -2
    assert call(p, imp=None) == -1
    assert call(p, imp=MISALIGNED) == -5
    assert call(p, ws=None) == -6
    ad = lr.AdaptiveParams(16, 0.5, 0.9)
    need = lr.adaptive_workspace_size(p, ad)
    assert call(p, ad=ad, ws_bytes=need - 1) == -6
    rec = lr.workspace_size(p)
    lg = (p.batch * p.num_q_heads * p.max_seq_len * 4 + 255) // 256 * 256
    assert need == rec + lg + 256          # records, logits [B, Hq, T], row statistics



def test_adaptive_kernel_names():
    ad = lr.AdaptiveParams(16, 0.5, 0.9)
    # bf16 latents with r a multiple of 32 and 4 or 8 heads: the matrix-core kernel
    for r in (32, 48, 64, 128):
        for G in (1, 2, 4, 8):
            p = params(rank=r, num_q_heads=2 * G, num_kv_heads=2)
            want = "partition_mfma_kernel" if r % 32 == 0 and G >= 4 else "partition_kernel"
            assert lr.adaptive_kernel(p, lr.AdaptiveParams(8, 0.5, 0.9)) == want, (r, G)
    assert lr.adaptive_kernel(params(latent_dtype=lr.I8, rank=32, num_q_heads=8,
                                     num_kv_heads=2), ad) == "partition_kernel"
    assert lr.lib().lrattn_adaptive_kernel(ctypes.byref(params(rank=16)), ctypes.byref(ad)) is None
    assert lr.lib().lrattn_adaptive_kernel(ctypes.byref(params()), None) is None
    with pytest.raises(lr.LrattnError):
        lr.adaptive_kernel(params(latent_dtype=lr.F16), ad)

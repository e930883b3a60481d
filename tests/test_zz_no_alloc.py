"""lrattn_decode_static (the decode for callers that cannot allocate: its
records live in the library's static per-device buffer) against
lrattn_decode on the same inputs, through the C-ABI: two calls in a row, the
second with a smaller input, each bitwise equal to lrattn_decode's output at
the same plan and within the oracle gate; and the host-side rejection of a
request whose records exceed the buffer."""
import numpy as np
import pytest

import workloads
from gpu_helpers import TOL, oracle_all_rows, rel_rowmax, say, to_device




def _pair(w, splits):
    import torch
    import rank_kv_cache_head_amd as lr
    dev = to_device(w)
    ref = lr.decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"],
                    dev["scales"], softmax_scale=w.softmax_scale, num_splits=splits)
    out = torch.full_like(ref, float("nan"))
    lr.decode_static(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"],
                     dev["scales"], out=out, softmax_scale=w.softmax_scale, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.gpu
def test_static_equals_decode_twice_second_smaller():
    # call 1: the ragged workload at full size and its 256 partitions per
    # head (8.5 MB of records, the largest of the five workloads)
    w1 = workloads.make("ragged")
    say("static decode: ragged full size, 256 splits")
    got1, ref1 = _pair(w1, workloads.SPLITS["ragged"])
    assert np.array_equal(got1, ref1)
    assert rel_rowmax(got1, oracle_all_rows(w1)) <= TOL[w1.latent_dtype]
    # call 2: a smaller input (fewer sequences, heads, tokens, other rank
    # and dtype) on the same buffer, which still holds call 1's records
    w2 = workloads.make("int8", B=3, Hq=8, Hkv=2, T=1500, seq_lens=[1500, 700, 1])
    say("static decode: smaller int8 input")
    got2, ref2 = _pair(w2, 5)
    assert np.array_equal(got2, ref2)
    assert rel_rowmax(got2, oracle_all_rows(w2)) <= TOL[w2.latent_dtype]


@pytest.mark.gpu
def test_static_rejects_records_beyond_the_buffer():
    import torch
    import rank_kv_cache_head_amd as lr
    # 4 x 64 x 4096 partitions x (32 + 4) floats: 151 MB of records
    big = dict(B=4, Hq=64, T=4096)
    q = torch.zeros((big["B"], big["Hq"], 128), dtype=torch.bfloat16, device="cuda")
    L = torch.zeros((big["B"], 64, big["T"], 32), dtype=torch.bfloat16, device="cuda")
    Bf = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.full((big["B"],), big["T"], dtype=torch.int32, device="cuda")
    out = torch.zeros((big["B"], big["Hq"], 128), device="cuda")
    p = lr.params_for(q, L, Bf, num_splits=big["T"])
    assert lr.workspace_size(p) > lr.STATIC_SCRATCH_BYTES
    say("static decode: oversized request")
    with pytest.raises(lr.LrattnError) as e:
        lr.decode_static(q, L, L, Bf, Bf, sl, out=out, num_splits=big["T"])
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert (out == 0).all()


def _cpu_params(**kw):
    import rank_kv_cache_head_amd as lr
    base = dict(batch=4, num_q_heads=40, num_kv_heads=40, head_dim=128, rank=48,
                max_seq_len=131072, q_dtype=lr.BF16, latent_dtype=lr.BF16,
                factor_dtype=lr.BF16, out_dtype=lr.F32, softmax_scale=0.0, num_splits=256)
    base.update(kw)
    return lr.Params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(num_splits=4096), -9),            # 4 x 40 x 4096 x 52 x 4 B of records
    (dict(rank=24), -4),
    (dict(num_q_heads=0), -2),
])
def test_static_rejects_on_host(kw, status):
    """Rejections that need no device: the parameter block and the buffer
    limit are checked before anything touches the GPU (fake pointers)."""
    import ctypes
    import rank_kv_cache_head_amd as lr
    p = _cpu_params(**kw)
    A = 0x10000
    st = lr.lib().lrattn_decode_static(ctypes.byref(p), A, A, A, A, A, None, A, A, None)
    assert st == status


def test_static_pointer_errors_on_host():
    import ctypes
    import rank_kv_cache_head_amd as lr
    p = _cpu_params()
    A, M = 0x10000, 0x10004
    L = lr.lib()
    assert L.lrattn_decode_static(ctypes.byref(p), None, A, A, A, A, None, A, A, None) == -1
    assert L.lrattn_decode_static(ctypes.byref(p), A, M, A, A, A, None, A, A, None) == -5
    assert L.lrattn_decode_static(ctypes.byref(p), A, A, A, A, A, A, A, A, None) == -1  # scales
    assert L.lrattn_decode_static(None, A, A, A, A, A, None, A, A, None) == -1

"""The GPU tests' per-(sequence, kv-head) oracle driver must return exactly
the oracle's own whole-batch decode: same rows, same head map, same int8
scales, same lengths (CPU only)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import f64_args, oracle_all_rows


@pytest.mark.parametrize("name,kw", [
    ("gqa_vlm", dict(B=3, Hq=8, Hkv=2, T=300, seq_lens=[300, 77, 1])),
    ("int8", dict(B=2, Hq=4, Hkv=4, T=200, seq_lens=[200, 31])),
    ("ragged", dict(B=3, Hq=2, Hkv=2, T=2000, len_lo=1024, len_hi=2000)),
    ("tiny", dict()),
])
def test_all_rows_equals_whole_decode(name, kw):
    w = workloads.make(name, **kw)
    args = f64_args(w)
    ref = oracle.decode(*args[:6], scales=args[6], softmax_scale=w.softmax_scale)
    got = oracle_all_rows(w)
    assert got.shape == ref.shape
    assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()

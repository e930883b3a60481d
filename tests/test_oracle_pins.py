"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.decode)


def test_decode_rows_matches_decode():
    import workloads
    w = workloads.make("ragged", seed=2, B=3, Hq=4, Hkv=4, d=16, r=8, T=40, len_lo=5)
    args = P._f64(w)
    full = oracle.decode(*args[:6], scales=args[6])
    rows = [(2, 3), (0, 0), (1, 2)]
    part = oracle.decode_rows(*args[:6], rows=rows, scales=args[6])
    for i, (b, h) in enumerate(rows):
        assert np.array_equal(part[i], full[b, h])


def test_zero_length_raises():
    import workloads
    w = workloads.make("tiny", seed=1, B=2, T=4, seq_lens=[4, 0])
    args = P._f64(w)
    with pytest.raises(ValueError):
        oracle.decode(*args[:6])


def test_bf16_decode_exact():
    # bf16 bit patterns decode to the binary32 with those high bits
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3EAB, 0x7F7F], dtype=np.uint16)
    vals = oracle.as_float64(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 0.0
    assert vals[3] == 0.333984375        # 0x3EAB = 1.0101011b x 2^-2
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127


def test_brute_force_on_the_tiny_workload_itself():
    """The tiny workload at its own size and seed (1 sequence, 4 heads, d 64,
    r 16, 256 tokens, fp32) through the 40-digit decimal definition: the
    oracle agrees to 1e-13 per row (about 8 s of decimal arithmetic, so it
    runs here once rather than inside every planted-mistake check)."""
    import workloads
    w = workloads.make("tiny")
    assert (w.batch, w.num_q_heads, w.head_dim, w.rank, w.max_seq_len) == (1, 4, 64, 16, 256)
    P.pin_brute(oracle.decode, cases=[("tiny", dict(seed=1))], tol=1e-13)

"""Pins for the append-step oracle (CPU only): hand-worked projection and
quantization cases, and invariants of the quantizer."""
import numpy as np

from oracle import append_step as ap


def test_projection_hand_worked():
    # x = (1, 2, 3); head 0 rows (1,0,0), (0,1,-1); head 1 row sums
    x = np.array([[1.0, 2.0, 3.0]])
    A = np.array([[[1.0, 0.0, 0.0], [0.0, 1.0, -1.0]],
                  [[1.0, 1.0, 1.0], [2.0, 0.0, 0.5]]])
    got = ap.project(x, A)
    assert got.shape == (1, 2, 2)
    assert np.array_equal(got[0], [[1.0, -1.0], [6.0, 3.5]])


def test_projection_per_sequence_and_head():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 8))
    A = rng.standard_normal((2, 4, 8))
    got = ap.project(x, A)
    for b in range(3):
        for g in range(2):
            for j in range(4):
                assert abs(got[b, g, j] - sum(x[b, k] * A[g, j, k] for k in range(8))) < 1e-12


def test_quantize_hand_worked_half_even():
    # s = 2/127; row / s = (63.5, -127, 31.75): 63.5 rounds to the even 64
    codes, s = ap.quantize_rows(np.array([1.0, -2.0, 0.5]))
    assert s == 2.0 / 127.0
    assert np.array_equal(codes, [64.0, -127.0, 32.0])
    # scale exactly 1: ties at even integers round down in magnitude
    # (half-even), which rounding half away from zero would not
    codes, s = ap.quantize_rows(np.array([[62.5, 127.0, -62.5, 0.5, 1.5, -2.5]]))
    assert s[0] == 1.0
    assert np.array_equal(codes[0], [62.0, 127.0, -62.0, 0.0, 2.0, -2.0])


def test_quantize_zero_row_and_invariants():
    codes, s = ap.quantize_rows(np.zeros((2, 5)))
    assert np.array_equal(s, [0.0, 0.0]) and not codes.any()
    rng = np.random.default_rng(1)
    L = rng.standard_normal((50, 32)) * rng.uniform(0.01, 10, (50, 1))
    codes, s = ap.quantize_rows(L)
    assert np.abs(codes).max() == 127 and (np.abs(codes).max(axis=1) == 127).all()
    assert np.abs(codes * s[:, None] - L).max(axis=1).max() <= 0.5 * s.max() * (1 + 1e-12)
    assert (np.abs(codes * s[:, None] - L) <= 0.5 * s[:, None] * (1 + 1e-12)).all()


def test_append_positions_and_layout():
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    AK = np.array([[[1.0, 0.0]], [[0.0, 2.0]]])     # Hkv 2, r 1, D 2
    AV = -AK
    rows, sc, written = ap.append(x, AK, AV, np.array([3, 7]), T=5, quantized=False)
    assert sc is None and list(written) == [True, False]
    assert np.array_equal(rows[0], [[[1.0], [0.0]], [[0.0], [2.0]]])
    assert np.array_equal(rows[1], -rows[0])
    codes, sc, _ = ap.append(x, AK, AV, np.array([0, 1]), T=5, quantized=True)
    assert np.array_equal(codes[0, 0, 0], [127.0]) and sc[0, 0, 0] == 1.0 / 127.0
    assert codes[0, 0, 1, 0] == 0.0 and sc[0, 0, 1] == 0.0

"""Seeded synthetic workloads: determinism, shapes, dtypes and distributions (CPU)."""
import numpy as np
import pytest

import oracle
import workloads as W


def test_deterministic_and_thread_independent():
    a = W.make("gqa_vlm", B=2, Hq=8, Hkv=2, T=700, threads=1)
    b = W.make("gqa_vlm", B=2, Hq=8, Hkv=2, T=700, threads=4)
    assert W.fingerprint(a) == W.fingerprint(b)
    c = W.make("gqa_vlm", seed=4, B=2, Hq=8, Hkv=2, T=700)
    assert W.fingerprint(a)["L_K"] != W.fingerprint(c)["L_K"]


def test_block_streams_are_independent_of_batch():
    # one stream per (b, kv-head) block: adding sequences leaves earlier blocks alone
    a = W.make("llm7b", B=1, Hq=2, Hkv=2, T=64)
    b = W.make("llm7b", B=3, Hq=2, Hkv=2, T=64)
    assert np.array_equal(a.L_K[0], b.L_K[0]) and np.array_equal(a.L_V[0], b.L_V[0])
    assert not np.array_equal(b.L_K[0], b.L_K[1])


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_shapes_and_dtypes(name):
    spec = W.SPECS[name]
    small = dict(B=min(spec["B"], 2), T=min(spec["T"], 2048))
    if name == "ragged":
        small.update(len_lo=100, len_hi=2048)
    w = W.make(name, **small)
    B, Hq, Hkv, d, r, T = (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rank, w.max_seq_len)
    assert w.q.shape == (B, Hq, d) and w.q.dtype == W.storage_dtype(w.q_dtype)
    assert w.L_K.shape == (B, Hkv, T, r) and w.L_K.dtype == W.storage_dtype(w.latent_dtype)
    assert w.B_K.shape == (Hkv, r, d) and w.B_V.dtype == W.storage_dtype(w.factor_dtype)
    assert w.seq_lens.dtype == np.int32 and w.seq_lens.shape == (B,)
    assert (w.seq_lens >= 1).all() and (w.seq_lens <= T).all()
    if w.latent_dtype == "i8":
        assert w.scales.shape == (2, B, Hkv, T) and w.scales.dtype == np.float32
    else:
        assert w.scales is None


def test_full_size_specs():
    s = W.SPECS
    assert (s["tiny"]["B"], s["tiny"]["Hq"], s["tiny"]["d"], s["tiny"]["r"], s["tiny"]["T"]) == (1, 4, 64, 16, 256)
    assert (s["llm7b"]["B"], s["llm7b"]["Hq"], s["llm7b"]["d"], s["llm7b"]["r"], s["llm7b"]["T"]) == (8, 32, 128, 32, 4096)
    g = s["gqa_vlm"]
    assert (g["B"], g["Hq"], g["Hkv"], g["d"], g["r"], g["T"], g["image_tokens"]) == (16, 32, 8, 128, 64, 16384, 576)
    i = s["int8"]
    assert (i["B"], i["Hq"], i["d"], i["r"], i["T"], i["latent_dtype"]) == (32, 32, 128, 32, 8192, "i8")
    r = s["ragged"]
    assert (r["B"], r["Hq"], r["d"], r["r"], r["T"], r["len_lo"], r["len_hi"]) == (4, 40, 128, 48, 131072, 1024, 131072)


def test_distributions():
    w = W.make("gqa_vlm", B=2, Hq=4, Hkv=1, T=4096)
    L = oracle.as_float64(w.L_K, "bf16")
    img, txt = L[:, :, :576], L[:, :, 576:]
    assert abs(img.std() - 2.0) < 0.05 and abs(txt.std() - 1.0) < 0.02
    f = oracle.as_float64(w.B_K, "bf16")
    assert abs(f.std() - 1 / 8) < 0.01
    w = W.make("int8", B=2, Hq=2, Hkv=2, T=4096)
    assert w.L_K.min() >= -127 and w.L_K.max() <= 127
    assert w.L_K.min() == -127 and w.L_K.max() == 127
    assert (w.scales >= 0.005).all() and (w.scales <= 0.02).all()
    w = W.make("ragged", B=64, Hq=1, Hkv=1, d=8, r=8, T=4096, len_lo=1024, len_hi=4096)
    assert w.seq_lens.min() >= 1024 and w.seq_lens.max() <= 4096
    assert w.seq_lens.std() > 400   # spread over the range, not constant


def test_padding_modes():
    w = W.make("ragged", B=2, Hq=1, Hkv=1, d=8, r=8, T=64, seq_lens=[10, 64], pad="nan")
    L = oracle.as_float64(w.L_K, "bf16")
    assert np.isnan(L[0, 0, 10:]).all() and np.isfinite(L[0, 0, :10]).all()
    assert np.isfinite(L[1]).all()
    w = W.make("int8", B=2, Hq=1, Hkv=1, d=8, r=8, T=64, seq_lens=[10, 64], pad="nan")
    assert np.isnan(w.scales[:, 0, 0, 10:]).all() and (w.L_K[0, 0, 10:] == 0).all()
    w = W.make("ragged", B=1, Hq=1, Hkv=1, d=8, r=8, T=64, seq_lens=[10])
    assert (w.L_K[0, 0, 10:] == 0).all()


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -0.0,
                  np.inf, np.nan], dtype=np.float32)
    bits = W.bf16_bits_from_f32(x)
    # ties go to even: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6 ; above the tie rounds up
    assert list(bits[:4]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81]
    assert bits[4] == 0x8000 and bits[5] == 0x7F80 and bits[6] == 0x7FC0


def test_algorithmic_bytes():
    w = W.make("gqa_vlm", B=2, Hq=8, Hkv=2, T=100)
    ab = w.algorithmic_bytes()
    assert ab["latents"] == 2 * 2 * 2 * 100 * 64 * 2
    w = W.make("int8", B=2, Hq=2, Hkv=2, T=50, seq_lens=[50, 10])
    ab = w.algorithmic_bytes()
    assert ab["latents"] == 2 * 60 * 2 * 32 and ab["scales"] == 2 * 60 * 2 * 4

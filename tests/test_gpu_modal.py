"""GPU parity of the decode with separate image and text factors
(AttentionPack page, section 2.A: the modalities are compressed apart)
against the fp64 oracle's decode_modal, through the C-ABI.

Gate as for lrattn_decode: max over output rows of
||gpu - oracle||_inf / ||oracle||_inf <= 2e-3 for bf16/fp16/int8 inputs and
<= 1e-5 for fp32 inputs.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import TOL, rel_rowmax, say, tensor, to_device

pytestmark = pytest.mark.gpu


def _sets(w, seed):
    """Two factor sets: the workload's own (image) and a second draw (text),
    stacked [2, Hkv, r, d], as stored and as float64."""
    w2 = workloads.make(w.name, seed=seed, B=w.batch, Hq=w.num_q_heads, Hkv=w.num_kv_heads,
                        d=w.head_dim, r=w.rank, T=16, seq_lens=[16] * w.batch,
                        q_dtype=w.q_dtype, latent_dtype=w.latent_dtype,
                        factor_dtype=w.factor_dtype)
    assert w2.B_K.dtype == w.B_K.dtype
    BK = np.stack([w.B_K, w2.B_K])
    BV = np.stack([w.B_V, w2.B_V])
    f = oracle.as_float64
    return BK, BV, f(BK, w.factor_dtype), f(BV, w.factor_dtype)


def _run(w, dev, BK, BV, ni, **kw):
    import torch
    import rank_kv_cache_head_amd as lr
    out = lr.modal_decode(dev["q"], dev["L_K"], dev["L_V"], tensor(BK, w.factor_dtype),
                          tensor(BV, w.factor_dtype), dev["seq_lens"], ni, dev["scales"],
                          softmax_scale=w.softmax_scale, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref(w, BK64, BV64, ni):
    f = oracle.as_float64
    sc = None if w.scales is None else w.scales.astype(np.float64)
    return oracle.decode_modal(f(w.q, w.q_dtype), f(w.L_K, w.latent_dtype),
                               f(w.L_V, w.latent_dtype), BK64, BV64, w.seq_lens, ni,
                               scales=sc, softmax_scale=w.softmax_scale)


CASES = {
    # name: (workload, overrides) -- several partitions per modality, lengths
    # shorter than the image block, a one-token sequence
    "gqa_bf16": ("gqa_vlm", dict(B=4, Hq=8, Hkv=2, T=1500, seq_lens=[1500, 700, 90, 1])),
    "mha_bf16_r32": ("llm7b", dict(B=3, Hq=4, Hkv=4, T=1200, seq_lens=[1200, 333, 17])),
    "int8": ("int8", dict(B=3, Hq=4, Hkv=4, T=1300, seq_lens=[1300, 640, 5])),
    "g8_d64": ("gqa_vlm", dict(B=2, Hq=16, Hkv=2, d=64, r=32, T=900, seq_lens=[900, 301])),
    "fp32": ("tiny", dict(B=2, T=256, seq_lens=[256, 100])),
    "f16_r48": ("gqa_vlm", dict(B=2, Hq=4, Hkv=4, r=48, T=1000, seq_lens=[1000, 555],
                                q_dtype="f16", latent_dtype="f16", factor_dtype="f16")),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_modal_decode_matches_oracle(case):
    base, kw = CASES[case]
    w = workloads.make(base, **kw)
    dev = to_device(w)
    BK, BV, BK64, BV64 = _sets(w, seed=900)
    T = w.max_seq_len
    for ni in (0, 1, 96, 576, T):
        ref = _ref(w, BK64, BV64, ni)
        for splits in (0, 1, 3, 7):
            say(f"modal {case} image_tokens={ni} splits={splits}")
            got = _run(w, dev, BK, BV, ni, num_splits=splits)
            err = rel_rowmax(got, ref)
            assert err <= TOL[w.latent_dtype], (ni, splits, err)


def test_modal_equal_sets_equals_decode():
    """With the same set twice the result is ordinary decode (to fp32
    accuracy: the image block is folded in partitions of its own)."""
    import torch
    import rank_kv_cache_head_amd as lr
    w = workloads.make("gqa_vlm", B=2, Hq=8, Hkv=2, T=1000, seq_lens=[1000, 400])
    dev = to_device(w)
    BK = np.stack([w.B_K, w.B_K])
    BV = np.stack([w.B_V, w.B_V])
    say("modal equal sets")
    got = _run(w, dev, BK, BV, 576)
    ref = lr.decode(dev["q"], dev["L_K"], dev["L_V"], dev["B_K"], dev["B_V"], dev["seq_lens"],
                    softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    assert rel_rowmax(got, ref.cpu().numpy().astype(np.float64)) <= 2e-5


def test_modal_nan_padding_and_determinism():
    kw = dict(B=3, Hq=8, Hkv=2, T=1024, seq_lens=[1024, 600, 33])
    wz = workloads.make("gqa_vlm", pad="zero", **kw)
    wn = workloads.make("gqa_vlm", pad="nan", **kw)
    BK, BV, _, _ = _sets(wz, seed=901)
    say("modal NaN padding / determinism")
    outs = [_run(w, to_device(w), BK, BV, 576) for w in (wz, wn, wz)]
    assert np.isfinite(outs[1]).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_modal_full_size_gqa_vlm():
    """gqa_vlm at full size, its 576-token image block with factors of its
    own, default plan; every sequence checked against the oracle (one at a
    time in float64)."""
    w = workloads.make("gqa_vlm")
    say("modal full gqa_vlm: inputs")
    dev = to_device(w)
    BK, BV, BK64, BV64 = _sets(w, seed=902)
    say("modal full gqa_vlm: decode")
    got = _run(w, dev, BK, BV, 576)
    assert np.isfinite(got).all()
    f = oracle.as_float64
    err = 0.0
    for b in range(w.batch):
        sel = [b]
        ref = oracle.decode_modal(f(w.q[sel], w.q_dtype), f(w.L_K[sel], w.latent_dtype),
                                  f(w.L_V[sel], w.latent_dtype), BK64, BV64, w.seq_lens[sel], 576)
        err = max(err, rel_rowmax(got[sel], ref))
    say(f"  err {err:.3e}")
    assert err <= TOL[w.latent_dtype], err

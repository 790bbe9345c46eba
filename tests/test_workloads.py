"""CPU checks of the shared input module (seeded generators, bf16 rounding,
workload accounting).  It feeds both the oracle and the GPU path, so its
rounding is pinned against torch's own float32 -> bfloat16 conversion and its
pair counts against closed forms.
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import workloads  # noqa: E402
from workloads import WORKLOADS, bf16_bits, bf16_round, gen_block, gen_small  # noqa: E402


def _torch_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_bf16_round_matches_torch_including_ties_and_extremes():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        # exact ties: low 16 bits 0x8000, with even and odd kept bit
        (np.arange(1, 2001, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-40, np.inf, -np.inf], dtype=np.float32),
    ])
    np.testing.assert_array_equal(bf16_round(x).view(np.uint32), _torch_bf16(x).view(np.uint32))


def test_bf16_bits_are_the_upper_half():
    x = bf16_round(np.random.default_rng(6).standard_normal(4096).astype(np.float32))
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits(x), t)


def test_gen_block_is_deterministic_bf16_exact_and_standard_normal():
    a = gen_block(3, "k", 5, 4096, 4, 64, "bf16")
    b = gen_block(3, "k", 5, 4096, 4, 64, "bf16")
    assert a.shape == (4096, 4, 64) and a.dtype == np.float32
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, bf16_round(a))  # already representable in bf16
    # N(0, 1): 1M samples put the mean within 5e-3 and the std within 5e-3 of 1
    assert abs(float(a.mean())) < 5e-3
    assert abs(float(a.std()) - 1.0) < 5e-3


def test_each_block_has_its_own_stream():
    base = gen_block(3, "q", 2, 256, 2, 32, "f32")
    for other in (gen_block(3, "q", 3, 256, 2, 32, "f32"),    # another block
                  gen_block(3, "k", 2, 256, 2, 32, "f32"),    # another tensor
                  gen_block(4, "q", 2, 256, 2, 32, "f32")):   # another seed
        assert not np.array_equal(base, other)
        # independent streams: no visible correlation between the two draws
        assert abs(float(np.corrcoef(base.ravel(), other.ravel())[0, 1])) < 0.03
    # a block drawn on its own equals the same block drawn among the others
    blocks = [gen_block(3, "q", j, 256, 2, 32, "f32") for j in range(4)]
    np.testing.assert_array_equal(blocks[2], base)


def test_gen_small_scale_and_streams():
    a = gen_small(9, (512, 2, 32), "f32", 2.0, 0)
    assert abs(float(a.std()) - 2.0) < 0.05
    assert not np.array_equal(a, gen_small(9, (512, 2, 32), "f32", 2.0, 1))
    b = gen_small(9, (512, 2, 32), "bf16", 1.0, 0)
    np.testing.assert_array_equal(b, bf16_round(b))


def test_visible_pairs_closed_forms():
    for w in WORKLOADS.values():
        if w.is_decode:
            assert w.visible_pairs(0) == w.q_len * w.seq_len
            continue
        c, D, S = w.block_len, w.n_blocks, w.seq_len
        total = sum(w.visible_pairs(r) for r in range(D))
        if w.causal:
            assert total == S * (S + 1) // 2  # every (query, key) pair with key <= query
        else:
            assert total == S * S
        assert w.visible_pairs(0) == (c * (c + 1) // 2 if w.causal else c * S)


def test_flop_accounting():
    w = WORKLOADS["causal_128k_h32_d128"]
    S = w.seq_len
    assert w.fwd_flop() == 4.0 * w.head_dim * w.heads * S * (S + 1) // 2
    assert w.bwd_flop() == 2.5 * w.fwd_flop()
    f = workloads.FFN_WORKLOADS["ffn_block8192_h4096_f16384"]
    assert f.flop() == 4.0 * f.rows * f.hidden * f.ffn  # two GEMMs of 2*m*n*k

"""GPU parity: backward ring step against the fp64 analytic oracle (small shapes).

Every rank runs forward then backward; dK/dV of each block accumulate over the
ranks, so after the last rank they are the full-sequence gradients, compared
with the oracle's dense backward (itself pinned by finite differences).
"""
import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra
import oracle
from tests.gpu_util import compare, dev, log, require_gpu
from workloads import gen_small

pytestmark = pytest.mark.gpu

# (dtype, head_dim, heads, kv_heads, block_len, n_blocks, causal)
CASES = [
    ("f32", 64, 2, 2, 128, 2, True),
    ("f32", 128, 2, 1, 70, 3, False),
    ("bf16", 128, 2, 2, 256, 4, True),
    ("bf16", 64, 4, 4, 200, 3, False),    # ragged
    ("bf16", 128, 8, 2, 160, 3, True),    # GQA 4, ragged
    ("bf16", 128, 3, 1, 96, 2, True),     # group 3
    ("bf16", 64, 2, 2, 1, 2, True),       # one token per block
    ("bf16", 64, 4, 2, 96, 3, True),      # head_dim 64, grouped heads; dQ tiles straddle the block end
    ("bf16", 128, 16, 1, 96, 2, False),   # group 16: more query heads per K/V head than waves
    ("bf16", 128, 2, 2, 300, 2, True),    # several tiles: diagonal band and ragged tail in one block
    # Large gradients.  Under the causal mask key 0 collects weight from every row of every
    # head of its group, so |dV| grows with the group and the sequence.  The error of the
    # bf16 path is the rounding of P and dS to the matrix-core operand type, relative to
    # the gradient; with bf16 operands these shapes exceed the 1e-2 bound (an fp64
    # emulation of bf16 rounding puts them at 1.1e-2 to 2.1e-2), with the half operands
    # the kernels use they sit near 1e-3 to 3e-3.
    ("bf16", 64, 4, 1, 96, 3, True),      # head_dim 64, GQA 4, 288 tokens: |dV| 8.2
    ("bf16", 128, 4, 1, 200, 3, True),    # GQA 4, 600 tokens
    ("bf16", 128, 8, 1, 200, 3, True),    # GQA 8, 600 tokens: |dV| 15
    ("bf16", 128, 16, 1, 256, 2, True),   # GQA 16, 512 tokens: |dV| 26
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_all_ranks_vs_oracle(case):
    require_gpu()
    dtype, d, hq, hkv, c, D, causal = case
    log(f"bwd case {case}")
    S = c * D
    q = gen_small(61, (S, hq, d), dtype, 1.0, 0)
    k = gen_small(61, (S, hkv, d), dtype, 1.0, 1)
    v = gen_small(61, (S, hkv, d), dtype, 1.0, 2)
    do = gen_small(61, (S, hq, d), dtype, 1.0, 3)
    dq_ref, dk_ref, dv_ref, _, _ = oracle.attention_bwd(q, k, v, do, causal=causal)

    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    dkb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    dvb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    dqs = []
    for r in range(D):
        qd = dev(q[r * c:(r + 1) * c], dtype)
        dod = dev(do[r * c:(r + 1) * c], dtype)
        o, l = ra.fwd(qd, kb, vb, causal=causal, rank=r)
        dq, _, _ = ra.bwd(qd, kb, vb, o, dod, l, causal=causal, rank=r, dk_blocks=dkb, dv_blocks=dvb)
        dqs.append(dq)
    torch.cuda.synchronize()
    compare("dq", torch.cat(dqs, 0), dq_ref, dtype)
    compare("dk", torch.cat(dkb, 0), dk_ref, dtype)
    compare("dv", torch.cat(dvb, 0), dv_ref, dtype)


def test_bwd_pipeline_ordering_is_deterministic():
    """Backward with poisoned staging and a slowed copy stream is bit-identical."""
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 2, 256, 5
    S = c * D
    q = gen_small(67, (c, h, d), dtype, 1.0, 0)
    k = gen_small(67, (S, h, d), dtype, 1.0, 1)
    v = gen_small(67, (S, h, d), dtype, 1.0, 2)
    do = gen_small(67, (c, h, d), dtype, 1.0, 3)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd, dod = dev(q, dtype), dev(do, dtype)
    o, l = ra.fwd(qd, kb, vb, causal=False, rank=2)
    res = []
    for poison, delay in ((False, 0), (True, 150000)):
        ra.ring_attn_debug(poison, delay)
        try:
            dq, dkb, dvb = ra.bwd(qd, kb, vb, o, dod, l, causal=False, rank=2)
            torch.cuda.synchronize()
        finally:
            ra.ring_attn_debug(False, 0)
        res.append((dq, dkb, dvb))
    assert torch.equal(res[0][0], res[1][0])
    for j in range(D):
        assert torch.equal(res[0][1][j], res[1][1][j]) and torch.equal(res[0][2][j], res[1][2][j])


def test_bwd_rejects_small_caller_workspace_before_enqueueing():
    require_gpu()
    d, h, c, D = 128, 2, 256, 3
    x = [dev(gen_small(61, (c, h, d), "bf16", 1.0, i), "bf16") for i in range(2 + 2 * D)]
    q, do = x[0], x[1]
    kb, vb = x[2:2 + D], x[2 + D:]
    o, l = ra.fwd(q, kb, vb, causal=False, rank=1)
    small = torch.empty((1024,), dtype=torch.float32, device="cuda")
    dq = torch.full((c, h, d), 7.0, device="cuda")
    dkb = [torch.zeros((c, h, d), device="cuda") for _ in range(D)]
    dvb = [torch.zeros((c, h, d), device="cuda") for _ in range(D)]
    try:
        ra.ring_attn_set_workspace(small, 4096)
        with pytest.raises(ra.RingAttnError, match="workspace"):
            ra.bwd(q, kb, vb, o, do, l, causal=False, rank=1, dq=dq, dk_blocks=dkb, dv_blocks=dvb)
        torch.cuda.synchronize()
    finally:
        ra.ring_attn_set_workspace(None, 0)
    assert bool((dq == 7.0).all())
    assert all(bool((t == 0).all()) for t in dkb + dvb)

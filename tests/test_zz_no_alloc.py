"""GPU: the decode entry point that allocates nothing (ring_attn_decode_noalloc).

Through the C ABI, the no-allocation variant must give what ring_attn_decode
gives -- bit for bit, since it runs the same kernels on the same partial
layout, only in the library's fixed device scratch -- and match the fp64
oracle.  Two calls in a row, the second smaller, show that the shared scratch
keeps no state a later call depends on.  A shape whose partials exceed the
scratch is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra
import oracle
from tests.gpu_util import compare, dev, log, require_gpu
from workloads import bf16_round, gen_small

pytestmark = pytest.mark.gpu


def _run(seed, d, hq, hkv, c, D, q_len, q_pos0):
    log(f"noalloc decode case d={d} hq={hq} hkv={hkv} c={c} D={D} q_len={q_len} q_pos0={q_pos0}")
    q = bf16_round(gen_small(seed, (q_len, hq, d), "f32", 1.0, 0))
    k = [bf16_round(gen_small(seed, (c, hkv, d), "f32", 1.0, 10 + j)) for j in range(D)]
    v = [bf16_round(gen_small(seed, (c, hkv, d), "f32", 1.0, 40 + j)) for j in range(D)]
    qd, kb, vb = dev(q, "bf16"), [dev(x, "bf16") for x in k], [dev(x, "bf16") for x in v]
    o_ref, l_ref = ra.decode(qd, kb, vb, q_pos0=q_pos0)
    out = torch.full((q_len, hq, d), float("nan"), device="cuda")
    lse = torch.full((hq, q_len), float("nan"), device="cuda")
    torch.cuda.synchronize()
    rc = ra.ring_attn_decode_noalloc(qd, kb, vb, D, c, q_len, hq, hkv, d, q_pos0, out, lse)
    assert rc == ra.RA_OK, ra.last_error()
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), "differs from ring_attn_decode"
    o64, l64 = oracle.decode_forward(q.astype(np.float64), [x.astype(np.float64) for x in k],
                                     [x.astype(np.float64) for x in v], q_pos0)
    compare("out", out, o64, "bf16")
    compare("lse", lse, l64, "bf16")


def test_noalloc_decode_matches_decode_on_two_calls_second_smaller():
    require_gpu()
    # GQA 4 x 20 rows (passes of 8, 8, 4 rows), causal cut inside block 2; then a smaller call
    _run(91, 128, 32, 8, 700, 4, 20, 2500)
    _run(92, 64, 4, 2, 300, 2, 3, 600)


def test_noalloc_decode_refuses_partials_beyond_its_scratch():
    require_gpu()
    # 32 K/V heads x 8 blocks of 65536 keys, 32 rows per head: the partials need more than
    # the fixed scratch (chunks of 8192 keys -> 2048 partials per row set, 33.8 MB)
    d, hq, hkv, c, D, q_len = 128, 32, 32, 65536, 8, 32
    kb = [torch.empty((c, hkv, d), dtype=torch.bfloat16, device="cuda") for _ in range(D)]
    q = torch.zeros((q_len, hq, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((q_len, hq, d), 7.0, device="cuda")
    lse = torch.full((hq, q_len), 7.0, device="cuda")
    rc = ra.ring_attn_decode_noalloc(q, kb, kb, D, c, q_len, hq, hkv, d, D * c, out, lse)
    assert rc == ra.RA_ERR_INVALID_ARG
    assert "scratch" in ra.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())

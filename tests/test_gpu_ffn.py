"""GPU parity: blockwise feedforward (two MFMA GEMMs per row block) vs the fp64 oracle.

Shapes cover ragged row counts, blocks that do not divide the rows, one row,
an intermediate width that is an odd multiple of the tile, and the bias-free
form; chunking is checked to leave every output bit unchanged; the full-size
case is one rank's 8192-token block at h = 4096, checked on sampled rows.
"""
import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra
import oracle
from tests.gpu_util import compare, dev, log, require_gpu
from workloads import FFN_WORKLOADS, gen_ffn, gen_small

pytestmark = pytest.mark.gpu

# (rows, hidden, ffn, chunk_rows, biases)
CASES = [
    (100, 128, 256, 0, True),
    (300, 256, 512, 128, True),    # three blocks, the last one ragged
    (1, 128, 128, 0, True),
    (513, 128, 384, 200, False),   # ffn = 3 tiles, no biases
    (2048, 512, 2048, 1000, True),
]


def _inputs(seed, rows, hidden, ffn, biases):
    x = gen_small(seed, (rows, hidden), "bf16", 1.0, 0)
    w1 = gen_small(seed, (ffn, hidden), "bf16", 1.0 / np.sqrt(hidden), 1)
    w2 = gen_small(seed, (hidden, ffn), "bf16", 1.0 / np.sqrt(ffn), 2)
    b1 = gen_small(seed, (ffn,), "f32", 0.1, 3) if biases else None
    b2 = gen_small(seed, (hidden,), "f32", 0.1, 4) if biases else None
    return x, w1, b1, w2, b2


def _run(x, w1, b1, w2, b2, chunk):
    f = lambda t: None if t is None else torch.from_numpy(t).cuda()
    return ra.ffn_blockwise(dev(x, "bf16"), dev(w1, "bf16"), dev(w2, "bf16"), b1=f(b1), b2=f(b2), chunk_rows=chunk)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_ffn_vs_oracle(case):
    require_gpu()
    rows, hidden, ffn, chunk, biases = case
    log(f"ffn case {case}")
    x, w1, b1, w2, b2 = _inputs(97, rows, hidden, ffn, biases)
    y = _run(x, w1, b1, w2, b2, chunk)
    torch.cuda.synchronize()
    compare("y", y, oracle.ffn_forward(x, w1, b1, w2, b2), "bf16")


def test_chunking_leaves_outputs_bit_identical():
    require_gpu()
    x, w1, b1, w2, b2 = _inputs(101, 700, 256, 512, True)
    ys = [_run(x, w1, b1, w2, b2, c) for c in (0, 128, 300, 699)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0], y)


def test_full_ffn_block_sampled_rows():
    require_gpu()
    w = FFN_WORKLOADS["ffn_block8192_h4096_f16384"]
    log(f"workload {w.name}")
    x, w1, b1, w2, b2 = gen_ffn(w)
    y = _run(x, w1, b1, w2, b2, w.chunk_rows)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 4095, 6143, 8190, 8191],
                                     np.random.default_rng(0).integers(0, w.rows, 8)]))
    ref = oracle.ffn_forward(x[rows], w1, b1, w2, b2)
    compare("y (sampled rows)", y[torch.from_numpy(rows).cuda()], ref, "bf16")


def test_large_tiles_match_small_tiles_bit_for_bit():
    """4096 rows x 4096 hidden x 4096 ffn: as one block both GEMMs take the 256x256
    workgroup tiles; in 1024-row chunks they take the 128x128 ones.  Every output
    element is accumulated over k in the same order either way, so the two must agree
    bit for bit; sampled rows are also checked against the oracle."""
    require_gpu()
    x, w1, b1, w2, b2 = _inputs(103, 4096, 4096, 4096, True)
    y_big = _run(x, w1, b1, w2, b2, 0)
    y_small = _run(x, w1, b1, w2, b2, 1024)
    torch.cuda.synchronize()
    assert torch.equal(y_big, y_small)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095], np.random.default_rng(1).integers(0, 4096, 6)]))
    compare("y (sampled rows)", y_big[torch.from_numpy(rows).cuda()], oracle.ffn_forward(x[rows], w1, b1, w2, b2),
            "bf16")

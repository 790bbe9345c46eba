"""GPU parity: forward ring step and merge against the fp64 oracle (small shapes).

Shapes span several MFMA/LDS tiles and ragged tails; every rank of each ring
is run and compared element by element with dense fp64 attention over the
full sequence.
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
    ("f32", 64, 1, 1, 256, 4, False),     # the tiny fp32 workload's shape
    ("f32", 64, 1, 1, 256, 4, True),
    ("f32", 128, 2, 1, 100, 3, True),     # ragged, grouped
    ("bf16", 64, 4, 4, 256, 4, False),
    ("bf16", 64, 2, 2, 300, 3, True),     # ragged tail
    ("bf16", 128, 4, 2, 200, 3, True),    # ragged + GQA 2
    ("bf16", 128, 8, 2, 384, 2, True),    # GQA 4 (one K/V head per workgroup of 4 query heads)
    ("bf16", 128, 16, 1, 160, 2, False),  # group larger than the wave count
    ("bf16", 128, 6, 2, 96, 3, False),    # group 3 (not a divisor of the wave count)
    ("bf16", 64, 2, 2, 1, 3, True),       # degenerate: one token per block
    ("bf16", 128, 1, 1, 33, 1, True),     # a ring of one
    ("bf16", 128, 2, 2, 512, 2, False),
]


def _inputs(seed, dtype, d, hq, hkv, c, D, qscale=1.0):
    S = c * D
    q = gen_small(seed, (S, hq, d), dtype, qscale, 0)
    k = gen_small(seed, (S, hkv, d), dtype, 1.0, 1)
    v = gen_small(seed, (S, hkv, d), dtype, 1.0, 2)
    return q, k, v


def _run_all_ranks(q, k, v, dtype, c, D, causal):
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    outs, lses = [], []
    for r in range(D):
        o, l = ra.fwd(dev(q[r * c:(r + 1) * c], dtype), kb, vb, causal=causal, rank=r)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    return torch.cat(outs, 0), torch.cat(lses, 1)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_fwd_all_ranks_vs_oracle(case):
    require_gpu()
    dtype, d, hq, hkv, c, D, causal = case
    log(f"fwd case {case}")
    q, k, v = _inputs(31, dtype, d, hq, hkv, c, D)
    o_ref, l_ref = oracle.attention_fwd(q, k, v, causal=causal)
    o, l = _run_all_ranks(q, k, v, dtype, c, D, causal)
    compare("out", o, o_ref, dtype)
    compare("lse", l, l_ref, dtype)


@pytest.mark.parametrize("variant", ["peaky", "late_max"])
def test_fwd_rescaling_stress(variant):
    """Scores that force many running-max updates (peaky) or put the row maxima
    in the last ring round (late_max), stressing the rescaling of earlier rounds."""
    require_gpu()
    dtype, d, hq, hkv, c, D = "bf16", 128, 2, 2, 256, 4
    q, k, v = _inputs(37, dtype, d, hq, hkv, c, D, qscale=4.0 if variant == "peaky" else 1.0)
    if variant == "late_max":
        # rank 1 visits blocks 1, 0, 3, 2: make block 2 (the last round) dominate
        k = k.copy()
        k[2 * c:3 * c] = np.asarray(torch.from_numpy(k[2 * c:3 * c] * 3.0).to(torch.bfloat16).float())
    o_ref, l_ref = oracle.attention_fwd(q, k, v, causal=False)
    o, l = _run_all_ranks(q, k, v, dtype, c, D, False)
    compare("out", o, o_ref, dtype)
    compare("lse", l, l_ref, dtype)


def test_noncausal_every_rank_matches_dense_in_its_own_order():
    """Each rank visits the blocks in a different rotation; all agree with the oracle
    (order independence of the online merge)."""
    require_gpu()
    dtype, d, hq, c, D = "bf16", 64, 2, 128, 5
    q1 = gen_small(41, (c, hq, d), dtype, 1.0, 0)
    k = gen_small(41, (c * D, hq, d), dtype, 1.0, 1)
    v = gen_small(41, (c * D, hq, d), dtype, 1.0, 2)
    o_ref, l_ref = oracle.attention_fwd(q1, k, v, causal=False)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd = dev(q1, dtype)
    for r in range(D):
        o, l = ra.fwd(qd, kb, vb, causal=False, rank=r)
        torch.cuda.synchronize()
        compare(f"out rank {r}", o, o_ref, dtype)
        compare(f"lse rank {r}", l, l_ref, dtype)


def test_merge_kernel_vs_oracle():
    require_gpu()
    rng = np.random.default_rng(5)
    rows, heads, d = 333, 3, 64
    oa = rng.standard_normal((rows, heads, d)).astype(np.float32)
    ob = rng.standard_normal((rows, heads, d)).astype(np.float32)
    la = (rng.standard_normal((heads, rows)) * 4).astype(np.float32)
    lb = (rng.standard_normal((heads, rows)) * 4).astype(np.float32)
    la[0, :10] = -np.inf        # empty partial a
    lb[1, 5:15] = -np.inf       # empty partial b
    la[2, 20:25] = -np.inf
    lb[2, 20:25] = -np.inf      # both empty
    oa[2, 20:25] = np.nan       # garbage under an empty partial must not leak
    o_ref, l_ref = oracle.merge_partials(oa.astype(np.float64), la.astype(np.float64),
                                         np.nan_to_num(ob).astype(np.float64), lb.astype(np.float64))
    o_ref = np.where(np.isfinite(l_ref).T[:, :, None], o_ref, 0.0)
    toa, tla, tob, tlb = (torch.from_numpy(x).cuda() for x in (oa, la, ob, lb))
    o, l = ra.merge(toa, tla, tob, tlb)
    torch.cuda.synchronize()
    compare("merge out", o, o_ref, "f32")
    compare("merge lse", l, l_ref.astype(np.float64), "f32")
    # in place into a
    ra.merge(toa, tla, tob, tlb, out=toa, lse=tla)
    torch.cuda.synchronize()
    compare("merge out (in place)", toa, o_ref, "f32")
    compare("merge lse (in place)", tla, l_ref, "f32")


def test_merge_of_ring_partials_equals_one_call():
    """Checkpoint/resume: a partial over the first rounds merged with one over the
    rest equals the single call (the running (out, lse) is a complete state)."""
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 2, 192, 4
    q, k, v = _inputs(43, dtype, d, h, h, c, D)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd = dev(q[3 * c:4 * c], dtype)
    o_full, l_full = ra.fwd(qd, kb, vb, causal=True, rank=3)
    # part a: blocks 3 (the masked diagonal, as a ring of one) and 2; part b: blocks 0 and 1
    ob, lb = ra.fwd(qd, [kb[0], kb[1]], [vb[0], vb[1]], causal=False, rank=0)
    oa, la = ra.fwd(qd, [kb[3]], [vb[3]], causal=True, rank=0)
    oc, lc = ra.fwd(qd, [kb[2]], [vb[2]], causal=False, rank=0)
    oa, la = ra.merge(oa, la, oc, lc)
    o_m, l_m = ra.merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    qp = oracle.positions_for_block(3, c)
    o_ref, l_ref = oracle.attention_fwd(q[3 * c:4 * c], k, v, causal=True, q_pos=qp)
    compare("resumed out", o_m, o_ref, dtype)
    compare("resumed lse", l_m, l_ref, dtype)
    compare("single-call out", o_full, o_ref, dtype)
    assert torch.allclose(o_m, o_full, atol=1e-5, rtol=0)


@pytest.mark.parametrize("poison,delay", [(True, 0), (False, 200000), (True, 100000)])
def test_rotation_pipeline_ordering(poison, delay):
    """NaN-poisoned staging and a slowed copy stream must leave results bit-identical."""
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 4, 512, 6
    q, k, v = _inputs(47, dtype, d, h, h, c, D)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd = dev(q[4 * c:5 * c], dtype)
    o0, l0 = ra.fwd(qd, kb, vb, causal=False, rank=4)
    torch.cuda.synchronize()
    try:
        ra.ring_attn_debug(poison, delay)
        o1, l1 = ra.fwd(qd, kb, vb, causal=False, rank=4)
        torch.cuda.synchronize()
    finally:
        ra.ring_attn_debug(False, 0)
    assert not torch.isnan(o1).any()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_profile_reports_kernels_and_copies():
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 8, 2048, 4
    q, k, v = _inputs(53, dtype, d, h, h, c, D)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd = dev(q[:c], dtype)
    ra.ring_attn_profile_enable(True)
    try:
        ra.fwd(qd, kb, vb, causal=False, rank=0)
        torch.cuda.synchronize()
        recs, copy_ms, hidden = ra.ring_attn_profile_read()
    finally:
        ra.ring_attn_profile_enable(False)
    log(f"  profile: {recs} copy_ms={copy_ms:.4f} hidden_ms={hidden:.4f}")
    assert recs["fwd_step"][1] == D and recs["copy"][1] == D - 1
    assert copy_ms > 0 and 0 <= hidden <= copy_ms + 1e-6


def test_caller_workspace():
    """Staging in caller-owned memory gives bit-identical results; a workspace
    too small for the call is rejected without touching the outputs."""
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 4, 512, 4
    q, k, v = _inputs(59, dtype, d, h, h, c, D)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd = dev(q[3 * c:4 * c], dtype)
    o0, l0 = ra.fwd(qd, kb, vb, causal=False, rank=3)
    torch.cuda.synchronize()
    need = ra.ring_attn_workspace_bytes(c, h, d, 2)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    small = torch.empty((need // 8,), dtype=torch.float32, device="cuda")
    try:
        ra.ring_attn_set_workspace(ws, need)
        o1, l1 = ra.fwd(qd, kb, vb, causal=False, rank=3)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        assert not torch.isnan(ws).all()  # the staging really went through the caller's memory
        ra.ring_attn_set_workspace(small, need // 2)
        o2 = torch.full_like(o0, 7.0)
        l2 = torch.full_like(l0, 7.0)
        with pytest.raises(ra.RingAttnError, match="workspace"):
            ra.fwd(qd, kb, vb, causal=False, rank=3, out=o2, lse=l2)
        torch.cuda.synchronize()
        assert bool((o2 == 7.0).all()) and bool((l2 == 7.0).all())
    finally:
        ra.ring_attn_set_workspace(None, 0)
    o3, l3 = ra.fwd(qd, kb, vb, causal=False, rank=3)
    torch.cuda.synchronize()
    assert torch.equal(o0, o3) and torch.equal(l0, l3)


def test_mfma_rate_probe_is_plausible():
    require_gpu()
    sink = torch.empty((ra.MFMA_RATE_SINK_FLOATS,), dtype=torch.float32, device="cuda")
    tf = ra.ring_attn_mfma_rate(2000, sink)
    torch.cuda.synchronize()
    log(f"  mfma loop: {tf:.1f} TFLOP/s")
    assert 300.0 < tf < 2600.0  # below the public dense bf16 figure, far above any scalar path
    assert torch.isfinite(sink).all()


def test_binding_refuses_strided_views():
    """The library reads dense row-major buffers; a transposed view must be refused, not misread."""
    require_gpu()
    q = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device="cuda").transpose(0, 1)  # [64, 2, 64], strided
    kb = [torch.zeros((64, 2, 64), dtype=torch.bfloat16, device="cuda")]
    with pytest.raises(ValueError, match="contiguous"):
        ra.fwd(q, kb, kb, causal=False, rank=0)


def test_shutdown_then_reuse_gives_identical_results():
    """ring_attn_shutdown releases every per-device stream, event and buffer; the next
    calls rebuild them lazily and must reproduce the earlier results bit for bit."""
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 2, 256, 3
    q, k, v = _inputs(53, dtype, d, h, h, c, D)
    do = gen_small(53, (c * D, h, d), dtype, 1.0, 3)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd, dod = dev(q[2 * c:3 * c], dtype), dev(do[2 * c:3 * c], dtype)
    x = dev(gen_small(53, (256, 128), dtype, 1.0, 4), dtype)
    w1 = dev(gen_small(53, (512, 128), dtype, 0.09, 5), dtype)
    w2 = dev(gen_small(53, (128, 512), dtype, 0.045, 6), dtype)

    def run():
        o, l = ra.fwd(qd, kb, vb, causal=True, rank=2)
        dkb = [torch.zeros((c, h, d), dtype=torch.float32, device="cuda") for _ in range(D)]
        dvb = [torch.zeros((c, h, d), dtype=torch.float32, device="cuda") for _ in range(D)]
        g, _, _ = ra.bwd(qd, kb, vb, o, dod, l, causal=True, rank=2, dk_blocks=dkb, dv_blocks=dvb)
        y = ra.ffn_blockwise(x, w1, w2, chunk_rows=128)
        torch.cuda.synchronize()
        return [o, l, g, y] + dkb + dvb

    first = run()
    ra.ring_attn_shutdown()
    second = run()
    for i, (a, b) in enumerate(zip(first, second)):
        assert torch.equal(a, b), f"output {i} changed after shutdown"


def test_calls_order_against_the_callers_stream():
    """K/V blocks written on a (delayed) caller stream right before the call are what the
    ring reads: the rotation copies on the library's side stream wait for the work
    already enqueued on the caller's stream."""
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 2, 512, 4
    q, k, v = _inputs(59, dtype, d, h, h, c, D)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    qd = dev(q[c:2 * c], dtype)
    o_ref, l_ref = ra.fwd(qd, kb, vb, causal=False, rank=1)
    kb2 = [torch.zeros_like(x) for x in kb]
    vb2 = [torch.zeros_like(x) for x in vb]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)  # a bounded spin keeps the caller's stream busy for a few ms
        for dst, src in zip(kb2 + vb2, kb + vb):
            dst.copy_(src)
        o, l = ra.fwd(qd, kb2, vb2, causal=False, rank=1)
    s.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_calls_on_two_streams_serialise():
    """Calls issued on two streams of one device share the library's staging and
    workspace buffers; the library orders each call after the previous one, so the
    interleaved calls give bit-identical results to the same calls run serially.
    The first stream is held busy by a bounded spin, so without that ordering the
    second stream's calls would refill the shared buffers under the first's."""
    require_gpu()
    dtype, d, h, c, D = "bf16", 128, 4, 512, 5
    q, k, v = _inputs(73, dtype, d, h, h, c, D)
    do = gen_small(73, (c * D, h, d), dtype, 1.0, 3)
    kb = [dev(k[j * c:(j + 1) * c], dtype) for j in range(D)]
    vb = [dev(v[j * c:(j + 1) * c], dtype) for j in range(D)]
    ranks = (1, 3)
    qs = {r: dev(q[r * c:(r + 1) * c], dtype) for r in ranks}
    dos = {r: dev(do[r * c:(r + 1) * c], dtype) for r in ranks}

    def outputs():
        return {r: dict(o=torch.empty((c, h, d), device="cuda"), l=torch.empty((h, c), device="cuda"),
                        dq=torch.empty((c, h, d), device="cuda"),
                        dk=[torch.zeros((c, h, d), device="cuda") for _ in range(D)],
                        dv=[torch.zeros((c, h, d), device="cuda") for _ in range(D)]) for r in ranks}

    def call(r, res, stream=None):
        x = res[r]
        ra.fwd(qs[r], kb, vb, causal=False, rank=r, out=x["o"], lse=x["l"], stream=stream)
        ra.bwd(qs[r], kb, vb, x["o"], dos[r], x["l"], causal=False, rank=r, dq=x["dq"], dk_blocks=x["dk"],
               dv_blocks=x["dv"], stream=stream)

    serial = outputs()
    for r in ranks:
        call(r, serial)
    inter = outputs()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s1):
        torch.cuda._sleep(20_000_000)  # bounded spin: the first call starts a few ms late
    call(ranks[0], inter, stream=s1)
    call(ranks[1], inter, stream=s2)
    torch.cuda.synchronize()
    for r in ranks:
        for key in ("o", "l", "dq"):
            assert torch.equal(serial[r][key], inter[r][key]), f"rank {r} {key} differs"
        for j in range(D):
            assert torch.equal(serial[r]["dk"][j], inter[r]["dk"][j]), f"rank {r} dk[{j}] differs"
            assert torch.equal(serial[r]["dv"][j], inter[r]["dv"][j]), f"rank {r} dv[{j}] differs"

#!/usr/bin/env python3
"""Benchmark of the ring-attention step on one MI355X.

One "step" is one pass of the whole hot path over the workload's synthetic
input: for every rank of the workload, the forward ring step (schedule,
double-buffered K/V rotation copies, QK^T / online softmax / PV, merge into
the running output) and, if the workload has a backward, the backward ring
step of every rank (row terms, dK/dV and dQ kernels, the same rotation).

Prints ONE JSON line.  ``value`` is the algorithmic TFLOP/s of the whole step
(forward 4*d*Hq per visible query/key pair, backward 2.5x that), with inputs
resident in HBM before the timed region.  Per-kernel averages come from HIP
events the library records around its own launches during the timed region.

Only one GPU is supported: ``--gpus N`` with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ring-attn fwd/bwd TFLOP/s on 1 MI355X + % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="causal_128k_h32_d128")
    p.add_argument("--fwd-only", action="store_true", help="time only the forward of every rank")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the rocm-smi shader-clock sample (for runs under a profiler)")
    p.add_argument("--cpu-rows", type=int, default=192, help="query rows in the CPU oracle sample")
    p.add_argument("--copy-ref-mib", type=int, default=0,
                   help="before timing, run one plain device copy of this many MiB (a reference kernel of "
                        "known traffic for scaling profiler byte counters)")
    p.add_argument("--summarize-profiles", nargs=3, metavar=("STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: turn rocprofv3 CSV output (kernel stats, FETCH_SIZE pass, WRITE_SIZE "
                        "pass, all taken with --copy-ref-mib on the workload named by --workload) into "
                        "profiles/traffic.json and print the summary tables")
    p.add_argument("--summarize-mfma", metavar="PMC_CSV",
                   help="no GPU work: matrix-core busy fraction and wave wait/issue shares per kernel from a "
                        "rocprofv3 --pmc pass of SQ counters")
    p.add_argument("--summarize-overlap", nargs=2, metavar=("KERNEL_TRACE_CSV", "MEMORY_COPY_TRACE_CSV"),
                   help="no GPU work: share of the device-to-device copy time hidden under kernels")
    p.add_argument("--summarize-gaps", nargs="+", metavar="CSV_OR_JSON",
                   help="no GPU work: KERNEL_TRACE_CSV [BENCH_JSON]: idle time of the compute stream between "
                        "consecutive kernels of the timed steps of a rocprofv3 --kernel-trace run of this bench (same "
                        "--steps/--warmup), an upper bound on the exposed K/V rotation copy time; with the JSON line "
                        "that run printed, a lower bound on the hidden fraction of its copies")
    p.add_argument("--sweep-block-len", action="store_true",
                   help="the overlap condition of the ring: for block lengths 1024..16384 (32 heads x 128, "
                        "non-causal, one rank against 8 blocks) measure per-round kernel time, copy time and "
                        "the exposed copy time, next to the prediction from c_min = F/B")
    return p.parse_args()


def build_inputs(w, torch):
    """Seeded synthetic blocks, uploaded once (outside the timed region)."""
    from workloads import bf16_bits, gen_block
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(x):
        if w.dtype == "bf16":
            return torch.from_numpy(bf16_bits(x).view("int16")).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    c = w.block_len
    t0 = time.time()
    kb = [up(gen_block(w.seed, "k", j, c, w.kv_heads, w.head_dim, w.dtype)) for j in range(w.n_blocks)]
    vb = [up(gen_block(w.seed, "v", j, c, w.kv_heads, w.head_dim, w.dtype)) for j in range(w.n_blocks)]
    qs = {r: up(gen_block(w.seed, "q", r, c, w.heads, w.head_dim, w.dtype)) for r in w.ranks}
    dos = {}
    if w.backward:
        dos = {r: up(gen_block(w.seed, "do", r, c, w.heads, w.head_dim, w.dtype)) for r in w.ranks}
    torch.cuda.synchronize()
    log(f"[bench] inputs generated and uploaded in {time.time() - t0:.1f}s (dtype {tdt})")
    return qs, kb, vb, dos


def cpu_baseline(w, rows: int):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    from workloads import gen_block
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    if w.is_decode:
        return cpu_baseline_decode(w, threads)
    r = max(w.ranks)
    c = w.block_len
    nblk = w.n_blocks if (w.zigzag or not w.causal) else r + 1
    k = np.concatenate([gen_block(w.seed, "k", j, c, w.kv_heads, w.head_dim, w.dtype) for j in range(nblk)])
    v = np.concatenate([gen_block(w.seed, "v", j, c, w.kv_heads, w.head_dim, w.dtype) for j in range(nblk)])
    q = gen_block(w.seed, "q", r, c, w.heads, w.head_dim, w.dtype)
    sel = np.linspace(0, c - 1, rows).astype(np.int64)
    if w.zigzag:  # global positions of the zig-zag layout; keys sorted by position
        qpos = oracle.zigzag_positions(r, w.n_blocks, c)[sel]
        kpos = np.concatenate([oracle.zigzag_positions(j, w.n_blocks, c) for j in range(nblk)])
        order = np.argsort(kpos)
        k, v, kpos = k[order], v[order], kpos[order]
    else:
        qpos = r * c + sel
        kpos = None
    t0 = time.time()
    if w.backward:
        do = gen_block(w.seed, "do", r, c, w.heads, w.head_dim, w.dtype)
        oracle.attention_bwd(q[sel], k, v, do[sel], causal=w.causal, q_pos=qpos, k_pos=kpos)
    else:
        oracle.attention_fwd(q[sel], k, v, causal=w.causal, q_pos=qpos, k_pos=kpos)
    dt = time.time() - t0
    pairs = float(np.sum(qpos + 1)) if w.causal else float(rows * w.seq_len)
    flop = 4.0 * w.head_dim * w.heads * pairs * (3.5 if w.backward else 1.0)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 numpy oracle, {'forward+backward' if w.backward else 'forward'} of {rows} "
                       f"evenly spaced query rows x {w.heads} heads of rank {r} against its "
                       f"{k.shape[0]} visible keys ({dt:.1f}s)"),
            "seconds": dt}


def cpu_baseline_decode(w, threads: int):
    """The fp64 decode oracle on the whole decode workload (every query head and row, the whole context)."""
    import numpy as np

    import oracle
    from workloads import gen_block
    c, group = w.block_len, w.heads // w.kv_heads
    heads = list(range(w.heads))
    k = [gen_block(w.seed, "k", j, c, w.kv_heads, w.head_dim, w.dtype) for j in range(w.n_blocks)]
    v = [gen_block(w.seed, "v", j, c, w.kv_heads, w.head_dim, w.dtype) for j in range(w.n_blocks)]
    q = gen_block(w.seed, "q", 0, w.q_len, w.heads, w.head_dim, w.dtype)
    t0 = time.time()
    oracle.decode_forward(q, k, v, w.seq_len)
    dt = time.time() - t0
    flop = 4.0 * w.head_dim * len(heads) * w.q_len * w.seq_len
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 numpy decode oracle, the whole workload: {w.q_len} query rows x {len(heads)} heads "
                       f"against all {w.seq_len} keys ({dt:.1f}s)"),
            "seconds": dt}


def read_sclk_mhz():
    """Current shader clock of GPU 0 from rocm-smi (None when unavailable); never blocks > 15 s."""
    import re
    import subprocess
    import shutil
    smi = shutil.which("rocm-smi")
    if smi is None:
        return None
    try:  # rocm-smi is a Python script: run it with this interpreter, not through its #! line
        r = subprocess.run([sys.executable, smi, "--showclocks"], capture_output=True, text=True, timeout=15)
    except Exception:
        return None
    for line in r.stdout.splitlines():
        if "sclk" in line and "GPU[0]" in line:
            m = re.search(r"\((\d+)\s*Mhz\)", line, re.IGNORECASE)
            if m:
                return int(m.group(1))
    return None


class ClockSampler:
    """Samples the shader clock once, `delay` seconds into the timed region (CPU thread)."""

    def __init__(self, delay: float = 2.0):
        import threading
        self.mhz = None
        self._t = threading.Timer(delay, self._run)
        self._t.daemon = True

    def _run(self):
        self.mhz = read_sclk_mhz()

    def start(self):
        self._t.start()

    def join(self):
        self._t.join(timeout=20)
        return self.mhz


def reference_copy(args, torch):
    """One plain device copy of --copy-ref-mib MiB: a kernel of known traffic that scales the
    profiler's byte counters (FETCH_SIZE / WRITE_SIZE) of the same run."""
    if args.copy_ref_mib <= 0:
        return
    nbytes = args.copy_ref_mib << 20
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] reference copy: {nbytes} bytes read + {nbytes} bytes written")
    del src, dst


def run_decode(args, w, torch, ra):
    """Decode workload: one step = one ring_attn_decode call over every block (HBM-bound)."""
    from workloads import bf16_bits, gen_block
    c = w.block_len

    def up(x):
        return torch.from_numpy(bf16_bits(x).view("int16")).view(torch.bfloat16).cuda()

    t0 = time.time()
    kb = [up(gen_block(w.seed, "k", j, c, w.kv_heads, w.head_dim, w.dtype)) for j in range(w.n_blocks)]
    vb = [up(gen_block(w.seed, "v", j, c, w.kv_heads, w.head_dim, w.dtype)) for j in range(w.n_blocks)]
    q = up(gen_block(w.seed, "q", 0, w.q_len, w.heads, w.head_dim, w.dtype))
    out = torch.empty((w.q_len, w.heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.heads, w.q_len), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] decode inputs uploaded in {time.time() - t0:.1f}s")

    def step():
        ra.decode(q, kb, vb, q_pos0=w.seq_len, out=out, lse=lse)

    reference_copy(args, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ra.ring_attn_profile_enable(True)
    ra.ring_attn_profile_read()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms_total = evs[0].elapsed_time(evs[-1])
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    recs, _, _ = ra.ring_attn_profile_read()
    ra.ring_attn_profile_enable(False)
    ms_step = ms_total / args.steps
    flop = w.fwd_flop()
    value = flop / (ms_step * 1e-3) / 1e12
    kern = {}
    for name, (ms, cnt) in recs.items():
        if cnt:
            kern[name] = {"launches_per_step": cnt // args.steps, "avg_launch_ms": ms / cnt,
                          "ms_per_step": ms / args.steps}
    # algorithmic bytes of one decode step: every K/V byte once, the query rows, out and lse
    alg_bytes = w.kv_bytes() + w.q_len * w.heads * w.head_dim * (2 + 4) + w.heads * w.q_len * 4
    dom_ms = kern.get("decode_partial", {}).get("avg_launch_ms")
    achieved = alg_bytes / (dom_ms * 1e-3) / 1e9 if dom_ms else None
    roofline = {"bound": "hbm", "kernel": "decode_partial", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": (achieved / PEAK_HBM_GBS) if achieved else None,
                "traffic": profiled_traffic("decode_partial", w.head_dim, w.dtype, w.name),
                "algorithmic_bytes": alg_bytes}
    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "seq_len": w.seq_len, "n_blocks": w.n_blocks, "block_len": c,
                   "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim, "q_len": w.q_len,
                   "pass": "decode", "batch": 1},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 4), "step_ms_min": round(step_ms[0], 4),
        "hbm_gbs_whole_step": round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
        "kernels": kern, "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(w, 0)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def run_ffn(args, w, torch, ra):
    """Blockwise feedforward workload: one step = ring_attn_ffn_blockwise over the block's rows."""
    import numpy as np

    from workloads import bf16_bits, gen_ffn
    x, w1, b1, w2, b2 = gen_ffn(w)

    def up16(a):
        return torch.from_numpy(bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()

    xd, w1d, w2d = up16(x), up16(w1), up16(w2)
    b1d, b2d = torch.from_numpy(b1).cuda(), torch.from_numpy(b2).cuda()
    y = torch.empty((w.rows, w.hidden), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step():
        ra.ffn_blockwise(xd, w1d, w2d, b1=b1d, b2=b2d, chunk_rows=w.chunk_rows, y=y)

    reference_copy(args, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ra.ring_attn_profile_enable(True)
    ra.ring_attn_profile_read()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms_total = evs[0].elapsed_time(evs[-1])
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    recs, _, _ = ra.ring_attn_profile_read()
    ra.ring_attn_profile_enable(False)
    ms_step = ms_total / args.steps
    value = w.flop() / (ms_step * 1e-3) / 1e12
    kern = {}
    for name, (ms, cnt) in recs.items():
        if cnt:
            per = ms / args.steps
            kern[name] = {"launches_per_step": cnt // args.steps, "avg_launch_ms": ms / cnt, "ms_per_step": per,
                          "achieved_tflops": (w.flop() / 2) / (per * 1e-3) / 1e12}
    dom = max(("ffn_up", "ffn_down"), key=lambda k: kern.get(k, {}).get("ms_per_step", 0.0))
    achieved = kern.get(dom, {}).get("achieved_tflops")
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": (achieved / PEAK_BF16_TFLOPS) if achieved else None,
                "traffic": profiled_traffic(dom, 0, "bf16", w.name)}
    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "hidden": w.hidden, "ffn": w.ffn,
                   "chunk_rows": w.chunk_rows, "pass": "feedforward", "batch": 1},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 4), "step_ms_min": round(step_ms[0], 4),
        "intermediate_bytes": w.chunk_rows * w.ffn * 2,
        "intermediate_bytes_unblocked": w.rows * w.ffn * 2,
        "kernels": kern, "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        sel = np.arange(w.rows)  # the whole block (about 10 s of fp64 work on 16 cores)
        t0 = time.time()
        oracle.ffn_forward(x[sel], w1, b1, w2, b2)
        dt = time.time() - t0
        result["cpu_baseline"] = {"value": 4.0 * len(sel) * w.hidden * w.ffn / dt / 1e12, "unit": "TFLOP/s",
                                  "cores": int(threads), "kind": "oracle",
                                  "sample": f"fp64 numpy feedforward oracle on all {len(sel)} rows of the block "
                                            f"({dt:.1f}s)", "seconds": dt}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def profiled_traffic(kind: str, head_dim: int, dtype: str, workload: str):
    """HBM bytes per dispatch of a kernel from the committed profiler summary, or None.

    profiles/traffic.json holds, per workload, FETCH_SIZE/WRITE_SIZE-derived bytes
    (scaled by a reference copy) per kernel, each with hashes of the kernel sources
    it was taken with; a workload that was not profiled, or any source change
    since, gives None.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if dtype != "bf16" or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("workloads", {}).get(workload)
    if rec is None:
        return None
    pattern = {"fwd_step": "fwd_bf16_kernel", "bwd_dkdv": "bwd_dkdv_bf16_kernel", "bwd_dq": "bwd_dq_bf16_kernel",
               "decode_partial": "decode_partial_kernel", "ffn_up": "gemm_bt_kernel<",
               "ffn_down": "gemm_bt_kernel<"}.get(kind)
    for name, t in rec.items():
        if not (pattern and pattern in name):
            continue
        if kind.startswith(("fwd", "bwd", "decode")) and not (f"<{head_dim}," in name or f"<{head_dim}>" in name):
            continue
        if kind == "ffn_up" and not name.endswith("true>") or kind == "ffn_down" and not name.endswith("false>"):
            continue
        recorded = t.get("source_sha256", {})
        for fname in kernel_sources(name):
            src = os.path.join(ROOT, "long_context_exact_ring_amd", "csrc", fname)
            if fname not in recorded or hashlib.sha256(open(src, "rb").read()).hexdigest() != recorded[fname]:
                return None  # the kernel changed since its counters were taken
        return round(t["read_bytes"] + t["write_bytes"])
    return None


COMMON_SOURCES = ("kcommon.h", "kernels.h")
KERNEL_SOURCES = (("fwd_bf16_kernel", ("fwd_step.hip", "fwd_common.h", "tile_stage.h")),
                  ("bwd_dkdv_bf16_kernel", ("bwd_bf16.hip",)), ("bwd_dq_bf16_kernel", ("bwd_bf16.hip",)),
                  ("bwd_pre_kernel", ("merge.hip",)), ("decode_", ("decode.hip",)),
                  ("gemm_bt_kernel", ("ffn.hip",)), ("merge", ("merge.hip",)))


def kernel_sources(name: str):
    """The source files a kernel's code comes from (its own file plus the shared headers)."""
    for pattern, files in KERNEL_SOURCES:
        if pattern in name:
            return files + COMMON_SOURCES
    return tuple(sorted({f for _, fs in KERNEL_SOURCES for f in fs})) + COMMON_SOURCES
REF_COPY_KERNEL = "__amd_rocclr_copyBuffer"


def summarize_profiles(stats_csv: str, fetch_csv: str, write_csv: str, copy_ref_mib: int, workload: str):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same counters read
    for the reference copy of known size, average per kernel, write profiles/traffic.json
    (with the kernel sources' hashes) and print markdown tables of both passes."""
    import collections
    import csv
    import hashlib
    if copy_ref_mib <= 0:
        sys.exit("--summarize-profiles needs the --copy-ref-mib the counter runs used")
    ref_kib = copy_ref_mib * 1024.0

    def per_kernel(path):
        acc, cnt, ref = collections.defaultdict(float), collections.Counter(), []
        for row in csv.DictReader(open(path)):
            name = row["Kernel_Name"].split("(")[0].replace("void ", "")
            val = float(row["Counter_Value"])
            if REF_COPY_KERNEL in name:
                ref.append(val)
                continue
            acc[name] += val
            cnt[name] += 1
        if not ref:
            sys.exit(f"{path}: no reference copy dispatch found")
        # host uploads can also run as copy kernels; the 1 GiB reference is by far the largest
        return {k: (acc[k] / cnt[k], cnt[k]) for k in acc}, max(ref)

    fetch, ref_f = per_kernel(fetch_csv)
    write, ref_w = per_kernel(write_csv)
    sf, sw = ref_kib / ref_f, ref_kib / ref_w
    rows = list(csv.DictReader(open(stats_csv)))
    avg_ns = {row["Name"].split("(")[0].replace("void ", ""): float(row["AverageNs"]) for row in rows}
    kernels = {}
    print(f"Scaling: the {copy_ref_mib} MiB reference copy ({ref_kib:.0f} KiB read + {ref_kib:.0f} KiB "
          f"written) reads FETCH_SIZE = {ref_f:.0f} KiB and WRITE_SIZE = {ref_w:.0f} KiB, so FETCH_SIZE is "
          f"scaled by {sf:.3f} and WRITE_SIZE by {sw:.3f}.\n")
    print("| kernel | dispatches | FETCH_SIZE (KiB, raw) | WRITE_SIZE (KiB, raw) | read (MB, scaled) | "
          "written (MB, scaled) | HBM GB/s (at the trace's average duration) |")
    print("|---|---|---|---|---|---|---|")
    for name in sorted(set(fetch) & set(write)):
        (f, n), (wv, _) = fetch[name], write[name]
        rb, wb = f * sf * 1024.0, wv * sw * 1024.0
        kernels[name] = {"read_bytes": rb, "write_bytes": wb}
        gbs = f"{(rb + wb) / avg_ns[name]:.0f}" if avg_ns.get(name) else "-"
        print(f"| `{name}` | {n} | {f:.0f} | {wv:.0f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {gbs} |")
    # merge into the committed record; every kernel entry carries the source hashes it was taken with
    csrc = os.path.join(ROOT, "long_context_exact_ring_amd", "csrc")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    workloads = rec.get("workloads", {})
    workloads[workload] = {
        name: dict(t, source_sha256={f: hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()
                                     for f in kernel_sources(name)})
        for name, t in kernels.items()}
    rec = {"workloads": workloads,
           "note": "per workload: HBM bytes per dispatch from FETCH_SIZE/WRITE_SIZE, scaled by a reference copy; "
                   "an entry is stale once any source file listed with it has changed"}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("\n| kernel | calls | avg (us) | total (ms) | % of kernel time |")
    print("|---|---|---|---|---|")
    for row in rows:
        print(f"| `{row['Name'][:90]}` | {row['Calls']} | {float(row['AverageNs']) / 1e3:.1f} | "
              f"{float(row['TotalDurationNs']) / 1e6:.1f} | {row['Percentage']} |")


def summarize_mfma(pmc_csv: str):
    """Matrix-core utilisation per kernel from one rocprofv3 --pmc pass of SQ counters.

    busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES): the register-only MFMA
    loop (ring_attn_mfma_rate, also in the run) reads 1.00 with it.  The wave-cycle
    shares come from SQ_WAIT_ANY, SQ_ACTIVE_INST_ANY and SQ_WAVE_CYCLES."""
    import collections
    import csv
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for row in csv.DictReader(open(pmc_csv)):
        name = row["Kernel_Name"].split("(")[0].replace("void ", "")
        acc[name][row["Counter_Name"]] += float(row["Counter_Value"])
        disp[name].add(row["Dispatch_Id"])
    print("| kernel | dispatches | MFMA busy | waves waiting (SQ_WAIT_ANY) | waves issuing (SQ_ACTIVE_INST_ANY) | "
          "LDS bank conflicts per LDS instruction |")
    print("|---|---|---|---|---|---|")
    for name in sorted(acc):
        c = acc[name]
        if not c.get("SQ_BUSY_CU_CYCLES"):
            continue
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4.0 * c["SQ_BUSY_CU_CYCLES"])
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        wait = f"{c['SQ_WAIT_ANY'] / wc:.2f}" if wc and "SQ_WAIT_ANY" in c else "-"
        act = f"{c['SQ_ACTIVE_INST_ANY'] / wc:.2f}" if wc and "SQ_ACTIVE_INST_ANY" in c else "-"
        lds = c.get("SQ_INSTS_LDS", 0.0)
        conf = f"{c['SQ_LDS_BANK_CONFLICT'] / lds:.3f}" if lds and "SQ_LDS_BANK_CONFLICT" in c else "-"
        print(f"| `{name}` | {len(disp[name])} | {busy:.2f} | {wait} | {act} | {conf} |")


def summarize_overlap(kernel_trace_csv: str, copy_trace_csv: str):
    """Share of the device-to-device copy time during which some kernel was running, from
    a rocprofv3 --kernel-trace --memory-copy-trace run (the K/V rotation copies)."""
    import csv
    spans = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in csv.DictReader(open(kernel_trace_csv)))
    merged = []
    for a, b in spans:
        if merged and a <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], b)
        else:
            merged.append([a, b])
    copies = [r for r in csv.DictReader(open(copy_trace_csv))
              if any("DEVICE_TO_DEVICE" in str(v) for v in r.values())]
    import bisect
    starts = [m[0] for m in merged]
    total = hidden = 0
    for r in copies:
        a, b = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        total += b - a
        i = max(bisect.bisect_right(starts, a) - 1, 0)
        while i < len(merged) and merged[i][0] < b:
            lo, hi = max(a, merged[i][0]), min(b, merged[i][1])
            if hi > lo:
                hidden += hi - lo
            i += 1
    print(f"device-to-device copies: {len(copies)}, {total / 1e6:.1f} ms in total, "
          f"{hidden / 1e6:.1f} ms of it while a kernel ran: hidden fraction {hidden / max(total, 1):.4f}")
    return hidden / max(total, 1)


def summarize_gaps(trace_csv: str, steps: int, warmup: int, bench_json: str | None = None):
    """Idle time of the compute stream inside the timed steps of a kernel-trace run.

    Every kernel of a ring step runs on the caller's stream; the K/V copies run on
    the copy engine and the stream only waits when a round's block has not arrived.
    So the gaps between consecutive kernels (launch latency included) bound the
    exposed copy time from above.  The bench's kernels are the same in every step:
    the timed steps are the last steps/(warmup+steps) of the kernels before the
    matrix-core rate probe that follows the timed region.  Gaps are also listed
    by the pair of kernels around them: a dK/dV -> dQ gap never waits for a copy
    (the same round), so it gives the launch-to-launch baseline.  With the JSON
    line the traced bench printed, the copy time of that same run (library
    events) turns the idle time into a lower bound on the hidden fraction."""
    import collections
    import csv
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    first = next(i for i, n in enumerate(names) if "fwd_bf16_kernel" in n or "fwd_step_kernel" in n)
    probe = next((i for i, n in enumerate(names) if "mfma_rate_kernel" in n), len(rows))
    ring = rows[first:probe]
    if len(ring) % (steps + warmup):
        sys.exit(f"{len(ring)} kernels do not split into {steps + warmup} equal steps")
    per = len(ring) // (steps + warmup)
    timed = ring[-steps * per:]

    def kind(name):
        for k in ("fwd_bf16", "fwd_step", "bwd_dkdv", "bwd_dq", "bwd_pre", "FillFunctor"):
            if k in name:
                return k
        return name[:40]

    gaps, by_pair = [], collections.defaultdict(list)
    for a, b in zip(timed, timed[1:]):
        g = max(0, int(b["Start_Timestamp"]) - int(a["End_Timestamp"]))
        gaps.append(g)
        by_pair[(kind(a["Kernel_Name"]), kind(b["Kernel_Name"]))].append(g)
    busy = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed)
    span = int(timed[-1]["End_Timestamp"]) - int(timed[0]["Start_Timestamp"])
    gap_ms = sum(gaps) / 1e6 / steps
    out = {"kernels_per_step": per, "span_ms_per_step": span / 1e6 / steps, "kernel_ms_per_step": busy / 1e6 / steps,
           "idle_ms_per_step": gap_ms, "largest_gap_us": max(gaps) / 1e3 if gaps else 0.0}
    if bench_json:
        rec = json.loads(open(bench_json).read().strip().splitlines()[-1])
        cms = rec["overlap"]["copy_ms_per_step"]
        out["copy_ms_per_step_same_run"] = cms
        out["copy_ms_per_launch_same_run"] = rec["kernels"]["copy"]["avg_launch_ms"]
        out["hidden_frac_lower_bound"] = max(0.0, 1.0 - gap_ms / cms)
    print("| previous kernel -> next kernel | gaps per step | idle (ms per step) | median gap (us) | max gap (us) |")
    print("|---|---|---|---|---|")
    for pair, gs in sorted(by_pair.items(), key=lambda kv: -sum(kv[1])):
        gs = sorted(gs)
        print(f"| {pair[0]} -> {pair[1]} | {len(gs) // steps} | {sum(gs) / 1e6 / steps:.1f} | "
              f"{gs[len(gs) // 2] / 1e3:.1f} | {gs[-1] / 1e3:.1f} |")
    print(json.dumps(out))
    return out


def sweep_block_len(args, torch, ra):
    """Per-round compute and copy time against the block length (the overlap condition).

    One rank's non-causal forward against D = 8 blocks of 32 heads x 128: every round
    is a full c x c block pair, the K/V copy of the next round (2 c Hkv d bf16 bytes)
    runs while the current round computes (4 d Hq c^2 flop).  The copy is hidden when
    c >= c_min = (F / B) (Hkv / Hq), F the forward kernel's rate and B the copy
    engine's, both measured here.  Exposed copy time per round is the call's wall time
    minus its kernel time, over the rounds that waited for a copy."""
    from workloads import bf16_bits, gen_block
    D, hq, hkv, d = 8, 32, 32, 128
    res = []
    for c in (1024, 2048, 4096, 8192, 16384):
        def up(x):
            return torch.from_numpy(bf16_bits(x).view("int16")).view(torch.bfloat16).cuda()
        kb = [up(gen_block(11, "k", j, c, hkv, d, "bf16")) for j in range(D)]
        vb = [up(gen_block(11, "v", j, c, hkv, d, "bf16")) for j in range(D)]
        q = up(gen_block(11, "q", 0, c, hq, d, "bf16"))
        out = torch.empty((c, hq, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((hq, c), dtype=torch.float32, device="cuda")
        for _ in range(2):
            ra.fwd(q, kb, vb, causal=False, rank=0, out=out, lse=lse)
        torch.cuda.synchronize()
        reps = max(3, min(40, int(2e4 / c)))
        ra.ring_attn_profile_enable(True)
        ra.ring_attn_profile_read()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            ra.fwd(q, kb, vb, causal=False, rank=0, out=out, lse=lse)
        e1.record()
        torch.cuda.synchronize()
        recs, copy_ms, _ = ra.ring_attn_profile_read()
        ra.ring_attn_profile_enable(False)
        wall = e0.elapsed_time(e1) / reps
        kms, kcnt = recs["fwd_step"]
        cms, ccnt = recs["copy"]
        t_k, t_c = kms / kcnt, cms / ccnt                      # per round
        F = 4.0 * d * hq * c * c / (t_k * 1e-3)                # flop/s of one full round
        B = 2.0 * 2 * c * hkv * d / (t_c * 1e-3)               # bytes/s of one K+V copy
        c_min = F / B * hkv / hq
        exposed = max(0.0, wall - kms / reps)                  # per call (D - 1 copied rounds)
        pred = (D - 1) * max(0.0, t_c - t_k)
        res.append({"block_len": c, "kernel_ms_per_round": t_k, "copy_ms_per_round": t_c,
                    "fwd_tflops": F / 1e12, "copy_gbs": B / 1e9, "c_min": c_min,
                    "exposed_ms_per_call": exposed, "predicted_exposed_ms_per_call": pred,
                    "wall_ms_per_call": wall})
        log(f"[sweep] c={c}: kernel {t_k:.3f} ms, copy {t_c:.3f} ms per round, c_min {c_min:.0f}, "
            f"exposed {exposed:.3f} ms (predicted {pred:.3f}) per call")
        del kb, vb, q, out, lse
        torch.cuda.empty_cache()
    print("| block_len c | kernel ms / round | copy ms / round | forward TFLOP/s | copy GB/s | c_min = (F/B)(Hkv/Hq) "
          "| exposed ms / call (measured) | exposed ms / call (predicted, (D-1) max(0, copy - kernel)) |")
    print("|---|---|---|---|---|---|---|---|")
    for r in res:
        print(f"| {r['block_len']} | {r['kernel_ms_per_round']:.3f} | {r['copy_ms_per_round']:.3f} | "
              f"{r['fwd_tflops']:.0f} | {r['copy_gbs']:.0f} | {r['c_min']:.0f} | {r['exposed_ms_per_call']:.3f} | "
              f"{r['predicted_exposed_ms_per_call']:.3f} |")
    print(json.dumps({"sweep": res}))


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, args.copy_ref_mib, args.workload)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_overlap:
        summarize_overlap(*args.summarize_overlap)
        return
    if args.summarize_gaps:
        summarize_gaps(args.summarize_gaps[0], args.steps, args.warmup,
                       args.summarize_gaps[1] if len(args.summarize_gaps) > 1 else None)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU ring is not built "
              f"in this library", file=sys.stderr)
        sys.exit(2)
    import torch

    from long_context_exact_ring_amd.build import build_if_missing
    build_if_missing()  # loads what is built; builds only in a fresh checkout
    import long_context_exact_ring_amd as ra
    from workloads import FFN_WORKLOADS, WORKLOADS

    if args.sweep_block_len:
        torch.cuda.set_device(0)
        sweep_block_len(args, torch, ra)
        return
    if args.workload in FFN_WORKLOADS:
        torch.cuda.set_device(0)
        run_ffn(args, FFN_WORKLOADS[args.workload], torch, ra)
        return
    w = WORKLOADS[args.workload]
    if w.is_decode:
        torch.cuda.set_device(0)
        run_decode(args, w, torch, ra)
        return
    do_bwd = w.backward and not args.fwd_only
    torch.cuda.set_device(0)
    qs, kb, vb, dos = build_inputs(w, torch)
    c, hq, hkv, d = w.block_len, w.heads, w.kv_heads, w.head_dim
    outs = {r: torch.empty((c, hq, d), dtype=torch.float32, device="cuda") for r in w.ranks}
    lses = {r: torch.empty((hq, c), dtype=torch.float32, device="cuda") for r in w.ranks}
    if do_bwd:
        dqs = {r: torch.empty((c, hq, d), dtype=torch.float32, device="cuda") for r in w.ranks}
        dkb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(w.n_blocks)]
        dvb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(w.n_blocks)]

    # per-rank device time (one rank's forward + backward calls), a load-balance indicator
    rank_ev = {r: [] for r in w.ranks}
    timing = {"on": False}

    def mark(r, which):
        if timing["on"]:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            rank_ev[r].append((which, e))

    def step():
        for r in w.ranks:
            mark(r, 0)
            ra.fwd(qs[r], kb, vb, causal=w.causal, rank=r, out=outs[r], lse=lses[r], zigzag=w.zigzag)
            mark(r, 1)
        if do_bwd:
            for t in dkb + dvb:
                t.zero_()
            for r in w.ranks:
                mark(r, 0)
                ra.bwd(qs[r], kb, vb, outs[r], dos[r], lses[r], causal=w.causal, rank=r, dq=dqs[r],
                       dk_blocks=dkb, dv_blocks=dvb, zigzag=w.zigzag)
                mark(r, 1)

    reference_copy(args, torch)
    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup step(s) done")

    ra.ring_attn_profile_enable(True)
    ra.ring_attn_profile_read()  # discard anything recorded before
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    timing["on"] = True
    clock = ClockSampler(min(2.0, 0.3 * args.steps))
    if not args.no_clock:
        clock.start()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    timing["on"] = False
    sclk = None if args.no_clock else clock.join()
    ms_total = evs[0].elapsed_time(evs[-1])
    rank_ms = {}
    for r, marks in rank_ev.items():
        tot = sum(marks[i][1].elapsed_time(marks[i + 1][1]) for i in range(0, len(marks) - 1, 2))
        rank_ms[r] = tot / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    recs, copy_ms, hidden_ms = ra.ring_attn_profile_read()
    ra.ring_attn_profile_enable(False)
    ms_step = ms_total / args.steps
    log(f"[bench] {args.steps} timed step(s): {ms_step:.3f} ms/step")
    # practical matrix-core ceiling at the clock the card holds under MFMA load (after the timed region)
    sink = torch.empty((ra.MFMA_RATE_SINK_FLOATS,), dtype=torch.float32, device="cuda")
    mfma_loop = ra.ring_attn_mfma_rate(20000, sink) if w.dtype == "bf16" else None

    fwd_flop, bwd_flop = w.fwd_flop(), (w.bwd_flop() if do_bwd else 0.0)
    step_flop = fwd_flop + bwd_flop
    value = step_flop / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS

    # per-kernel averages over the timed region (library HIP events on the launch stream)
    kern = {}
    alg = {"fwd_step": fwd_flop, "bwd_dkdv": 0.8 * bwd_flop, "bwd_dq": 0.2 * bwd_flop}
    for name, (ms, cnt) in recs.items():
        if cnt:
            per = ms / args.steps
            kern[name] = {"launches_per_step": cnt // args.steps, "avg_launch_ms": ms / cnt,
                          "ms_per_step": per}
            if name in alg and alg[name] > 0:
                kern[name]["achieved_tflops"] = alg[name] / (per * 1e-3) / 1e12
    mm = [(v["ms_per_step"], k) for k, v in kern.items() if k in alg and alg[k] > 0]
    dom = max(mm)[1] if mm else "fwd_step"
    dom_ms = kern.get(dom, {}).get("ms_per_step", float("nan"))
    achieved = alg[dom] / (dom_ms * 1e-3) / 1e12 if dom in kern else None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": (achieved / peak) if achieved else None,
                "traffic": profiled_traffic(dom, d, w.dtype, w.name)}

    overlap = {"copy_ms_per_step": copy_ms / args.steps, "hidden_ms_per_step": hidden_ms / args.steps,
               "hidden_frac": (hidden_ms / copy_ms) if copy_ms > 0 else None,
               "copy_engine": os.environ.get("RING_ATTN_COPY", "sdma")}
    # the overlap condition c >= c_min = (F / B)(Hkv / Hq), with F the forward kernels' rate
    # and B the copy engine's rate, both measured in this run
    if "copy" in kern and "fwd_step" in kern:
        copy_bytes = 2.0 * c * hkv * d * (2 if w.dtype == "bf16" else 4)  # K + V of one block
        B = copy_bytes / (kern["copy"]["avg_launch_ms"] * 1e-3)
        F = fwd_flop / (kern["fwd_step"]["ms_per_step"] * 1e-3)
        elem = 2 if w.dtype == "bf16" else 4
        overlap["copy_gbs"] = round(B / 1e9, 1)
        overlap["c_min_tokens"] = round(F / B * hkv / hq * elem / 2, 1)
        overlap["block_len_over_c_min"] = round(c / overlap["c_min_tokens"], 2)

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "seq_len": w.seq_len, "n_blocks": w.n_blocks, "block_len": c,
                   "heads": hq, "kv_heads": hkv, "head_dim": d, "causal": w.causal,
                   "ranks": len(w.ranks), "pass": "forward+backward" if do_bwd else "forward",
                   "batch": 1},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 3), "step_ms_min": round(step_ms[0], 3),
        "mfma_loop_tflops": round(mfma_loop, 1) if mfma_loop else None,
        "sclk_mhz_during_run": sclk,
        "peak_at_sclk_tflops": round(256 * 4096 * sclk * 1e6 / 1e12, 1) if sclk else None,
        "pct_of_mfma_loop": round(100.0 * value / mfma_loop, 2) if mfma_loop else None,
        "fwd_tflops": None, "bwd_tflops": None,
        "kernels": kern, "overlap": overlap, "roofline": roofline,
        "layout": "zigzag" if w.zigzag else "contiguous",
        "rank_ms": [round(rank_ms[r], 3) for r in w.ranks],
        "rank_balance": round(sum(rank_ms.values()) / len(rank_ms) / max(rank_ms.values()), 4) if rank_ms else None,
    }
    if "fwd_step" in kern:
        # forward-only rate over the forward kernels' own time
        result["fwd_tflops"] = round(fwd_flop / (kern["fwd_step"]["ms_per_step"] * 1e-3) / 1e12, 2)
    if do_bwd and "bwd_dkdv" in kern:
        bms = sum(kern[k]["ms_per_step"] for k in ("bwd_dkdv", "bwd_dq", "bwd_pre") if k in kern)
        result["bwd_tflops"] = round(bwd_flop / (bms * 1e-3) / 1e12, 2)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

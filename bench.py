#!/usr/bin/env python3
"""Benchmark of the gfx950 warp-pipelined GEMM; prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--schedule S] [--splits N|auto] [--gpus 1]

A step is one C = A.B of the whole product (by default FP16 operands, FP32
accumulation, FP16 output on the compute-bound 4096x4096x8192 shape, one
launch; the other workloads include 8192^3 BF16, 8192^3 FP8 E4M3 and the
512x4096x8192 row block one GPU of eight would hold, which runs split K: two
launches per step), on inputs already resident in HBM.  Inputs are seeded synthetic matrices (A and
B uniform in [-1, 1), B given N x K); enough rotating input sets are kept on
the device that one pass over them exceeds the 256 MB last-level cache, and
consecutive steps use consecutive sets.  Before the W warm-up launches the
GPU runs untimed launches until its clock has settled (at least --settle-ms of
GPU time, then until the per-launch time stops falling; reported as settle_ms
and settle_launches), so the K timed launches measure the sustained rate
however small K and W are.  The K timed launches are bracketed by device
synchronisation and timed with HIP events on the stream they are enqueued on.
Throughput = 2MNK / time.

The CPU baseline runs the oracle (a plain binary64 triple loop) on a bounded
block of output rows of the same workload, on the host's cores, and the GPU
result on those rows is checked against it.

The attention workloads (--workload attn_...) time attention_fwd over the
whole batch instead: one launch per step, throughput = 4 B H (allowed query
-key pairs) D / time; the CPU baseline runs the float64 attention oracle on a
bounded sample of query rows.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402

METRIC = "FP16 GEMM TFLOP/s at M=N=4096,K=8192 and % of MI355X MFMA peak"
# Published MI355X dense MFMA peaks (TFLOP/s) per operand type.
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0}
# 256 CUs x 4 SIMDs x FLOP/clk (1024 FP16/BF16, 2048 FP8) x 2.4 GHz: the same
# peaks from the unit counts.
PEAK_TFLOPS_UNITS = {"f16": 256 * 4 * 1024 * 2.4e9 / 1e12, "bf16": 256 * 4 * 1024 * 2.4e9 / 1e12,
                     "fp8": 256 * 4 * 2048 * 2.4e9 / 1e12}
# The pages' MI355X figures for these exact shapes: the 8-wave warp-pipelined
# Triton kernel (FP16, M=N=4096, K=8192 and K=16384) and the hand-written
# 4-wave HIP C++ FP8 kernel at matrix size 8192.  Context for vs_baseline.
PAGES_TFLOPS = {"f16_4096x4096x8192": 1437.0, "f16_4096x4096x16384": 1485.0, "fp8_8192": 3292.0}
MALL_BYTES = 256 * 2 ** 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
def counter_record(workload: str, schedule: str):
    """The committed counter record (profiles/traffic.json) of this kernel on
    this workload, if it was taken on the kernel's current code (the
    comment-free text of its sources); else None."""
    from matrix_core_scheduling_amd import profiling

    kernel = schedule
    if kernel not in profiling.KERNEL_SOURCES:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(profiling.traffic_key(workload, kernel))
    except (OSError, ValueError):
        return None
    if not t or t.get("kernel_code_sha256") != profiling.kernel_code_hash(kernel):
        return None
    return t


def traffic_for(workload: str, schedule: str):
    """HBM bytes per launch from the committed counter runs, or None."""
    t = counter_record(workload, schedule)
    return t.get("hbm_bytes_per_launch") if t else None


def mfma_busy_for(workload: str, schedule: str):
    """MFMA-busy fraction and clock of the committed counter run, or None."""
    t = counter_record(workload, schedule)
    if not t or "mfma_busy" not in t:
        return None
    return {"mfma_busy": t["mfma_busy"], "clock_GHz": t["clock_GHz"], "source": "profiles/traffic.json"}


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(mib: int) -> int:
    """Ten device-to-device copies of a known size: reading the HBM byte
    counters over these gives the factor that turns counter readings into bytes."""
    import torch

    n = mib * 2 ** 20 // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "copies": 10}))
    return 0


def settle(launch, stream, min_ms: float, max_ms: float):
    """Untimed launches until the GPU clock has settled, whatever --warmup asks.

    A GPU that sat idle (while the host generated the inputs) starts at
    another clock than the one it holds under sustained load: the first tens
    of milliseconds of launches run up to ~25 % slow.  Launches go in chunks
    of about 20 ms of GPU time, each timed with HIP events on the launch
    stream; settling ends once at least ``min_ms`` of GPU time has run and
    the latest chunk's per-launch time is no more than 0.5 % below the best
    earlier chunk (the time has stopped falling), or after ``max_ms``.
    Returns (GPU milliseconds, launches, per-launch ms of the last chunk)."""
    import torch

    if max_ms <= 0:
        return 0.0, 0, None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(4):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    total, n = e0.elapsed_time(e1), 4
    per = max(1, int(math.ceil(20.0 / max(total / 4, 1e-3))))
    best = last = None
    while total < max_ms:
        e0.record(stream)
        for i in range(per):
            launch(n + i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        total += ms
        n += per
        last = ms / per
        if best is not None and total >= min_ms and last >= 0.995 * best:
            break
        best = last if best is None else min(best, last)
    return total, n, last


def bench_attention(a, w) -> int:
    """One attention_fwd launch per step over the whole (B, H) batch."""
    import numpy as np
    import torch

    import matrix_core_scheduling_amd as mcs

    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    dev = torch.device("cuda:0")
    set_bytes = 2 * w.B * w.H * w.D * (w.Sq + 2 * w.Sk)
    nrot = max(1, math.ceil(2 * MALL_BYTES / set_bytes))
    print(f"[bench] workload {w.name}: generating {nrot} input sets", file=sys.stderr, flush=True)

    def to_dev(bits):
        return torch.from_numpy(bits.reshape(-1).view(np.int16)).to(dev).view(tdt)

    host0, sets = None, []
    for r in range(nrot):
        q, k, v = w.operands(r)
        if r == 0:
            host0 = (q, k, v)
        sets.append(tuple(to_dev(x) for x in (q, k, v)))
    outs = [torch.empty(w.B * w.H * w.Sq * w.D, dtype=tdt, device=dev) for _ in range(nrot)]
    lses = [torch.empty(w.B * w.H * w.Sq, dtype=torch.float32, device=dev) for _ in range(nrot)]
    dtype = {"f16": mcs.GEMM_DTYPE_F16, "bf16": mcs.GEMM_DTYPE_BF16}[w.dtype]
    scheds = {"auto": mcs.GEMM_SCHED_PIPELINED, "pipelined": mcs.GEMM_SCHED_PIPELINED,
              "in_phase": mcs.GEMM_SCHED_IN_PHASE, "interleaved": mcs.GEMM_SCHED_INTERLEAVED}
    if a.schedule not in scheds:
        print("attention runs the pipelined (8 waves, groups one stage apart), in_phase or interleaved "
              "(4 waves) schedule", file=sys.stderr)
        return 2
    sched = scheds[a.schedule]
    sched_name = {mcs.GEMM_SCHED_PIPELINED: "pipelined", mcs.GEMM_SCHED_IN_PHASE: "in_phase",
                  mcs.GEMM_SCHED_INTERLEAVED: "interleaved"}[sched]
    # counter records: the 8-wave kernel's (either offset) and the 4-wave kernel's
    prof = "attention4" if sched == mcs.GEMM_SCHED_INTERLEAVED else "attention"
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def launch(i):
        Q, K, V = sets[i % nrot]
        st = mcs.attention_fwd_ex(dtype, w.B, w.H, w.Sq, w.Sk, w.D, Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                  outs[i % nrot].data_ptr(), lses[i % nrot].data_ptr(), w.scale, int(w.causal),
                                  sched, sh)
        if st != mcs.GEMM_OK:
            raise mcs.GemmError(st, "attention_fwd")

    settle_ms, settle_n, settle_last = settle(launch, stream, a.settle_ms, a.settle_max_ms)
    print(f"[bench] settled: {settle_n} launches, {settle_ms:.1f} ms of GPU time; warm-up {a.warmup}",
          file=sys.stderr, flush=True)
    for i in range(a.warmup):
        launch(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(a.steps):
        launch(a.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / a.steps
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    launch(0)
    torch.cuda.synchronize()

    cpu = check = None
    if not a.no_cpu_baseline:
        import oracle.attention as at

        q, k, v = host0
        threads = host_threads()
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        # the oracle on query rows of the first heads: probe, then a ~cpu_seconds sample
        for _ in range(2):               # the second call is timed (the first loads the oracle)
            t = time.perf_counter()
            at.attention(q[:1, :1], k[:1, :1], v[:1, :1], w.dtype, w.scale, w.causal, rows=np.arange(128))
            per_head = max(time.perf_counter() - t, 1e-3)
        heads = int(max(1, min(w.B * w.H, a.cpu_seconds / per_head)))
        # with every head in the sample, widen the row sample to fill the time budget
        extra = int(max(64, min(w.Sq, 128 * a.cpu_seconds / (per_head * heads)) - 64))
        rng = np.random.default_rng(w.seed)
        rows = np.unique(np.concatenate([np.arange(64), rng.integers(0, w.Sq, extra)]))
        hb = [(h // w.H, h % w.H) for h in range(heads)]
        print(f"[bench] CPU oracle on {rows.size} query rows x {heads} heads", file=sys.stderr, flush=True)
        t = time.perf_counter()
        refs = [at.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], w.dtype, w.scale,
                             w.causal, rows=rows) for b, h in hb]
        cpu_s = time.perf_counter() - t
        mask = at.allowed_keys(w.Sq, w.Sk, w.causal)[rows]
        flops = 4.0 * heads * mask.sum() * w.D
        cpu = {"value": round(flops / cpu_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"{rows.size} query rows (rows 0-63 and seeded random ones) of each of the first "
                         f"{heads} (batch, head) pairs of the same workload, {cpu_s:.1f} s on {cpu_model()}"}
        import oracle

        og = outs[0].view(w.B, w.H, w.Sq, w.D).cpu().view(torch.int16).numpy().view(np.uint16)
        og = oracle.decode(og, w.dtype)
        lg = lses[0].view(w.B, w.H, w.Sq).cpu().double().numpy()
        bad = 0
        for (b, h), (oref, lref, aa, sabs) in zip(hb, refs):
            bad += int((~at.within_tolerance(og[b:b + 1, h:h + 1, rows], oref, aa, sabs, w.D, w.Sk,
                                             w.dtype)).sum())
            bad += int((~at.lse_within_tolerance(lg[b:b + 1, h:h + 1, rows], lref, sabs, w.D, w.Sk)).sum())
        n = heads * rows.size * (w.D + 1)
        check = {"rows": heads * rows.size, "elements": n, "outside_tolerance": bad, "pass": bad == 0}

    traffic = traffic_for(w.name, prof)
    peak = PEAK_TFLOPS[w.dtype]
    name = {"f16": "FP16", "bf16": "BF16"}[w.dtype]
    line = {
        "metric": f"{name} attention forward TFLOP/s at B={w.B},H={w.H},Sq={w.Sq},Sk={w.Sk},D={w.D}"
                  f"{',causal' if w.causal else ''} and % of MI355X MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "D": w.D,
                   "causal": w.causal, "operands": w.dtype, "accumulate": "f32", "values": w.dist,
                   "seed": w.seed, "rotating_sets": nrot, "kernel": "attention",
                   "schedule": sched_name},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "wall_s_timed": round(wall, 4),
        "settle_ms": round(settle_ms, 2),
        "settle_launches": settle_n,
        "settled_ms_per_launch": None if settle_last is None else round(settle_last, 6),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic,
                     "mfma_busy": mfma_busy_for(w.name, prof)},
        "cpu_baseline": cpu,
        "check": check,
    }
    print(json.dumps(line), flush=True)
    return 0 if (check is None or check["pass"]) else 3


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 1,000 untimed and 1,000 timed launches, as the pages' FlyDSL/HIP comparison does
    # ("Porting High-Performance HIP Kernels to FlyDSL", section "Results"); a fresh
    # process needs tens of milliseconds of work before the clock settles.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default=si.HEADLINE, choices=sorted(si.WORKLOADS) + sorted(si.ATTN_WORKLOADS))
    ap.add_argument("--schedule", default="auto", choices=["auto", "pipelined", "in_phase", "interleaved", "tile128", "generic"])
    ap.add_argument("--splits", default="auto",
                    help="K-slices (gemm_ex_splitk) or 'auto' (gemm_splitk_suggest; 1 for the default shape)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed GPU time run before the warm-up, whatever --warmup says (clock settling)")
    ap.add_argument("--settle-max-ms", type=float, default=3000.0,
                    help="upper bound of the settling period (0 disables it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM, run 10 device copies of MIB MiB (calibrates HBM byte counters)")
    a = ap.parse_args(argv)
    if a.copy_calibration:
        return copy_calibration(a.copy_calibration)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this GEMM runs on a single MI355X and nothing here "
              "shards it across GPUs (run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import matrix_core_scheduling_amd as mcs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if not os.path.exists(mcs.LIBRARY):
        from matrix_core_scheduling_amd import build
        build.build()
    mcs.load()
    if a.workload in si.ATTN_WORKLOADS:
        return bench_attention(a, si.ATTN_WORKLOADS[a.workload])

    w = si.WORKLOADS[a.workload]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[w.dtype]
    set_bytes = w.elem_bytes * (w.M * w.K + w.K * w.N)
    nrot = max(1, math.ceil(2 * MALL_BYTES / set_bytes))
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: generating {nrot} rotating input sets", file=sys.stderr, flush=True)

    def to_dev(bits):
        raw = bits.reshape(-1)
        raw = raw if w.dtype == "fp8" else raw.view(np.int16)
        return torch.from_numpy(raw).to(dev).view(tdt)

    host0 = None
    sets = []
    for r in range(nrot):
        ab, bb = w.operands(r)
        if r == 0:
            host0 = (ab, bb)
        sets.append((to_dev(ab), to_dev(bb)))
        del ab, bb
    cdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[w.out_type]
    outs = [torch.empty(w.M * w.N, dtype=cdt, device=dev) for _ in range(nrot)]
    out_type = {"same": mcs.GEMM_OUT_SAME, "f32": mcs.GEMM_OUT_F32, "bf16": mcs.GEMM_OUT_BF16}[w.out]
    dtype = {"f16": mcs.GEMM_DTYPE_F16, "bf16": mcs.GEMM_DTYPE_BF16, "fp8": mcs.GEMM_DTYPE_FP8_E4M3}[w.dtype]
    sched = {"auto": mcs.GEMM_SCHED_AUTO, "pipelined": mcs.GEMM_SCHED_PIPELINED,
             "in_phase": mcs.GEMM_SCHED_IN_PHASE, "interleaved": mcs.GEMM_SCHED_INTERLEAVED,
             "tile128": mcs.GEMM_SCHED_TILE128, "generic": mcs.GEMM_SCHED_GENERIC}[a.schedule]
    # the kernel that runs (AUTO picks by the number of output tiles)
    eff = a.schedule
    if a.schedule == "auto":
        eff = "tile128" if mcs.gemm_auto_schedule(w.M, w.N) == mcs.GEMM_SCHED_TILE128 else "pipelined"
    eff_sched = {"pipelined": mcs.GEMM_SCHED_PIPELINED, "in_phase": mcs.GEMM_SCHED_IN_PHASE,
                 "interleaved": mcs.GEMM_SCHED_INTERLEAVED, "tile128": mcs.GEMM_SCHED_TILE128,
                 "generic": mcs.GEMM_SCHED_GENERIC}[eff]
    lda, ldb, ldc = w.K, (w.K if w.trans_b else w.N), w.N
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    fn = {"f16": mcs.load().gemm_f16, "bf16": mcs.load().gemm_bf16, "fp8": mcs.load().gemm_fp8}[w.dtype]
    splits = (mcs.gemm_splitk_suggest(dtype, w.M, w.N, w.K, 0) if a.splits == "auto" else int(a.splits))
    ws_bytes = mcs.gemm_splitk_workspace_bytes(dtype, w.M, w.N, w.K, splits) if splits > 1 else 0
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def launch(i):
        A, B = sets[i % nrot]
        C = outs[i % nrot]
        if splits > 1:
            st = mcs.gemm_ex_splitk(dtype, w.M, w.N, w.K, A.data_ptr(), lda, B.data_ptr(), ldb, w.trans_b,
                                    C.data_ptr(), ldc, out_type, sched, splits, ws.data_ptr(), ws_bytes, sh)
        elif sched == mcs.GEMM_SCHED_AUTO:
            st = fn(w.M, w.N, w.K, A.data_ptr(), lda, B.data_ptr(), ldb, w.trans_b, C.data_ptr(), ldc,
                    out_type, sh)
        else:
            st = mcs.gemm_ex(dtype, w.M, w.N, w.K, A.data_ptr(), lda, B.data_ptr(), ldb, w.trans_b,
                             C.data_ptr(), ldc, out_type, sched, sh)
        if st != mcs.GEMM_OK:
            raise mcs.GemmError(st, "launch")

    settle_ms, settle_n, settle_last = settle(launch, stream, a.settle_ms, a.settle_max_ms)
    print(f"[bench] settled: {settle_n} launches, {settle_ms:.1f} ms of GPU time; warm-up {a.warmup}",
          file=sys.stderr, flush=True)
    for i in range(a.warmup):
        launch(i)
    torch.cuda.synchronize()

    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(a.steps):
        launch(a.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / a.steps
    tflops = w.flops / (ms_step * 1e-3) / 1e12

    # five more batches of >= ~50 ms, median of their per-launch means (stability)
    per = max(1, int(math.ceil(50.0 / max(ms_step, 1e-3))))
    batch_ms = []
    for b in range(5):
        x0 = torch.cuda.Event(enable_timing=True)
        x1 = torch.cuda.Event(enable_timing=True)
        x0.record(stream)
        for i in range(per):
            launch(i + b)
        x1.record(stream)
        torch.cuda.synchronize()
        batch_ms.append(x0.elapsed_time(x1) / per)
    batch_med = float(np.median(batch_ms))

    # result of set 0 for the check below (same launch configuration)
    launch(0)
    torch.cuda.synchronize()
    info = mcs.gemm_kernel_info(dtype, w.trans_b, out_type, eff_sched)

    cpu = None
    check = None
    if not a.no_cpu_baseline:
        import oracle

        ab, bb = host0
        threads = host_threads()
        # time per call = fixed cost (widening B) + rows x per-row cost: two probes
        probe = []
        for r in (threads, 3 * threads):
            t = time.perf_counter()
            oracle.gemm(ab, bb, w.dtype, w.trans_b, rows=(0, r), nthreads=threads, with_sabs=False)
            probe.append(time.perf_counter() - t)
        per_row = max((probe[1] - probe[0]) / (2 * threads), 1e-6)
        fixed = max(probe[0] - threads * per_row, 0.0)
        rows = int(min(w.M, max(2 * threads, (a.cpu_seconds - 2 * fixed) / per_row)))
        rows = max(2, rows - rows % 2)
        half = rows // 2
        blocks = [(0, half), (w.M - half, w.M)]
        print(f"[bench] CPU oracle on {rows} rows with {threads} threads", file=sys.stderr, flush=True)
        t = time.perf_counter()
        refs = [oracle.gemm(ab, bb, w.dtype, w.trans_b, rows=blk, nthreads=threads) for blk in blocks]
        cpu_s = time.perf_counter() - t
        cpu = {"value": round(2.0 * rows * w.N * w.K / cpu_s / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"output rows [0,{half}) and [{w.M - half},{w.M}) of the same product "
                         f"({rows}x{w.N}x{w.K}), {cpu_s:.1f} s on {cpu_model()}"}
        Cg = outs[0].view(w.M, w.N).cpu()
        if w.out_type == "f32":
            cg = Cg.double().numpy()
        else:
            cg = oracle.decode(Cg.view(torch.int16).numpy().view(np.uint16), w.out_type)
        bad = 0
        for (r0, r1), (cref, sabs) in zip(blocks, refs):
            bad += int((~oracle.within_tolerance(cg[r0:r1], cref, sabs, out=w.out_type)).sum())
        check = {"rows": rows, "elements": rows * w.N, "outside_tolerance": bad, "pass": bad == 0}

    traffic = traffic_for(w.name, eff)
    peak = PEAK_TFLOPS[w.dtype]
    metric = METRIC if w.name == si.HEADLINE else (
        f"{ {'f16': 'FP16', 'bf16': 'BF16', 'fp8': 'FP8 E4M3'}[w.dtype]} GEMM TFLOP/s at "
        f"M={w.M},N={w.N},K={w.K} and % of MI355X MFMA peak")
    line = {
        "metric": metric,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGES_TFLOPS[w.name], 4) if w.name in PAGES_TFLOPS else None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "operands": w.dtype,
                   "accumulate": "f32", "out": w.out_type,
                   "b_layout": "N x K row-major" if w.trans_b else "K x N row-major",
                   "values": w.dist, "seed": w.seed, "rotating_sets": nrot,
                   "schedule": a.schedule, "kernel": eff, "splits": splits},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "pct_of_unit_peak": round(100.0 * tflops / PEAK_TFLOPS_UNITS[w.dtype], 2),
        "batch_median_ms": round(batch_med, 6),
        "wall_s_timed": round(wall, 4),
        "settle_ms": round(settle_ms, 2),
        "settle_launches": settle_n,
        "settled_ms_per_launch": None if settle_last is None else round(settle_last, 6),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic,
                     "mfma_busy": mfma_busy_for(w.name, eff)},
        "kernel": {"vgprs": info["num_regs"], "scratch_bytes_per_lane": info["local_bytes"],
                   "lds_bytes": info["shared_bytes"], "threads": info["block_threads"]},
        "cpu_baseline": cpu,
        "check": check,
    }
    print(json.dumps(line), flush=True)
    return 0 if (check is None or check["pass"]) else 3


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the gfx950 dense BF16 GEMM C = A * B^T (libhkg.so).

One step = one call of hkg_gemm_bf16 on the square workload
(8192 x 8192 x 8192, A and B uniform in [-1, 1] rounded to bf16, seed 0),
inputs resident in HBM.  Prints ONE JSON line on stdout:

  value        TFLOP/s over the timed steps (2 M N K per step)
  roofline     the tile kernel against the 2.5 PFLOP/s dense bf16 MFMA peak
  decode       the M = 16 decode GEMM (16 x 4096 x 4096, N(0,1) activations,
               N(0, 0.02) weights) as HBM GB/s against 8 TB/s, timed over
               buffer sets rotated across 2x the 256 MB last-level cache so
               every launch streams B from HBM
  cpu_baseline the CPU oracle (fp64, OpenMP) on a bounded row sample of the
               square workload, scaled to TFLOP/s
  epilogue     the same two workloads with a fused bias + GELU (square) and
               bias + SiLU (decode) epilogue
  vendor_context  torch.mm (hipBLASLt) on the same inputs with the same
               timing, for comparison across machines whose clocks differ
  grouped      the grouped (mixture-of-experts) GEMM on the uniform and ragged
               MoE workloads (TFLOP/s of the experts' rows, 2 sum(M_g) N K per
               call), with torch._grouped_mm for context
  layouts      square_8192 with the weight in column layout (x @ W, W stored
               K x N: "NN") and with both operands in column layout ("TN"), through
               hkg_gemm_bf16_ex (per-call transpose of the column operands),
               and the transpose pass alone (GB/s); torch.mm on the same views
               for context
  other_configs  the tiny, MLP-up (128 x 12288 x 4096) and prefill-down
               (4096 x 4096 x 12288) workloads in the planner's configuration,
               per call over rotating buffer sets (graph), torch.mm for context
  middle       the compute-bound middle (1024 and 2048 x 4096 x 4096: too few
               256 x 256 tiles to fill the device), timed as other_configs
  mxfp8        the block-scaled FP8 GEMM (E4M3, E8M0 scale per 32 k) on
               mx_square_8192 (TFLOP/s against the 5.0 PFLOP/s dense fp8
               MFMA peak) and mx_decode_32x4096x4096 (HBM GB/s, rotating
               buffers), with scales packed once (the kernel) and per call
               (hkg_gemm_mxfp8 with natural-layout scales); torch._scaled_mm
               with one scale per tensor for context
  mxfp4        the block-scaled FP4 GEMM (E2M1 two per byte, E8M0 scale per
               32 k) on mx4_square_8192 (TFLOP/s against the 10.1 PFLOP/s
               dense fp4 MFMA peak) and mx4_decode_32x14336x4096 (HBM GB/s,
               rotating buffers), packed scales and per-call packing

Progress and diagnostics go to stderr.  Timing uses HIP events on the stream
the kernels are launched on (torch's current stream), bracketed by device
synchronisation.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BF16 GEMM TFLOP/s @8192³ (% of 2.5 PF) + HBM GB/s @M=16 decode (% of 8 TB/s)"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0           # MI355X dense fp8 MFMA
PEAK_FP4_TFLOPS = 10100.0          # MI355X dense fp4 MFMA
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E
LLC_BYTES = 256 * 2**20
# HipKittens' best 8192^3 BF16 GEMM on MI355X (talk notes, Table 2).
PAGES_8192_TFLOPS = 1610.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def source_digest(fname):
    with open(os.path.join(ROOT, "tile_level_dense_amd", "csrc", fname), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM-side bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE scaled by a reference
    copy), if they were taken on that kernel and its current source; else
    None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get("workloads", {}).get(workload)
    if not e or e.get("kernel") != kernel or e.get("source_digest") != source_digest(e.get("source", "")):
        return None
    return e.get("bytes_per_launch")


# Untimed graph replays before a graph-timed leg: at least 50 (hundreds of
# launches, several milliseconds), so a memory-bound leg that follows the
# MFMA-bound square leg is not timed while the clocks are still settling
# (with 6 replays the first graph-timed decode leg read ~8% slower than the
# same kernel timed on its own).
def graph_warmup(warmup, sets):
    return max(50, warmup // sets)


# Timing protocol of every leg: W warm-up calls, then an untimed clock-settle
# period of back-to-back calls (SETTLE_S seconds of device time: the engine
# clock needs a few hundred milliseconds of sustained load to reach its
# loaded level, and a 5-launch warm-up timed the ramp, ~10% slow at 8192^3),
# then WINDOWS windows of K calls each, every window bracketed by device
# synchronisation and timed with HIP events on the stream the calls are
# launched on; the leg's figure is the median window.  Engine and memory
# clocks and socket power are sampled from the start of the settle period to
# the end of the windows (amdsmi's metrics table, refreshed by the firmware
# about once a second; null where unavailable or not refreshed meanwhile).
# The 8192^3 legs settle SQUARE_SETTLE x longer (1.2 s by default), so a
# refresh falls while they run and their clocks are those of the loaded GPU.
SETTLE_S = 0.5
SQUARE_SETTLE = 2.4
WINDOWS = 5
TIMINGS = {}


class ClockSampler:
    """Background sampling of the GPU's engine clock, memory clock, socket
    power and activity through amdsmi's metrics table (optional: every
    failure leaves the figures null).  The firmware refreshes that table
    about once a second, so a leg's figures come only from refreshes made
    while the leg was running (a reading from before it would show the idle
    clock); the engine clock is the mean over the XCDs."""

    def __init__(self):
        self.handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if handles:
                self.amdsmi = amdsmi
                self.handle = handles[0]
                self.read()
        except Exception as ex:            # noqa: BLE001 - clocks are context only
            log("clock sampling unavailable: %s" % str(ex)[:120])
            self.handle = None
        self.samples = []
        self._thread = None
        self._stop = None

    def read(self):
        """(engine MHz, memory MHz, gfx activity %, socket W, firmware timestamp)."""
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)

        def num(v):
            return v if isinstance(v, (int, float)) and v != 0xFFFF else None
        xcd = [num(v) for v in (m.get("current_gfxclks") or [])]
        xcd = [v for v in xcd if v is not None]
        sclk = float(np.mean(xcd)) if xcd else num(m.get("current_gfxclk"))
        return (sclk, num(m.get("current_uclk")), num(m.get("average_gfx_activity")),
                num(m.get("current_socket_power")), m.get("firmware_timestamp"))

    def activity(self, n=5, gap_s=0.02):
        """gfx activity % over n samples with nothing of ours running (idle check)."""
        if self.handle is None:
            return None
        out = []
        for _ in range(n):
            try:
                out.append(self.read()[2])
            except Exception:              # noqa: BLE001
                return None
            time.sleep(gap_s)
        return out

    def start(self):
        self.samples = []
        if self.handle is None:
            return
        import threading
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    self.samples.append(self.read())
                except Exception:          # noqa: BLE001
                    return
                self._stop.wait(0.01)
        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        if not self.samples:
            return None
        # keep the refreshes made after sampling began (the first reading's
        # firmware timestamp marks a table filled before the leg)
        first_ts = self.samples[0][4]
        fresh = [x for x in self.samples if x[4] is not None and x[4] != first_ts]
        refreshes = len(set(x[4] for x in fresh))
        if not fresh:
            return dict(samples=len(self.samples), metric_refreshes=0, sclk_mhz_median=None,
                        note="no metrics refresh while the leg ran")
        sc = [x[0] for x in fresh if x[0] is not None]
        mc = [x[1] for x in fresh if x[1] is not None]
        pw = [x[3] for x in fresh if x[3] is not None]
        return dict(samples=len(fresh), metric_refreshes=refreshes,
                    sclk_mhz_median=round(float(np.median(sc)), 1) if sc else None,
                    sclk_mhz_min=round(float(min(sc)), 1) if sc else None,
                    sclk_mhz_max=round(float(max(sc)), 1) if sc else None,
                    mclk_mhz_median=float(np.median(mc)) if mc else None,
                    socket_power_w_median=float(np.median(pw)) if pw else None)


CLOCKS = None


def time_launches(torch, fn, steps, warmup, label=None, per_call=1, settle_s=None):
    """Median ms per fn() over WINDOWS windows of `steps` calls each, after
    `warmup` calls and settle_s (default SETTLE_S) seconds of untimed calls;
    per_call divides (fn launching that many GEMMs, e.g. a graph over
    rotating buffers).  Clocks are sampled from the start of the settle
    calls to the end of the windows, the load being steady throughout."""
    settle_s = SETTLE_S if settle_s is None else settle_s
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    # Estimate one call's device time, then settle the clocks.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    fn()
    stop.record()
    torch.cuda.synchronize()
    est_ms = max(start.elapsed_time(stop), 1e-3)
    settle = int(min(200000, max(1, np.ceil(settle_s * 1e3 / est_ms))))
    if CLOCKS is not None:
        CLOCKS.start()
    done = 0
    while done < settle:
        chunk = min(settle - done, max(1, int(20.0 / est_ms)))     # ~20 ms between host syncs
        for _ in range(chunk):
            fn()
        done += chunk
        torch.cuda.synchronize()
    wins = []
    for _ in range(WINDOWS):
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        wins.append(start.elapsed_time(stop) / steps / per_call)
    clk = CLOCKS.stop() if CLOCKS is not None else None
    med = float(np.median(wins))
    if label:
        TIMINGS[label] = dict(ms_per_call_median=round(med, 6), windows=[round(w, 6) for w in wins],
                              calls_per_window=steps * per_call, warmup_calls=warmup * per_call,
                              settle_calls=settle * per_call, settle_ms=round(settle * est_ms, 1),
                              spread_pct=round(100.0 * (max(wins) - min(wins)) / med, 2), clocks=clk)
    return med


def bench_square(torch, hkg, steps, warmup):
    import workloads
    name = "square_8192"
    w = workloads.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    log("generating %s inputs" % name)
    A, B = workloads.workload_inputs(name)
    a, b = to_dev(A, torch), to_dev(B, torch)
    del A, B
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    plan = hkg.plan(M, N, K)
    log("plan", plan.kernel_name.decode(), plan.reason.decode())
    ms = time_launches(torch, lambda: hkg.gemm(a, b, out=c), steps, warmup, label="square",
                       settle_s=SQUARE_SETTLE * SETTLE_S)
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    log("square: %.3f ms/step, %.1f TFLOP/s" % (ms, tflops))
    # Fused epilogue (bias + GELU, one bias value per column) on the same
    # inputs: its cost over the plain GEMM.
    bias = torch.linspace(-1.0, 1.0, N, device="cuda").to(torch.bfloat16)
    ms_e = time_launches(torch, lambda: hkg.gemm(a, b, out=c, bias=bias, epilogue="bias_gelu"), steps, warmup,
                         label="square_bias_gelu", settle_s=SQUARE_SETTLE * SETTLE_S)
    log("square with bias+GELU epilogue: %.3f ms/step, %.1f TFLOP/s" % (ms_e, flops / (ms_e * 1e-3) / 1e12))
    # Context only: the vendor library on the same inputs, same protocol.
    ms_v = time_launches(torch, lambda: torch.mm(a, b.t(), out=c), steps, warmup, label="square_torch_mm",
                         settle_s=SQUARE_SETTLE * SETTLE_S)
    tflops_v = flops / (ms_v * 1e-3) / 1e12
    log("square, torch.mm (hipBLASLt) for context: %.3f ms/step, %.1f TFLOP/s" % (ms_v, tflops_v))
    # Context: the same kernel on constant operands (every element 0.01147),
    # where the matrix cores switch little and draw less power, so the engine
    # clock stays higher; the gap to the uniform [-1, 1] inputs above is the
    # power limit, not the schedule.
    ac = torch.full((M, K), 0.01147, dtype=torch.bfloat16, device="cuda")
    bc = torch.full((N, K), 0.01147, dtype=torch.bfloat16, device="cuda")
    ms_c = time_launches(torch, lambda: hkg.gemm(ac, bc, out=c), steps, warmup, label="square_constant_inputs",
                         settle_s=SQUARE_SETTLE * SETTLE_S)
    del ac, bc
    log("square on constant inputs (power context): %.3f ms/step, %.1f TFLOP/s" % (ms_c, flops / (ms_c * 1e-3) / 1e12))
    return dict(M=M, N=N, K=K, ms=ms, tflops=tflops, flops=flops, plan=plan, vendor_tflops=tflops_v,
                epi_ms=ms_e, epi_tflops=flops / (ms_e * 1e-3) / 1e12, const_tflops=flops / (ms_c * 1e-3) / 1e12)


def bench_decode(torch, hkg, steps, warmup):
    import workloads
    name = "decode_16x4096x4096"
    w = workloads.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    A, B = workloads.workload_inputs(name)
    alg_bytes = 2.0 * (M * K + N * K + M * N)
    per_set = 2 * (M * K + N * K + M * N)
    sets = int(np.ceil(2 * LLC_BYTES / per_set))
    a0, b0 = to_dev(A, torch), to_dev(B, torch)
    bufs = [(a0.clone(), b0.clone(), torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))
            for _ in range(sets)]
    plan = hkg.plan(M, N, K)
    log("decode plan", plan.kernel_name.decode(), "rotating over %d buffer sets (%.0f MiB)"
        % (sets, sets * per_set / 2**20))
    # Capture one pass over all sets in a graph so host launch cost does not
    # pace the ~microsecond kernels; replays run the launches back to back.
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for a, b, c in bufs:                      # warm the code path outside capture
            hkg.gemm(a, b, out=c)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for a, b, c in bufs:
            hkg.gemm(a, b, out=c)
    reps = max(1, steps // sets)
    ms_rot = time_launches(torch, graph.replay, reps, graph_warmup(warmup, sets), label="decode", per_call=sets)
    # Hot buffers (B resident in the last-level cache) for context.
    a, b, c = bufs[0]
    graph_hot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_hot, stream=stream):
        for _ in range(sets):
            hkg.gemm(a, b, out=c)
    ms_hot = time_launches(torch, graph_hot.replay, reps, graph_warmup(warmup, sets), label="decode_llc_resident",
                            per_call=sets)
    gbps = alg_bytes / (ms_rot * 1e-3) / 1e9
    gbps_hot = alg_bytes / (ms_hot * 1e-3) / 1e9
    # Fused bias + SiLU epilogue over the same rotating buffers.
    bias = torch.linspace(-1.0, 1.0, N, device="cuda").to(torch.bfloat16)
    with torch.cuda.stream(stream):
        for a, b, c in bufs:
            hkg.gemm(a, b, out=c, bias=bias, epilogue="bias_silu")
    torch.cuda.synchronize()
    graph_e = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_e, stream=stream):
        for a, b, c in bufs:
            hkg.gemm(a, b, out=c, bias=bias, epilogue="bias_silu")
    ms_e = time_launches(torch, graph_e.replay, reps, graph_warmup(warmup, sets), label="decode_bias_silu",
                         per_call=sets)
    log("decode with bias+SiLU epilogue: %.2f us/call rotating (%.0f GB/s)"
        % (ms_e * 1e3, (alg_bytes + 2 * N) / (ms_e * 1e-3) / 1e9))
    log("decode: %.2f us/call rotating (%.0f GB/s), %.2f us hot (%.0f GB/s)"
        % (ms_rot * 1e3, gbps, ms_hot * 1e3, gbps_hot))
    # Context only: the vendor library over the same rotating buffers.
    with torch.cuda.stream(stream):
        for a, b, c in bufs:
            torch.mm(a, b.t(), out=c)
    torch.cuda.synchronize()
    graph_v = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_v, stream=stream):
        for a, b, c in bufs:
            torch.mm(a, b.t(), out=c)
    ms_v = time_launches(torch, graph_v.replay, reps, graph_warmup(warmup, sets), label="decode_torch_mm",
                         per_call=sets)
    gbps_v = alg_bytes / (ms_v * 1e-3) / 1e9
    log("decode, torch.mm (hipBLASLt) for context: %.2f us/call rotating (%.0f GB/s)" % (ms_v * 1e3, gbps_v))
    # Launch floor of a per-call figure: back-to-back launches of a kernel
    # that does almost nothing (a one-element fill), captured in a graph the
    # same way.  A call can take no less than this plus its bytes at the HBM
    # peak, which caps the per-call rate of this workload.
    tiny = torch.zeros(1, device="cuda")
    graph_f = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_f, stream=stream):
        for _ in range(sets):
            tiny.fill_(1.0)
    ms_f = time_launches(torch, graph_f.replay, reps, graph_warmup(warmup, sets), label="launch_floor", per_call=sets)
    cap = alg_bytes / ((ms_f * 1e-3) + alg_bytes / (PEAK_HBM_GBPS * 1e9)) / 1e9
    log("launch floor %.2f us per graph launch: a per-call decode reaches at most %.0f GB/s (%.1f%% of 8 TB/s)"
        % (ms_f * 1e3, cap, 100 * cap / PEAK_HBM_GBPS))
    # Context: a plain device copy moving the same bytes per call (half of
    # them read, half written) over rotating buffers, graph-launched the same
    # way: what a streaming kernel of this size reaches per call here.
    half = per_set // 4                          # bf16 elements: half the bytes read, half written
    copies = [(torch.empty(half, dtype=torch.bfloat16, device="cuda").fill_(1.0),
               torch.empty(half, dtype=torch.bfloat16, device="cuda")) for _ in range(sets)]
    with torch.cuda.stream(stream):
        for src, dst in copies:
            dst.copy_(src)
    torch.cuda.synchronize()
    graph_c = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_c, stream=stream):
        for src, dst in copies:
            dst.copy_(src)
    ms_c = time_launches(torch, graph_c.replay, reps, graph_warmup(warmup, sets), label="decode_copy_same_bytes",
                         per_call=sets)
    gbps_c = 4.0 * half / (ms_c * 1e-3) / 1e9
    log("copy of the same bytes per call (torch copy_, context): %.2f us/call (%.0f GB/s)" % (ms_c * 1e3, gbps_c))
    del copies
    return dict(M=M, N=N, K=K, ms=ms_rot, gbps=gbps, gbps_hot=gbps_hot, ms_hot=ms_hot,
                alg_bytes=alg_bytes, sets=sets, plan=plan, launches=reps * sets, vendor_gbps=gbps_v,
                epi_ms=ms_e, epi_gbps=(alg_bytes + 2 * N) / (ms_e * 1e-3) / 1e9, floor_us=ms_f * 1e3,
                floor_cap_gbps=cap, copy_us=ms_c * 1e3, copy_gbps=gbps_c)


def mx_to_dev(x, torch):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")


def vendor_fp8(torch, a, b, out):
    """torch._scaled_mm on the same E4M3 codes with unit per-tensor scales
    (not block-scaled; context only), or None where unsupported."""
    one = torch.ones((), device="cuda")
    af, bf = a.view(torch.float8_e4m3fn), b.view(torch.float8_e4m3fn)
    try:
        torch._scaled_mm(af, bf.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
    except Exception as ex:              # noqa: BLE001 - context figure only
        log("torch._scaled_mm unavailable: %s" % str(ex)[:100])
        return None
    return lambda: torch._scaled_mm(af, bf.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)


def bench_mx_square(torch, hkg, steps, warmup, fmt="fp8"):
    """The 8192^3 block-scaled workload: MXFP8 (E4M3) or MXFP4 (E2M1, two
    codes per byte)."""
    import workloads
    fp4 = fmt == "fp4"
    name = "mx4_square_8192" if fp4 else "mx_square_8192"
    w = (workloads.MX4_WORKLOADS if fp4 else workloads.MX_WORKLOADS)[name]
    M, N, K = w["M"], w["N"], w["K"]
    log("generating %s inputs" % name)
    A, SA, B, SB = (workloads.mx4_workload_inputs if fp4 else workloads.mx_workload_inputs)(name)
    a, sa, b, sb = (mx_to_dev(x, torch) for x in (A, SA, B, SB))
    del A, SA, B, SB
    pa, pb = hkg.mx_pack_scales(sa, K), hkg.mx_pack_scales(sb, K)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gemm = hkg.gemm_mxfp4 if fp4 else hkg.gemm_mxfp8
    plan = (hkg.mx4_plan if fp4 else hkg.mx_plan)(M, N, K)
    tag = "mx4" if fp4 else "mx"
    log("%s plan" % tag, plan.kernel_name.decode(), plan.reason.decode())
    flops = 2.0 * M * N * K
    ms = time_launches(torch, lambda: gemm(a, pa, b, pb, out=c, packed=True), steps, warmup,
                       label="%s_square" % tag)
    ms_nat = time_launches(torch, lambda: gemm(a, sa, b, sb, out=c), steps, warmup,
                           label="%s_square_per_call_packing" % tag)
    log("%s square: %.3f ms/step (%.1f TFLOP/s) packed scales, %.3f ms with per-call packing"
        % (tag, ms, flops / ms / 1e9, ms_nat))
    ms_v = None
    if not fp4:
        fn = vendor_fp8(torch, a, b, c)
        ms_v = time_launches(torch, fn, steps, warmup, label="mx_square_scaled_mm") if fn else None
        if ms_v:
            log("mx square, torch._scaled_mm per-tensor fp8 for context: %.3f ms (%.1f TFLOP/s)"
                % (ms_v, flops / ms_v / 1e9))
    return dict(name=name, M=M, N=N, K=K, ms=ms, tflops=flops / ms / 1e9, ms_nat=ms_nat,
                tflops_nat=flops / ms_nat / 1e9, flops=flops, plan=plan,
                vendor_tflops=(flops / ms_v / 1e9) if ms_v else None)


def bench_mx_decode(torch, hkg, steps, warmup, fmt="fp8"):
    """The block-scaled decode workload over rotating buffer sets: MXFP8
    (32 x 4096 x 4096) or MXFP4 (32 x 14336 x 4096)."""
    import workloads
    fp4 = fmt == "fp4"
    name = "mx4_decode_32x14336x4096" if fp4 else "mx_decode_32x4096x4096"
    w = (workloads.MX4_WORKLOADS if fp4 else workloads.MX_WORKLOADS)[name]
    M, N, K = w["M"], w["N"], w["K"]
    A, SA, B, SB = (workloads.mx4_workload_inputs if fp4 else workloads.mx_workload_inputs)(name)
    eb = 0.5 if fp4 else 1.0            # bytes per element
    alg_bytes = float(eb * (M * K + N * K) + (M + N) * (K // 32) + 2 * M * N)
    per_set = int(eb * (M * K + N * K)) + (M + N) * (K // 32) * 2 + 2 * M * N
    sets = int(np.ceil(2 * LLC_BYTES / per_set))
    a0, sa0, b0, sb0 = (mx_to_dev(x, torch) for x in (A, SA, B, SB))
    bufs = []
    for _ in range(sets):
        a, sa, b, sb = a0.clone(), sa0.clone(), b0.clone(), sb0.clone()
        bufs.append((a, sa, hkg.mx_pack_scales(sa, K), b, sb, hkg.mx_pack_scales(sb, K),
                     torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
    plan = (hkg.mx4_plan if fp4 else hkg.mx_plan)(M, N, K)
    gemm = hkg.gemm_mxfp4 if fp4 else hkg.gemm_mxfp8
    tag = "mx4" if fp4 else "mx"
    log("%s decode plan" % tag, plan.kernel_name.decode(), plan.reason.decode(), "over %d buffer sets" % sets)
    stream = torch.cuda.Stream()
    reps = max(1, steps // sets)

    def graph_of(call):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for buf in bufs:
                call(*buf)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for buf in bufs:
                call(*buf)
        return g

    g_pk = graph_of(lambda a, sa, pa, b, sb, pb, c: gemm(a, pa, b, pb, out=c, packed=True))
    ms = time_launches(torch, g_pk.replay, reps, graph_warmup(warmup, sets), label="%s_decode" % tag,
                       per_call=sets)
    g_nat = graph_of(lambda a, sa, pa, b, sb, pb, c: gemm(a, sa, b, sb, out=c))
    ms_nat = time_launches(torch, g_nat.replay, reps, graph_warmup(warmup, sets),
                           label="%s_decode_natural_scales" % tag, per_call=sets)
    gbps = alg_bytes / (ms * 1e-3) / 1e9
    log("%s decode: %.2f us/call rotating (%.0f GB/s) packed scales, %.2f us from natural-layout scales"
        % (tag, ms * 1e3, gbps, ms_nat * 1e3))
    ms_v = None
    if not fp4 and vendor_fp8(torch, bufs[0][0], bufs[0][3], bufs[0][6]):
        one = torch.ones((), device="cuda")
        g_v = graph_of(lambda a, sa, pa, b, sb, pb, c: torch._scaled_mm(
            a.view(torch.float8_e4m3fn), b.view(torch.float8_e4m3fn).t(), scale_a=one, scale_b=one,
            out_dtype=torch.bfloat16))
        ms_v = time_launches(torch, g_v.replay, reps, graph_warmup(warmup, sets), label="mx_decode_scaled_mm",
                             per_call=sets)
        log("mx decode, torch._scaled_mm per-tensor fp8 for context: %.2f us" % (ms_v * 1e3))
    return dict(name=name, M=M, N=N, K=K, ms=ms, gbps=gbps, ms_nat=ms_nat, alg_bytes=alg_bytes, sets=sets,
                plan=plan, launches=reps * sets, vendor_us=ms_v * 1e3 if ms_v else None)


ALL_CONFIGS = ("tiny_256", "mlp_up_128x12288x4096", "prefill_down_4096x4096x12288")
MIDDLE_CONFIGS = ("middle_1024x4096x4096", "middle_2048x4096x4096")


def bench_configs(torch, hkg, names=ALL_CONFIGS):
    """The remaining dense workloads (tiny, MLP-up, prefill-down) in the
    planner's launch configuration: per-call time over buffer sets rotated
    across 2x the last-level cache, launches captured in a graph; torch.mm
    over the same buffers for context.  (Prefill-down runs the square
    workload's kernel at another size: a kernel trace of the full run mixes
    the two in that kernel's average; the per-workload traces come from
    --only runs.)"""
    import workloads
    out = {}
    stream = torch.cuda.Stream()
    for name in names:
        w = workloads.WORKLOADS[name] if name in workloads.WORKLOADS else workloads.MIDDLE_WORKLOADS[name]
        M, N, K = w["M"], w["N"], w["K"]
        A, B = workloads.workload_inputs(name)
        a0, b0 = to_dev(A, torch), to_dev(B, torch)
        del A, B
        per_set = 2 * (M * K + N * K + M * N)
        sets = int(min(64, max(2, np.ceil(2 * LLC_BYTES / per_set))))
        bufs = [(a0.clone(), b0.clone(), torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))
                for _ in range(sets)]
        plan = hkg.plan(M, N, K)

        def graph_of(call):
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for a, b, c in bufs:
                    call(a, b, c)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for a, b, c in bufs:
                    call(a, b, c)
            return g

        flops = 2.0 * M * N * K
        est = max(flops / 1.0e15, per_set / 4.0e12, 5e-6)          # rough seconds per call
        # each window: at least 100 calls and ~20 ms of device time
        reps = int(min(200, max(np.ceil(100 / sets), np.ceil(0.02 / (est * sets)))))
        warm = int(max(3, 0.02 / (est * sets)))                    # ~20 ms of untimed replays
        g = graph_of(lambda a, b, c: hkg.gemm(a, b, out=c))
        ms = time_launches(torch, g.replay, reps, warm, label=name, per_call=sets)
        gv = graph_of(lambda a, b, c: torch.mm(a, b.t(), out=c))
        ms_v = time_launches(torch, gv.replay, reps, warm, label=name + "_torch_mm", per_call=sets)
        log("%s: %s, %.2f us/call (%.1f TFLOP/s, %.0f GB/s); torch.mm %.2f us"
            % (name, plan.kernel_name.decode(), ms * 1e3, flops / (ms * 1e-3) / 1e12,
               per_set / (ms * 1e-3) / 1e9, ms_v * 1e3))
        out[name] = dict(us=ms * 1e3, tflops=flops / (ms * 1e-3) / 1e12, gbps=per_set / (ms * 1e-3) / 1e9,
                         kernel=plan.kernel_name.decode(), split_k=plan.split_k, vendor_us=ms_v * 1e3, sets=sets,
                         flops=flops, alg_bytes=float(per_set), launches=reps * sets)
        del bufs, a0, b0
        torch.cuda.empty_cache()
    return out


def bench_grouped(torch, hkg, steps, warmup):
    import workloads
    out = {}
    for name in ("moe_uniform_8x1024_4096x4096", "moe_ragged_16_8192_4096x4096"):
        w = workloads.GROUPED_WORKLOADS[name]
        A, B, offs = workloads.grouped_workload_inputs(name)
        M, K = A.shape
        G, N = B.shape[0], B.shape[1]
        a, b = to_dev(A, torch), to_dev(B, torch)
        o = torch.from_numpy(offs).to("cuda")
        del A, B
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        plan = hkg.grouped_plan(G, M, N, K)
        flops = 2.0 * float(sum(w["sizes"])) * N * K
        ms = time_launches(torch, lambda: hkg.grouped_gemm(a, b, o, out=c), steps, warmup, label=name)
        log("grouped %s: %s, %.3f ms (%.1f TFLOP/s)" % (name, plan.kernel_name.decode(), ms, flops / ms / 1e9))
        ms_v = None
        try:
            bt = b.transpose(1, 2)
            torch._grouped_mm(a, bt, offs=o, out_dtype=torch.bfloat16)
            ms_v = time_launches(torch, lambda: torch._grouped_mm(a, bt, offs=o, out_dtype=torch.bfloat16),
                                 steps, warmup, label=name + "_grouped_mm")
            log("grouped %s, torch._grouped_mm for context: %.3f ms (%.1f TFLOP/s)" % (name, ms_v, flops / ms_v / 1e9))
        except Exception as ex:          # noqa: BLE001 - context figure only
            log("torch._grouped_mm unavailable: %s" % str(ex)[:100])
        out[name] = dict(ms=ms, tflops=flops / ms / 1e9, plan=plan, flops=flops,
                         vendor_tflops=(flops / ms_v / 1e9) if ms_v else None)
        del a, b, c
    return out


def bench_layouts(torch, hkg, steps, warmup):
    import workloads
    A, B = workloads.workload_inputs("square_8192")
    M, K = A.shape
    N = B.shape[0]
    a, b = to_dev(A, torch), to_dev(B, torch)
    del A, B
    at = a.t().contiguous()                 # A stored K x M (column layout)
    bt = b.t().contiguous()                 # B stored K x N (column layout): x @ W
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * M * N * K
    ms_nn = time_launches(torch, lambda: hkg.gemm_ex(a, bt.t(), out=c), steps, warmup, label="layouts_nn")
    ms_tn = time_launches(torch, lambda: hkg.gemm_ex(at.t(), bt.t(), out=c), steps, warmup, label="layouts_tn")
    y = torch.empty_like(b)
    ms_pack = time_launches(torch, lambda: hkg.pack(bt.t()), steps, warmup, label="layouts_transpose")
    ms_v = time_launches(torch, lambda: torch.mm(a, bt, out=c), steps, warmup, label="layouts_nn_torch_mm")
    log("layouts: NN %.3f ms (%.1f TFLOP/s), TN %.3f ms (%.1f), transpose of one operand %.3f ms (%.0f GB/s); "
        "torch.mm NN %.3f ms" % (ms_nn, flops / ms_nn / 1e9, ms_tn, flops / ms_tn / 1e9, ms_pack,
                                 4.0 * N * K / ms_pack / 1e6, ms_v))
    del y
    return dict(nn_tflops=flops / ms_nn / 1e9, tn_tflops=flops / ms_tn / 1e9, nn_ms=ms_nn, tn_ms=ms_tn,
                transpose_ms=ms_pack, transpose_gbps=4.0 * N * K / ms_pack / 1e6, vendor_nn_tflops=flops / ms_v / 1e9)


def calibration_copy(torch, mib=1024):
    """One device-to-device copy of a known size (mib MiB read, mib MiB
    written), the reference dispatch for scaling HBM byte counters."""
    src = torch.empty(mib * 2**20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    # Hand the 2 GiB back to the driver: left in the caching allocator, the
    # legs' buffers are carved out of it, and the rotating decode buffers
    # placed there stream ~8% slower (10.75 vs 9.88 us per call measured)
    # than the separately allocated buffers a model's weights get.
    torch.cuda.empty_cache()


def cpu_baseline(target_s=15.0):
    """The oracle on the first rows of the square workload, timed on the host."""
    import oracle
    import workloads
    w = workloads.WORKLOADS["square_8192"]
    M, N, K = w["M"], w["N"], w["K"]
    A, B = workloads.workload_inputs("square_8192")
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=(0, threads), want_sums=False)
    t1 = time.perf_counter() - t0
    rows = int(min(M, max(threads, threads * round(target_s / max(t1, 1e-3)))))
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=(0, rows), want_sums=False)
    dt = time.perf_counter() - t0
    tflops = 2.0 * rows * N * K / dt / 1e12
    log("cpu oracle: %d rows x %d x %d in %.1f s on %d threads: %.2e TFLOP/s" % (rows, N, K, dt, threads, tflops))
    return dict(value=tflops, unit="TFLOP/s", cores=threads, kind="oracle", cpu_model=cpu_model(),
                host_cpus_visible=len(os.sched_getaffinity(0)),
                sample="rows 0..%d of the 8192^3 workload (%d x 8192 outputs, K = 8192), %.1f s"
                       % (rows - 1, rows, dt))


def config_roofline(name, r):
    """Roofline of one of the remaining dense workloads: HBM-bound below the
    machine balance (2.5 PFLOP/s / 8 TB/s = 312.5 flop per byte), MFMA-bound
    above it; the tiny workload is bound by launch latency (no peak)."""
    if name.startswith("tiny"):
        return {"bound": "latency", "achieved": round(r["us"], 3), "unit": "us per call", "peak": None,
                "frac": None, "traffic": None, "kernel": r["kernel"]}
    if r["flops"] / r["alg_bytes"] < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9):
        return {"bound": "hbm", "achieved": round(r["gbps"], 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(r["gbps"] / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(name, r["kernel"]),
                "kernel": r["kernel"],
                "per_launch": "2 (M K + N K + M N) = %d bytes per launch" % r["alg_bytes"]}
    return {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(r["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(name, r["kernel"]),
            "kernel": r["kernel"], "per_launch": "2 M N K = %.4g flop per launch" % r["flops"]}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    global CLOCKS, SETTLE_S
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~75 ms of warm-up at 8192^3: the engine clock settles under sustained
    # MFMA load within a few tens of launches; shorter warm-ups time the ramp.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=2000)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed calls before each leg's timed windows (clock settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (debug runs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny / MLP-up / prefill-down and compute-bound middle legs (counter runs)")
    ap.add_argument("--only", choices=["square", "decode", "mx", "mx4", "grouped", "layouts", "configs", "middle"],
                    help="time one leg only (profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (gfx950) GPU", file=sys.stderr)
        return 1
    import tile_level_dense_amd as hkg
    hkg.lib()

    SETTLE_S = args.settle
    CLOCKS = ClockSampler()
    idle = CLOCKS.activity()
    if idle and max(idle) > 5:
        log("device not idle before timing: gfx activity %s %%" % idle)
    calibration_copy(torch)
    if args.only == "decode":
        dec = bench_decode(torch, hkg, args.decode_steps, max(args.warmup * 10, 100))
        print(json.dumps({"decode_gbps": round(dec["gbps"], 1), "us_per_call": round(dec["ms"] * 1e3, 3),
                          "llc_resident_gbps": round(dec["gbps_hot"], 1)}), flush=True)
        return 0
    if args.only == "layouts":
        lay = bench_layouts(torch, hkg, args.steps, args.warmup)
        print(json.dumps({k: round(v, 3) for k, v in lay.items()}), flush=True)
        return 0
    if args.only == "grouped":
        grp = bench_grouped(torch, hkg, args.steps, args.warmup)
        print(json.dumps({k: round(v["tflops"], 2) for k, v in grp.items()}), flush=True)
        return 0
    if args.only in ("configs", "middle"):
        cfg = bench_configs(torch, hkg, ALL_CONFIGS if args.only == "configs" else MIDDLE_CONFIGS)
        print(json.dumps({k: round(v["us"], 3) for k, v in cfg.items()}), flush=True)
        return 0
    if args.only == "mx":
        mxs = bench_mx_square(torch, hkg, args.steps, args.warmup)
        mxd = bench_mx_decode(torch, hkg, args.decode_steps, max(args.warmup * 10, 100))
        print(json.dumps({"mx_square_tflops": round(mxs["tflops"], 2), "mx_decode_gbps": round(mxd["gbps"], 1)}),
              flush=True)
        return 0
    if args.only == "mx4":
        m4s = bench_mx_square(torch, hkg, args.steps, args.warmup, fmt="fp4")
        m4d = bench_mx_decode(torch, hkg, args.decode_steps, max(args.warmup * 10, 100), fmt="fp4")
        print(json.dumps({"mx4_square_tflops": round(m4s["tflops"], 2), "mx4_decode_gbps": round(m4d["gbps"], 1)}),
              flush=True)
        return 0
    sq = bench_square(torch, hkg, args.steps, args.warmup)
    if args.only == "square":
        print(json.dumps({"square_tflops": round(sq["tflops"], 2), "ms_per_step": round(sq["ms"], 4)}), flush=True)
        return 0
    dec = bench_decode(torch, hkg, args.decode_steps, max(args.warmup * 10, 100))
    mxs = bench_mx_square(torch, hkg, args.steps, args.warmup)
    mxd = bench_mx_decode(torch, hkg, args.decode_steps, max(args.warmup * 10, 100))
    m4s = bench_mx_square(torch, hkg, args.steps, args.warmup, fmt="fp4")
    m4d = bench_mx_decode(torch, hkg, args.decode_steps, max(args.warmup * 10, 100), fmt="fp4")
    grp = bench_grouped(torch, hkg, args.steps, args.warmup)
    lay = bench_layouts(torch, hkg, args.steps, args.warmup)
    cfg = {} if args.no_configs else bench_configs(torch, hkg)
    mid = {} if args.no_configs else bench_configs(torch, hkg, MIDDLE_CONFIGS)
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    tile_kernel = sq["plan"].kernel_name.decode()
    skinny_kernel = dec["plan"].kernel_name.decode()
    tr = measured_traffic("square_8192", tile_kernel)
    tr_dec = measured_traffic("decode_16x4096x4096", skinny_kernel)
    line = {
        "metric": METRIC,
        "value": round(sq["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sq["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(sq["tflops"] / PAGES_8192_TFLOPS, 4),
        "baseline_note": "HipKittens 8192^3 BF16 GEMM on MI355X, 1610 TFLOP/s (pages' best figure)",
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "square_8192: C = A B^T, M = N = K = 8192, bf16 in, fp32 accumulate, bf16 out",
                   "M": sq["M"], "N": sq["N"], "K": sq["K"], "kernel": tile_kernel,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(sq["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(sq["tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": tr, "kernel": tile_kernel,
                     "per_launch": "2 M N K = %.4g flop per launch (one launch per step)" % sq["flops"],
                     "clocks_during_timing": (TIMINGS.get("square") or {}).get("clocks"),
                     "vendor_clocks_during_timing": (TIMINGS.get("square_torch_mm") or {}).get("clocks")},
        "decode": {"workload": "decode_16x4096x4096: M = 16, N = 4096, K = 4096",
                   "value": round(dec["gbps"], 1), "unit": "GB/s",
                   "frac_of_hbm": round(dec["gbps"] / PEAK_HBM_GBPS, 4),
                   "us_per_call": round(dec["ms"] * 1e3, 3),
                   "roofline": {"bound": "hbm", "achieved": round(dec["gbps"], 1), "peak": PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": round(dec["gbps"] / PEAK_HBM_GBPS, 4),
                                "traffic": tr_dec, "kernel": skinny_kernel,
                                "per_launch": "2 (M K + N K + M N) = %d bytes per launch" % dec["alg_bytes"]},
                   "rotating_sets": dec["sets"], "launches_timed": dec["launches"],
                   "llc_resident_gbps": round(dec["gbps_hot"], 1),
                   "launch_floor_us": round(dec["floor_us"], 3),
                   "per_call_cap_gbps": round(dec["floor_cap_gbps"], 1),
                   "per_call_cap_note": "per-call rate of this workload if its bytes moved at the 8 TB/s peak "
                                        "after the measured launch floor of a graph of one-element fills",
                   "copy_same_bytes_gbps": round(dec["copy_gbps"], 1),
                   "copy_same_bytes_us": round(dec["copy_us"], 3),
                   "copy_note": "torch copy_ moving the same bytes per call (half read, half written), rotating "
                                "buffers, graph-launched: a streaming kernel's per-call rate at this size"},
        "cpu_baseline": cpu,
        "epilogue": {"square_bias_gelu_tflops": round(sq["epi_tflops"], 2),
                     "square_bias_gelu_ms": round(sq["epi_ms"], 4),
                     "decode_bias_silu_gbps": round(dec["epi_gbps"], 1),
                     "decode_bias_silu_us": round(dec["epi_ms"] * 1e3, 3),
                     "note": "fused bias + activation (FlyDSL guide epilogues); decode bytes include the bias"},
        "vendor_context": {"library": "torch.mm (hipBLASLt), same inputs and timing in the same run",
                           "square_tflops": round(sq["vendor_tflops"], 2),
                           "decode_gbps": round(dec["vendor_gbps"], 1)},
        "power_context": {"square_constant_inputs_tflops": round(sq["const_tflops"], 2),
                          "note": "the same square kernel with every operand element 0.01147: little "
                                  "switching in the matrix cores, less power, a higher engine clock"},
        "grouped": {name: {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                           "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2),
                                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
                                        "traffic": measured_traffic(name, r["plan"].kernel_name.decode()),
                                        "kernel": r["plan"].kernel_name.decode(),
                                        "per_launch": "2 sum(M_g) N K = %.4g flop per launch" % r["flops"]},
                           "vendor_grouped_mm_tflops": round(r["vendor_tflops"], 2) if r["vendor_tflops"] else None}
                    for name, r in grp.items()},
        "layouts": {"workload": "square_8192 with column-layout operands (per-call transpose)",
                    "nn_tflops": round(lay["nn_tflops"], 2), "tn_tflops": round(lay["tn_tflops"], 2),
                    "transpose_ms": round(lay["transpose_ms"], 4), "transpose_gbps": round(lay["transpose_gbps"], 1),
                    "prepacked_nn": "equals the square_8192 value: a pre-packed weight runs the row-layout kernel",
                    "vendor_nn_tflops": round(lay["vendor_nn_tflops"], 2)},
        "other_configs": {name: {"us_per_call": round(r["us"], 3), "tflops": round(r["tflops"], 2),
                                 "gbps": round(r["gbps"], 1), "kernel": r["kernel"], "split_k": r["split_k"],
                                 "rotating_sets": r["sets"], "launches_per_window": r["launches"],
                                 "vendor_us": round(r["vendor_us"], 3),
                                 "roofline": config_roofline(name, r)}
                          for name, r in cfg.items()},
        "middle": {name: {"us_per_call": round(r["us"], 3), "tflops": round(r["tflops"], 2),
                          "kernel": r["kernel"], "rotating_sets": r["sets"],
                          "launches_per_window": r["launches"], "vendor_us": round(r["vendor_us"], 3),
                          "roofline": config_roofline(name, r)}
                   for name, r in mid.items()},
        "timing": {"protocol": "per leg: W warm-up calls, then untimed back-to-back calls for %.2f s of device "
                               "time (clock settle), then %d windows of K calls, each bracketed by device "
                               "synchronisation and timed with HIP events on the launch stream; the figure is "
                               "the median window (8192^3 legs settle %.2f s); engine clock (mean over the XCDs), "
                               "memory clock and socket power from amdsmi's metrics table, keeping refreshes made "
                               "while the leg ran" % (SETTLE_S, WINDOWS, SQUARE_SETTLE * SETTLE_S),
                   "settle_s": SETTLE_S, "square_settle_s": SQUARE_SETTLE * SETTLE_S, "windows": WINDOWS,
                   "idle_gfx_activity_pct_before": idle, "legs": TIMINGS},
        "mxfp8": {
            "square": {"workload": "mx_square_8192: E4M3 A, B N(0,1), E8M0 scale per 32 k, M = N = K = 8192",
                       "tflops": round(mxs["tflops"], 2), "ms": round(mxs["ms"], 4),
                       "per_call_packing_tflops": round(mxs["tflops_nat"], 2),
                       "roofline": {"bound": "mfma", "achieved": round(mxs["tflops"], 2), "peak": PEAK_FP8_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(mxs["tflops"] / PEAK_FP8_TFLOPS, 4),
                                    "traffic": measured_traffic("mx_square_8192", mxs["plan"].kernel_name.decode()),
                                    "kernel": mxs["plan"].kernel_name.decode(),
                                    "per_launch": "2 M N K = %.4g flop per launch" % mxs["flops"]},
                       "vendor_fp8_per_tensor_tflops": round(mxs["vendor_tflops"], 2) if mxs["vendor_tflops"] else None},
            "decode": {"workload": "mx_decode_32x4096x4096: M = 32, N = K = 4096, B N(0, 0.02)",
                       "gbps": round(mxd["gbps"], 1), "us_per_call": round(mxd["ms"] * 1e3, 3),
                       "natural_scales_us": round(mxd["ms_nat"] * 1e3, 3),
                       "roofline": {"bound": "hbm", "achieved": round(mxd["gbps"], 1), "peak": PEAK_HBM_GBPS,
                                    "unit": "GB/s", "frac": round(mxd["gbps"] / PEAK_HBM_GBPS, 4),
                                    "traffic": measured_traffic("mx_decode_32x4096x4096", mxd["plan"].kernel_name.decode()),
                                    "kernel": mxd["plan"].kernel_name.decode(),
                                    "per_launch": "M K + N K + (M + N) K / 32 + 2 M N = %d bytes" % mxd["alg_bytes"]},
                       "rotating_sets": mxd["sets"], "launches_timed": mxd["launches"],
                       "vendor_fp8_per_tensor_us": round(mxd["vendor_us"], 3) if mxd["vendor_us"] else None},
        },
        "mxfp4": {
            "square": {"workload": "mx4_square_8192: E2M1 A, B (all 16 codes), E8M0 scale per 32 k, "
                                   "M = N = K = 8192",
                       "tflops": round(m4s["tflops"], 2), "ms": round(m4s["ms"], 4),
                       "per_call_packing_tflops": round(m4s["tflops_nat"], 2),
                       "roofline": {"bound": "mfma", "achieved": round(m4s["tflops"], 2), "peak": PEAK_FP4_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(m4s["tflops"] / PEAK_FP4_TFLOPS, 4),
                                    "traffic": measured_traffic(m4s["name"], m4s["plan"].kernel_name.decode()),
                                    "kernel": m4s["plan"].kernel_name.decode(),
                                    "per_launch": "2 M N K = %.4g flop per launch" % m4s["flops"]}},
            "decode": {"workload": "mx4_decode_32x14336x4096: M = 32, N = 14336, K = 4096",
                       "gbps": round(m4d["gbps"], 1), "us_per_call": round(m4d["ms"] * 1e3, 3),
                       "natural_scales_us": round(m4d["ms_nat"] * 1e3, 3),
                       "roofline": {"bound": "hbm", "achieved": round(m4d["gbps"], 1), "peak": PEAK_HBM_GBPS,
                                    "unit": "GB/s", "frac": round(m4d["gbps"] / PEAK_HBM_GBPS, 4),
                                    "traffic": measured_traffic(m4d["name"], m4d["plan"].kernel_name.decode()),
                                    "kernel": m4d["plan"].kernel_name.decode(),
                                    "per_launch": "(M K + N K) / 2 + (M + N) K / 32 + 2 M N = %d bytes"
                                                  % m4d["alg_bytes"]},
                       "rotating_sets": m4d["sets"], "launches_timed": m4d["launches"]},
        },
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Benchmark of the FP4 block-scaled quantise / GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--only NAME] [--no-cpu-baseline]

Prints ONE JSON line.  The headline (`value`) is the 8192^3 MXFP4 GEMM: A and B
N(0,1) with 0.2% outliers x20, pre-quantised to 32-blocks with E8M0 scales,
FP32 accumulation, BF16 output; one step = one GEMM; exactly K timed steps
after W warm-up steps, with 8 rotating copies of the operands so repeated
steps are not served from the 256 MB Infinity Cache.  Before each workload's
warm-up its step runs untimed for --settle seconds (default 0.25) so that the
GPU's clocks have reached their sustained level under load.  The same line carries
the dominant kernel's roofline (HIP events around the timed launches, on the
launch stream), the GPU's shader clock and socket power sampled while the
headline ran ("gpu_telemetry": the chip runs at its power cap under this
load, so the clock it settles to bounds the matrix-core rate), the CPU oracle
timed on a bounded sample of the same workload, and, under "workloads", the
other measured workloads:

  nvfp4_decode_m{1,8,32}  W 8192x8192 NVFP4 (pre-quantised), X Mx8192 BF16
                          quantised on the fly; step = tensor amax + quantise
                          + decode GEMV (one fused kernel at M = 1, two
                          kernels at M = 8 and 32); GB/s of algorithmic
                          bytes vs 8 TB/s.
  nvfp4_mlp               A 4096x4096 BF16 quantised on the fly, W 14336x4096
                          NVFP4; step = amax + quantise + GEMM; TFLOP/s.
  mxfp4_moe               32 experts 5760x2880 MXFP4, 16384 BF16 tokens
                          quantised once per step, Zipf(1.2) top-4 routing;
                          step = quantise + grouped GEMM; TFLOP/s.
  nvfp4_moe               the same with NVFP4 operands (per-expert tensor
                          scales); step = amax + quantise + grouped GEMM.
  mxfp4_256               A, B 256x256 FP32; step = quantise A, B + GEMM (FP32
                          out); microseconds.
  mxfp4_quantize_8192     8192x8192 FP32 -> MXFP4; GB/s.
  mxfp4_gemm_requant_8192 the headline GEMM with bias, ReLU and MXFP4 output
                          in the same kernel (fp4_gemm_ex); TFLOP/s.
  nvfp4_quantize_sr_8192  8192x8192 BF16 -> NVFP4 with stochastic rounding
                          (fp4_quantize_sr); GB/s.
  hadamard16_8192         random Hadamard transform, 8192x8192 BF16; GB/s.
  nvfp4_quantize_2d_weight 14336x4096 FP32 -> NVFP4 with 16x16 patch scales;
                          GB/s.
  w4a8_gemm_8192          the headline's inputs with A quantised to MXFP8
                          (E4M3) instead: MXFP8 x MXFP4 GEMM (fp4_gemm_w4a8),
                          BF16 out; TFLOP/s vs the 5.0 PFLOP/s FP8 peak (the
                          matrix core runs FP8 x FP4 at the FP8 rate).
  mxfp8_quantize_8192     8192x8192 FP32 -> MXFP8; GB/s.

Launch-bound steps (decode, 256^3) are captured once in a HIP graph and
replayed; every replayed result is checked against the eager one.
"""
import argparse
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP4_TFLOPS = 10100.0   # MI355X dense MXFP4 / FP6 matrix peak
PEAK_FP16_TFLOPS = 2500.0   # MI355X dense FP16 / BF16 matrix peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ROTATE = 8
METRIC = "FP4 GEMM TFLOPS & % MXFP4 MFMA peak; decode-shape HBM GB/s & % peak"


# ---- algorithmic work -------------------------------------------------------
def gemm_flops(M, N, K):
    return 2.0 * M * N * K


def fp4_operand_bytes(rows, K, block):
    """Codes (0.5 B per value) plus one scale byte per block."""
    return rows * K * 0.5 + rows * (K // block)


def gemm_bytes(M, N, K, block=32, out_bytes=2, include_c=True):
    """Algorithmic bytes of a GEMM on pre-quantised operands: each operand's
    codes and scales read once, C written once."""
    b = fp4_operand_bytes(M, K, block) + fp4_operand_bytes(N, K, block)
    return b + (M * N * out_bytes if include_c else 0)


def arithmetic_intensity(M, N, K, block=32, out_bytes=2, include_c=True):
    return gemm_flops(M, N, K) / gemm_bytes(M, N, K, block, out_bytes, include_c)


# ---- timing helpers ---------------------------------------------------------
SETTLE_S = 0.25


class Telemetry:
    """GFX clock (MHz) and socket power (W) sampled every 10 ms on a host
    thread while a workload runs, through amdsmi (the driver's metrics).  The
    readings lag the load by a few hundred milliseconds, so samples from the
    first `skip_s` seconds are dropped.  summary() is None when amdsmi is
    missing or cannot reach the GPU."""

    def __init__(self, skip_s=1.0):
        self.clk, self.pwr, self.cap, self.err = [], [], None, None
        self.skip_s = skip_s
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            cap = amdsmi.amdsmi_get_power_info(self._h).get("power_limit")
            self.cap = cap / 1e6 if isinstance(cap, (int, float)) and cap > 1e4 else cap
        except Exception as e:  # no amdsmi, no driver access: telemetry is optional
            self._smi, self.err = None, "%s: %s" % (type(e).__name__, e)

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            if time.perf_counter() - t0 < self.skip_s:
                time.sleep(0.01)
                continue
            try:
                c = self._smi.amdsmi_get_clock_info(self._h, self._smi.AmdSmiClkType.GFX).get("clk")
                p = self._smi.amdsmi_get_power_info(self._h).get("current_socket_power")
                if isinstance(c, (int, float)):
                    self.clk.append(float(c))
                if isinstance(p, (int, float)):
                    self.pwr.append(float(p))
            except Exception as e:
                self.err = "%s: %s" % (type(e).__name__, e)
                return
            time.sleep(0.01)

    def __enter__(self):
        if self._smi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self, what):
        if self._smi is None or not self.clk:
            return None if self.err is None else {"error": self.err}

        def stats(v):
            v = sorted(v)
            return {"median": v[len(v) // 2], "p10": v[len(v) // 10], "p90": v[(len(v) * 9) // 10]} if v else None
        return {"during": what, "source": "amdsmi", "samples": len(self.clk), "gfxclk_mhz": stats(self.clk),
                "socket_power_w": stats(self.pwr), "power_cap_w": self.cap}


def time_steps(torch, step, steps, warmup):
    """Run the step untimed for SETTLE_S seconds (the GPU's clocks need tens of
    milliseconds under load to reach their sustained level: with 10 warm-up
    8192^3 GEMMs alone the timed ones ran 10% slower), then `warmup` untimed
    steps, then time exactly `steps` steps with HIP events on the current
    (launch) stream.  Returns ms per step."""
    i = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(4):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def graph_steps(torch, step, per_graph, check):
    """Capture `per_graph` steps (rotating inputs) into one HIP graph; returns
    a replay function.  `check()` compares the step's output with an eager
    result after each of a few replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            step(i)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        check()
    return g


def to_dev(torch, x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_record(kernel_src):
    """HBM traffic of the headline kernel from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "gemm_mxfp4_8192_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha256_16") != src_hash(kernel_src):
        return None
    return rec.get("traffic_bytes_per_launch")


# ---- workloads --------------------------------------------------------------
def mxfp4_gemm_8192(torch, fp4, synth, args):
    n = 8192
    a, b = synth.mxfp4_8192(n)
    qa0 = fp4.quantize(to_dev(torch, a), fp4.MXFP4)
    qb0 = fp4.quantize(to_dev(torch, b), fp4.MXFP4)
    qa = [qa0] + [fp4.Quantized(qa0.codes.clone(), qa0.scales.clone(), None, fp4.MXFP4, n, n)
                  for _ in range(ROTATE - 1)]
    qb = [qb0] + [fp4.Quantized(qb0.codes.clone(), qb0.scales.clone(), None, fp4.MXFP4, n, n)
                  for _ in range(ROTATE - 1)]
    C = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        fp4.gemm(qa[i % ROTATE], qb[i % ROTATE], out=C)

    ms = time_steps(torch, step, args.steps, args.warmup)
    tflops = gemm_flops(n, n, n) / (ms * 1e-3) / 1e12
    # Clock and power under the same load: 2.5 s of the same steps after the
    # timed ones (the driver's readings need longer than the timed region).
    if args.telemetry_s <= 0:
        return dict(ms=ms, tflops=tflops, a=a, b=b, telemetry=None)
    with Telemetry() as tel:
        t0, i = time.perf_counter(), 0
        while time.perf_counter() - t0 < args.telemetry_s:
            step(i)
            i += 1
            if i % 32 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    return dict(ms=ms, tflops=tflops, a=a, b=b,
                telemetry=tel.summary("%.1f s of headline steps right after the timed ones (first 1 s dropped)"
                                      % args.telemetry_s))


def mxfp4_gemm_requant_8192(torch, fp4, synth, a, b):
    """The 8192^3 MXFP4 GEMM with the whole epilogue in the kernel: + bias,
    ReLU, and the result quantised again to MXFP4 along N (the next layer's
    operand), 8 rotating operand copies as the headline."""
    n = 8192
    qa0 = fp4.quantize(to_dev(torch, a), fp4.MXFP4)
    qb0 = fp4.quantize(to_dev(torch, b), fp4.MXFP4)
    qa = [qa0] + [fp4.Quantized(qa0.codes.clone(), qa0.scales.clone(), None, fp4.MXFP4, n, n)
                  for _ in range(ROTATE - 1)]
    qb = [qb0] + [fp4.Quantized(qb0.codes.clone(), qb0.scales.clone(), None, fp4.MXFP4, n, n)
                  for _ in range(ROTATE - 1)]
    bias = torch.from_numpy((0.5 * synth.gaussian(11, (n,))).astype(np.float32)).cuda()
    out = fp4.Quantized(torch.empty((n, n // 2), dtype=torch.uint8, device="cuda"),
                        torch.empty(fp4.fp4_scale_bytes(fp4.MXFP4, n, n), dtype=torch.uint8, device="cuda"),
                        None, fp4.MXFP4, n, n)
    torch.cuda.synchronize()

    def step(i):
        fp4.gemm_ex(qa[i % ROTATE], qb[i % ROTATE], bias=bias, act=fp4.ACT_RELU, out=fp4.OUT_MXFP4, C=out)

    ms = time_steps(torch, step, 30, 5)
    tf = gemm_flops(n, n, n) / (ms * 1e-3) / 1e12
    out_bytes = n * n // 2 + fp4.fp4_scale_bytes(fp4.MXFP4, n, n)
    return {"ms_per_step": round(ms, 4), "TFLOP_per_s": round(tf, 1), "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
            "output_bytes": int(out_bytes),
            "step": "MXFP4 GEMM + bias + ReLU + MXFP4 re-quantisation of C in one kernel (fp4_gemm_ex)"}


def nvfp4_quantize_sr_8192(torch, fp4, synth):
    """8192 x 8192 BF16 gradient-like tensor (N(0, 1e-3^2), 0.1% outliers x20)
    -> NVFP4 with its own tensor scale, elements rounded stochastically
    (fp4_quantize_sr; amax pass + quantise pass), beside the same with
    round-to-nearest-even."""
    n = 8192
    x = to_dev(torch, synth.to_bf16_bits(synth.gaussian(81, (n, n), std=1e-3, bernoulli=0.001)))
    q = fp4.quantize(x, fp4.NVFP4, sr_seed=1)
    ws = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, n, 0, n)
    ms_sr = time_steps(torch, lambda i: fp4.quantize(x, fp4.NVFP4, ws=ws, out=q, sr_seed=i + 1), 30, 5)
    ms_rn = time_steps(torch, lambda i: fp4.quantize(x, fp4.NVFP4, ws=ws, out=q), 30, 5)
    # Algorithmic bytes: the input read once, codes and scales written once.
    # The step reads the input twice (amax pass, then quantise pass); that
    # second read is not credited.
    nbytes = n * n * 2 + n * n // 2 + n * n // 16
    gbs = nbytes / (ms_sr * 1e-3) / 1e9
    return {"us_per_step": round(ms_sr * 1e3, 2), "algorithmic_bytes": int(nbytes), "GB_per_s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "passes_over_input": 2,
            "us_per_step_round_to_nearest": round(ms_rn * 1e3, 2),
            "step": "tensor amax + NVFP4 quantise with stochastic rounding (Philox4x64-10 per element)"}


def hadamard16_8192(torch, fp4, synth):
    """Random Hadamard transform of an 8192 x 8192 BF16 tensor on 16-value
    blocks (fp4_hadamard16), BF16 out; GB/s of input read + output written."""
    n = 8192
    x = to_dev(torch, synth.to_bf16_bits(synth.gaussian(82, (n, n))))
    y = torch.empty_like(x)
    ms = time_steps(torch, lambda i: fp4.hadamard16(x, seed=i, out=y), 30, 5)
    nbytes = 2 * n * n * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"us_per_step": round(ms * 1e3, 2), "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "step": "y = (1/4) H16 D x per 16-value block along K, BF16 in and out"}


def nvfp4_quantize_2d_weight(torch, fp4, synth):
    """The MLP weight (14336 x 4096, FP32) to NVFP4 with 16 x 16 patch scales
    (tensor amax + 2-D quantise), beside the 1 x 16 quantiser."""
    _, w = synth.nvfp4_mlp()
    wd = to_dev(torch, w)
    del w
    q = fp4.quantize(wd, fp4.NVFP4, two_d=True)
    ws = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, wd.shape[0], 0, wd.shape[1])
    ms2 = time_steps(torch, lambda i: fp4.quantize(wd, fp4.NVFP4, ws=ws, out=q, two_d=True), 20, 3)
    ms1 = time_steps(torch, lambda i: fp4.quantize(wd, fp4.NVFP4, ws=ws, out=q), 20, 3)
    n = wd.numel()
    # Input read once (the amax pass's second read is not credited), codes
    # and scales written once.
    nbytes = n * 4 + n // 2 + n // 16
    gbs = nbytes / (ms2 * 1e-3) / 1e9
    return {"rows": int(wd.shape[0]), "K": int(wd.shape[1]), "us_per_step": round(ms2 * 1e3, 2),
            "algorithmic_bytes": int(nbytes), "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "passes_over_input": 2,
            "us_per_step_1x16": round(ms1 * 1e3, 2),
            "step": "tensor amax + NVFP4 quantise with one scale per 16 x 16 patch (FP32 in)"}


def w4a8_gemm_8192(torch, fp4, synth, a, b):
    """8192^3 W4A8: the headline's A quantised to MXFP8 (E4M3 elements, E8M0
    32-blocks), its B to MXFP4; 8 rotating operand copies; BF16 out."""
    n = 8192
    qa0 = fp4.quantize(to_dev(torch, a), fp4.MXFP8)
    qb0 = fp4.quantize(to_dev(torch, b), fp4.MXFP4)
    qa = [qa0] + [fp4.Quantized(qa0.codes.clone(), qa0.scales.clone(), None, fp4.MXFP8, n, n)
                  for _ in range(ROTATE - 1)]
    qb = [qb0] + [fp4.Quantized(qb0.codes.clone(), qb0.scales.clone(), None, fp4.MXFP4, n, n)
                  for _ in range(ROTATE - 1)]
    C = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    ms = time_steps(torch, lambda i: fp4.gemm_w4a8(qa[i % ROTATE], qb[i % ROTATE], out=C), 30, 5)
    tf = gemm_flops(n, n, n) / (ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 4), "TFLOP_per_s": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "step": "MXFP8 (E4M3) x MXFP4 GEMM, FP32 accumulation, BF16 out (fp4_gemm_w4a8)"}


def mxfp8_quantize_8192(torch, fp4, a):
    x = to_dev(torch, a)
    q = fp4.quantize(x, fp4.MXFP8)
    ms = time_steps(torch, lambda i: fp4.quantize(x, fp4.MXFP8, out=q), 50, 5)
    n = a.size
    nbytes = n * 4 + n + n // 32
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"us_per_step": round(ms * 1e3, 2), "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def cpu_baseline_gemm(a, b, K, budget_s=12.0):
    """The oracle (quantise + FP64 GEMM) on a slab of the 8192^3 workload,
    sized to roughly `budget_s` seconds; TFLOP/s of the slab's arithmetic."""
    import oracle
    t0 = time.perf_counter()
    ra = oracle.quantize(a[:64], oracle.FMT_MXFP4)
    rb = oracle.quantize(b[:64], oracle.FMT_MXFP4)
    oracle.gemm(ra[0], ra[1], rb[0], rb[1], 64, 64, K, oracle.FMT_MXFP4)
    dt = time.perf_counter() - t0
    cols = int(max(64, min(8192, 64 * budget_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    ra = oracle.quantize(a[:64], oracle.FMT_MXFP4)
    rb = oracle.quantize(b[:cols], oracle.FMT_MXFP4)
    oracle.gemm(ra[0], ra[1], rb[0], rb[1], 64, cols, K, oracle.FMT_MXFP4)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(gemm_flops(64, cols, K) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "oracle MXFP4 quantise of 64 rows of A and %d rows of B plus FP64 GEMM 64x%dx%d of the "
                      "8192^3 workload, %.1f s" % (cols, cols, K, dt)}


# ---- the oracle on every config (python bench.py --cpu-baseline-all) ---------
def _host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def oracle_worker(budget_s):
    """Times the oracle (quantise + FP64 GEMM) on every config with this
    process's OpenMP thread count; prints one JSON line.  The quantisers run
    in full; a GEMM that would take longer than `budget_s` runs on a slab of
    output rows (or weight rows) and is scaled linearly to the full problem
    (the oracle's cost per output element is the same for every element)."""
    import oracle
    import synth
    oracle.build()
    oracle.lib()

    def timed(fn, *a, **kw):
        t0 = time.perf_counter()
        r = fn(*a, **kw)
        return r, time.perf_counter() - t0

    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)

    def gemm_slab(ra, rb, rows_a, rows_b, K, fmt, scale_rows_to, **kw):
        """FP64 GEMM of a slab of A's rows against rb; rows sized so the slab
        takes about budget_s (the oracle runs its threads over output rows:
        at least 4 rows per thread, a multiple of the thread count); returns
        (seconds for scale_rows_to rows, slab rows)."""
        probe = min(rows_a, threads)
        _, tp = timed(oracle.gemm, np.ascontiguousarray(ra[0][:probe]), ra[1], rb[0], rb[1], probe, rows_b, K, fmt, **kw)
        rows = int(max(4 * threads, min(rows_a, probe * budget_s / max(tp, 1e-4))))
        rows = min(rows_a, (rows + threads - 1) // threads * threads)
        # a row slab of the quantised A: codes rows are contiguous, and the
        # scale tiles of the first `rows` rows are the first ceil(rows/32) tiles
        _, ts = timed(oracle.gemm, np.ascontiguousarray(ra[0][:rows]), ra[1], rb[0], rb[1], rows, rows_b, K, fmt, **kw)
        return ts * scale_rows_to / rows, rows

    out = {}
    # 1. MXFP4 256^3, FP32 inputs, full
    a, b = synth.mxfp4_256()
    (ra, tqa), (rb, tqb) = timed(oracle.quantize, a, 0), timed(oracle.quantize, b, 0)
    _, tg = timed(oracle.gemm, ra[0], ra[1], rb[0], rb[1], 256, 256, 256, 0)
    out["mxfp4_256"] = {"quantize_s": tqa + tqb, "gemm_s": tg, "step_s": tqa + tqb + tg, "slab": "none (full)",
                        "flop": gemm_flops(256, 256, 256)}
    # 2. NVFP4 decode: X quantised in full; GEMM over a slab of weight rows
    #    (all M activation rows), scaled to N = 8192
    w = synth.nvfp4_decode_weight()
    rw, tqw = timed(oracle.quantize, w, 1)
    del w
    for M in (1, 8, 32):
        x = synth.nvfp4_decode_act(M)
        rx, tqx = timed(oracle.quantize, x, 1)
        # (the oracle's sampled product runs its threads over the outputs, so
        # a decode shape of 1-32 rows still uses every thread)
        def outputs(nr):
            return np.repeat(np.arange(M), nr), np.tile(np.arange(nr), M)
        r, c = outputs(64)
        _, t1 = timed(oracle.gemm_sampled, rx[0], rx[1], rw[0], rw[1], M, 8192, 8192, 1, r, c, tsA=rx[3], tsB=rw[3])
        nrows = int(max(64, min(8192, 64 * budget_s / max(t1, 1e-4)))) // 64 * 64
        r, c = outputs(nrows)
        _, ts = timed(oracle.gemm_sampled, rx[0], rx[1], rw[0], rw[1], M, 8192, 8192, 1, r, c, tsA=rx[3], tsB=rw[3])
        tg = ts * 8192 / nrows
        out["nvfp4_decode_m%d" % M] = {"quantize_s": tqx, "gemm_s": tg, "step_s": tqx + tg,
                                       "slab": "%d of 8192 weight rows" % nrows if nrows < 8192 else "none (full)",
                                       "weight_quantize_offline_s": tqw, "flop": gemm_flops(M, 8192, 8192)}
    del rw
    # 3. MXFP4 8192^3: both operands quantised in full; GEMM on a slab of A rows
    a, b = synth.mxfp4_8192()
    (ra, tqa), (rb, tqb) = timed(oracle.quantize, a, 0), timed(oracle.quantize, b, 0)
    del a, b
    tg, rows = gemm_slab(ra, rb, 8192, 8192, 8192, 0, 8192)
    out["mxfp4_8192"] = {"quantize_s": tqa + tqb, "gemm_s": tg, "step_s": tg,
                         "slab": "%d of 8192 rows of A" % rows, "flop": gemm_flops(8192, 8192, 8192),
                         "note": "the benchmark's step takes pre-quantised operands; quantize_s is reported apart"}
    del ra, rb
    # 4. NVFP4 MLP: A (BF16) and W quantised in full; GEMM on a slab of A rows
    a, w = synth.nvfp4_mlp()
    (ra, tqa), (rw, tqw) = timed(oracle.quantize, a, 1), timed(oracle.quantize, w, 1)
    del a, w
    tg, rows = gemm_slab(ra, rw, 4096, 14336, 4096, 1, 4096, tsA=ra[3], tsB=rw[3])
    out["nvfp4_mlp"] = {"quantize_s": tqa, "gemm_s": tg, "step_s": tqa + tg, "slab": "%d of 4096 rows of A" % rows,
                        "weight_quantize_offline_s": tqw, "flop": gemm_flops(4096, 14336, 4096)}
    del ra, rw
    # 5. MoE: the 16384 tokens quantised in full; every routed row costs the
    #    same N x K products, so the grouped GEMM is timed on a slab of rows of
    #    one expert (expert 0) and scaled to the 65536 routed rows
    x = synth.mxfp4_moe_act()
    rx, tqx = timed(oracle.quantize, x, 0)
    w0 = synth.mxfp4_moe_weights(experts=[0])[0]
    rw0, tqw0 = timed(oracle.quantize, w0, 0)
    del w0
    tg, rows = gemm_slab(rx, rw0, 16384, 5760, 2880, 0, 65536)
    out["mxfp4_moe"] = {"quantize_s": tqx, "gemm_s": tg, "step_s": tqx + tg,
                        "slab": "%d routed rows against expert 0, scaled to 65536" % rows,
                        "weight_quantize_offline_s_per_expert": tqw0, "flop": gemm_flops(65536, 5760, 2880)}
    for v in out.values():
        v["tflop_per_s"] = round(v["flop"] / v["step_s"] / 1e12, 7)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    print(json.dumps({"threads": threads, "configs": out}))


def cpu_baseline_all(budget_s):
    """The oracle on every config, single-threaded and on all the host's
    cores (OMP_NUM_THREADS, else the affinity mask), one worker process each."""
    import subprocess
    info = _host_info()
    allc = int(os.environ.get("OMP_NUM_THREADS") or info["affinity_cpus"] or os.cpu_count() or 1)
    runs = {}
    for t in sorted({1, allc}):
        env = dict(os.environ, OMP_NUM_THREADS=str(t))
        sys.stderr.write("[bench] oracle on every config, %d thread(s)\n" % t)
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-worker",
                            "--oracle-budget", str(budget_s)], env=env, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("oracle worker failed:\n" + r.stderr[-2000:])
        runs[str(t)] = json.loads(r.stdout.strip().splitlines()[-1])["configs"]
    print(json.dumps({"kind": "oracle", "host": info, "threads_all": allc, "runs": runs}))


def nvfp4_decode(torch, fp4, synth, M):
    N = K = 8192
    w = synth.nvfp4_decode_weight()
    qw0 = fp4.quantize(to_dev(torch, w), fp4.NVFP4)
    del w
    qw = [qw0] + [fp4.Quantized(qw0.codes.clone(), qw0.scales.clone(), qw0.tensor_scale.clone(), fp4.NVFP4, N, K)
                  for _ in range(ROTATE - 1)]
    x = to_dev(torch, synth.nvfp4_decode_act(M))
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    # The one-kernel path re-quantises X in every workgroup; it beats the
    # quantise + GEMM step at small M only (measured: M = 1 11.6 vs 14.3 us,
    # M = 2 12.4 vs 14.0 us, M = 4 16.9 vs 14.6 us).
    fused = M <= 2 and bool(fp4.fp4_gemm_nvfp4_act_supported(M, N, K, fp4.BF16))
    # fp4_quantize's NVFP4 paths: one launch up to 256 KB (every workgroup
    # reduces the maximum) and up to 1 MB (workgroups exchange it), two above
    one_launch_q = M * K * 2 <= 1024 * 1024
    if fused:
        # one kernel: tensor amax + NVFP4 quantise of X + GEMV
        def step(i):
            fp4.gemm_nvfp4_act(x, qw[i % ROTATE], out=C)
    else:
        qx = fp4.quantize(x, fp4.NVFP4)  # output buffers reused by every step
        wsq = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, M, 0, K)
        wsg = fp4.workspace(fp4.OP_GEMM, fp4.NVFP4, M, N, K)

        def step(i):
            fp4.quantize(x, fp4.NVFP4, ws=wsq, out=qx)
            fp4.gemm(qx, qw[i % ROTATE], out=C, ws=wsg)

    step(0)
    torch.cuda.synchronize()
    ref = C.clone()

    def check():
        assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), "graph replay differs from eager"

    per_graph = ROTATE * 4
    g = graph_steps(torch, step, per_graph, check)
    reps = 30
    ms = time_steps(torch, lambda i: g.replay(), reps, 3) / per_graph
    nbytes = fp4_operand_bytes(N, K, 16) + M * K * 2 + M * N * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"M": M, "N": N, "K": K, "us_per_step": round(ms * 1e3, 3), "algorithmic_bytes": int(nbytes),
            "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "step": ("one kernel: tensor amax + NVFP4 quantise of X + decode GEMV" if fused else
                     ("two kernels: one-launch tensor amax + NVFP4 quantise of X, decode GEMV" if one_launch_q else
                      "three kernels: tensor amax, NVFP4 quantise of X, decode GEMV")) + " (HIP graph replay)"}


def nvfp4_mlp(torch, fp4, synth):
    M, N, K = 4096, 14336, 4096
    a, w = synth.nvfp4_mlp()
    x = to_dev(torch, a)
    qw = fp4.quantize(to_dev(torch, w), fp4.NVFP4)
    del a, w
    qx = fp4.quantize(x, fp4.NVFP4)
    wsq = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, M, 0, K)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(i):
        fp4.quantize(x, fp4.NVFP4, ws=wsq, out=qx)
        fp4.gemm(qx, qw, out=C)

    ms = time_steps(torch, step, 20, 3)
    tf = gemm_flops(M, N, K) / (ms * 1e-3) / 1e12
    return {"M": M, "N": N, "K": K, "ms_per_step": round(ms, 4), "TFLOP_per_s": round(tf, 1),
            "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4), "frac_fp16_peak": round(tf / PEAK_FP16_TFLOPS, 4),
            "step": "tensor amax + NVFP4 quantise of A (BF16) + NVFP4 GEMM (FP16 matrix core), BF16 out"}


def mxfp4_moe(torch, fp4, synth):
    E, N, K, T = 32, 5760, 2880, 16384
    counts = synth.zipf_counts()
    row_idx, off = synth.moe_routing(counts)
    x = to_dev(torch, synth.mxfp4_moe_act())
    sbytes = fp4.fp4_scale_bytes(fp4.MXFP4, N, K)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, sbytes), dtype=torch.uint8, device="cuda")
    for e in range(E):
        w = synth.mxfp4_moe_weights(E, N, K, experts=[e])[0]
        fp4.quantize(to_dev(torch, w), fp4.MXFP4, out=fp4.Quantized(codes[e], scales[e], None, fp4.MXFP4, N, K))
    qx = fp4.quantize(x, fp4.MXFP4)
    ri = torch.from_numpy(row_idx).cuda()
    go = torch.from_numpy(off).cuda()
    total = int(off[-1])
    C = torch.empty((total, N), dtype=torch.bfloat16, device="cuda")
    wsg = torch.empty(fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, fp4.MXFP4, total, N, K, E), dtype=torch.uint8,
                      device="cuda")

    def step(i):
        fp4.quantize(x, fp4.MXFP4, out=qx)
        fp4.gemm_grouped(qx, ri, go, codes, scales, N, K, fp4.MXFP4, out=C, ws=wsg)

    ms = time_steps(torch, step, 10, 2)
    tf = gemm_flops(total, N, K) / (ms * 1e-3) / 1e12
    nonempty = int((counts > 0).sum())
    # Algorithmic bytes: the non-empty experts' weights (codes + scales) and
    # the BF16 tokens read once, C written once.  The quantised tokens are an
    # intermediate (written by the quantiser, gathered by the GEMM) and are
    # not credited.
    nbytes = nonempty * fp4_operand_bytes(N, K, 32) + T * K * 2 + total * N * 2
    return {"experts": E, "N": N, "K": K, "tokens": T, "routed_rows": total, "ms_per_step": round(ms, 4),
            "TFLOP_per_s": round(tf, 1), "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
            "algorithmic_bytes": int(nbytes),
            "step": "MXFP4 quantise of the 16384 tokens (BF16) + grouped GEMM (token rows copied into expert "
                    "order first, in the call's workspace), BF16 out"}


def nvfp4_moe(torch, fp4, synth):
    """The MoE workload with NVFP4 operands: each expert quantised on its own
    (its own tensor scale), the tokens quantised per step (tensor amax + NVFP4
    quantise), the grouped GEMM on the FP16 matrix core."""
    E, N, K, T = 32, 5760, 2880, 16384
    counts = synth.zipf_counts()
    row_idx, off = synth.moe_routing(counts)
    x = to_dev(torch, synth.mxfp4_moe_act())
    sbytes = fp4.fp4_scale_bytes(fp4.NVFP4, N, K)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, sbytes), dtype=torch.uint8, device="cuda")
    ts = torch.empty(E, dtype=torch.float32, device="cuda")
    for e in range(E):
        w = synth.mxfp4_moe_weights(E, N, K, experts=[e])[0]
        fp4.quantize(to_dev(torch, w), fp4.NVFP4,
                     out=fp4.Quantized(codes[e], scales[e], ts[e:e + 1], fp4.NVFP4, N, K))
    qx = fp4.quantize(x, fp4.NVFP4)
    ws = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, T, 0, K)
    ri = torch.from_numpy(row_idx).cuda()
    go = torch.from_numpy(off).cuda()
    total = int(off[-1])
    C = torch.empty((total, N), dtype=torch.bfloat16, device="cuda")

    def step(i):
        fp4.quantize(x, fp4.NVFP4, out=qx, ws=ws)
        fp4.gemm_grouped(qx, ri, go, codes, scales, N, K, fp4.NVFP4, b_tensor_scale=ts, out=C)

    ms = time_steps(torch, step, 10, 2)
    tf = gemm_flops(total, N, K) / (ms * 1e-3) / 1e12
    return {"experts": E, "N": N, "K": K, "tokens": T, "routed_rows": total, "ms_per_step": round(ms, 4),
            "TFLOP_per_s": round(tf, 1), "frac_fp16_peak": round(tf / PEAK_FP16_TFLOPS, 4),
            "step": "tensor amax + NVFP4 quantise of the 16384 tokens (BF16) + grouped NVFP4 GEMM "
                    "(FP16 matrix core, per-expert tensor scales), BF16 out"}


def mxfp4_256(torch, fp4, synth):
    a, b = synth.mxfp4_256()
    xa, xb = to_dev(torch, a), to_dev(torch, b)
    qa = fp4.quantize(xa, fp4.MXFP4)
    qb = fp4.quantize(xb, fp4.MXFP4)
    C = torch.empty((256, 256), dtype=torch.float32, device="cuda")

    def step(i):
        fp4.quantize(xa, fp4.MXFP4, out=qa)
        fp4.quantize(xb, fp4.MXFP4, out=qb)
        fp4.gemm(qa, qb, out=C)

    step(0)
    torch.cuda.synchronize()
    ref = C.clone()

    def check():
        assert torch.equal(C, ref), "graph replay differs from eager"

    g = graph_steps(torch, step, 32, check)
    ms = time_steps(torch, lambda i: g.replay(), 30, 3) / 32
    return {"us_per_step": round(ms * 1e3, 3), "TFLOP_per_s": round(gemm_flops(256, 256, 256) / (ms * 1e-3) / 1e12, 3),
            "step": "MXFP4 quantise of A and B (FP32) + GEMM, FP32 out (HIP graph replay)"}


def mxfp4_quantize_8192(torch, fp4, a):
    x = to_dev(torch, a)
    q = fp4.quantize(x, fp4.MXFP4)
    ms = time_steps(torch, lambda i: fp4.quantize(x, fp4.MXFP4, out=q), 50, 5)
    n = a.size
    nbytes = n * 4 + fp4_operand_bytes(a.shape[0], a.shape[1], 32)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"us_per_step": round(ms * 1e3, 2), "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--only", default=None, help="run only the headline (mxfp4_gemm_8192) or one other workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--settle", type=float, default=SETTLE_S,
                   help="seconds of untimed steps before each workload's warm-up (clock ramp)")
    p.add_argument("--telemetry-s", type=float, default=2.5,
                   help="seconds of headline steps sampled for clock and power after the timed ones (0: none)")
    p.add_argument("--cpu-baseline-all", action="store_true",
                   help="only time the CPU oracle on every config, single-threaded and on all cores")
    p.add_argument("--oracle-worker", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--oracle-budget", type=float, default=4.0,
                   help="seconds per oracle GEMM slab in --cpu-baseline-all")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 256 MiB device copy (x*1 -> y) 3 times, to scale the HBM byte counters")
    return p.parse_args()


def calibrate_copy(torch):
    n = 64 << 20
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "torch.mul(x, 1.0, out=y)", "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 3}))


def main():
    args = parse()
    if args.oracle_worker:
        oracle_worker(args.oracle_budget)
        return
    if args.cpu_baseline_all:
        cpu_baseline_all(args.oracle_budget)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this library runs on a single MI355X and has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import block_scaled_fp4_03_amd as fp4
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    t_start = time.perf_counter()
    global SETTLE_S
    SETTLE_S = args.settle

    head = mxfp4_gemm_8192(torch, fp4, synth, args)
    sys.stderr.write("[bench] mxfp4_gemm_8192 %.4f ms %.1f TFLOP/s\n" % (head["ms"], head["tflops"]))
    cpu = None if args.no_cpu_baseline else cpu_baseline_gemm(head["a"], head["b"], 8192)
    sys.stderr.write("[bench] cpu_baseline %s\n" % json.dumps(cpu))

    extra = {}
    a8192 = head.pop("a")
    b8192 = head.pop("b")
    todo = [("mxfp4_quantize_8192", lambda: mxfp4_quantize_8192(torch, fp4, a8192)),
            ("mxfp4_gemm_requant_8192", lambda: mxfp4_gemm_requant_8192(torch, fp4, synth, a8192, b8192)),
            ("nvfp4_quantize_sr_8192", lambda: nvfp4_quantize_sr_8192(torch, fp4, synth)),
            ("hadamard16_8192", lambda: hadamard16_8192(torch, fp4, synth)),
            ("nvfp4_quantize_2d_weight", lambda: nvfp4_quantize_2d_weight(torch, fp4, synth)),
            ("w4a8_gemm_8192", lambda: w4a8_gemm_8192(torch, fp4, synth, a8192, b8192)),
            ("mxfp8_quantize_8192", lambda: mxfp8_quantize_8192(torch, fp4, a8192)),
            ("nvfp4_decode_m1", lambda: nvfp4_decode(torch, fp4, synth, 1)),
            ("nvfp4_decode_m8", lambda: nvfp4_decode(torch, fp4, synth, 8)),
            ("nvfp4_decode_m32", lambda: nvfp4_decode(torch, fp4, synth, 32)),
            ("nvfp4_mlp", lambda: nvfp4_mlp(torch, fp4, synth)),
            ("mxfp4_moe", lambda: mxfp4_moe(torch, fp4, synth)),
            ("nvfp4_moe", lambda: nvfp4_moe(torch, fp4, synth)),
            ("mxfp4_256", lambda: mxfp4_256(torch, fp4, synth))]
    for name, fn in todo:
        if args.only is not None and args.only != name:
            continue
        extra[name] = fn()
        torch.cuda.empty_cache()
        sys.stderr.write("[bench] %s %s\n" % (name, json.dumps(extra[name])))

    kernel_src = os.path.join(ROOT, "block_scaled_fp4_03_amd", "csrc", "gemm.hip")
    tflops = head["tflops"]
    line = {
        "metric": METRIC,
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": "mxfp4_gemm_8192x8192x8192", "M": 8192, "N": 8192, "K": 8192,
                   "operands": "pre-quantised MXFP4 (E2M1 codes, E8M0 32-blocks), N(0,1) with 0.2% outliers x20",
                   "out": "bf16", "accumulate": "fp32", "parallelism": "single-gpu", "rotating_copies": ROTATE,
                   "settle_s": SETTLE_S},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP4_TFLOPS, 4), "traffic": traffic_record(kernel_src),
                     "kernel": "gemm_kernel<MXFP4, BF16, dense>",
                     "algorithmic_flops_per_launch": gemm_flops(8192, 8192, 8192)},
        "cpu_baseline": cpu,
        "gpu_telemetry": head["telemetry"],
        "workloads": extra,
        "wall_s": round(time.perf_counter() - t_start, 1),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

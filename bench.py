"""Benchmark of the FP4 block-scaled GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The headline workload is the 8192^3 MXFP4 GEMM
(A, B N(0,1) with 0.2% outliers x20, pre-quantised to 32-blocks with E8M0
scales, FP32 accumulation, BF16 output): `value` is its throughput in TFLOP/s
over exactly K timed steps, inputs resident in HBM, with 8 rotating copies of
the operands so repeated steps cannot be served from the 256 MB Infinity Cache.
The line also carries the roofline of the dominant kernel (HIP events around
the timed launches on the launch stream) and the CPU oracle timed on a bounded
sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP4_TFLOPS = 10100.0   # MI355X dense MXFP4 / FP6 matrix peak
PEAK_FP16_TFLOPS = 2500.0   # MI355X dense FP16 / BF16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ROTATE = 8


def gemm_flops(M, N, K):
    return 2.0 * M * N * K


def gemm_bytes(M, N, K, fmt_block=32, out_bytes=2, include_c=True):
    """Algorithmic bytes of a GEMM on pre-quantised operands: codes (0.5 B per
    value) and one scale byte per block of each operand read once, C written
    once."""
    ab = (M + N) * K * 0.5 + (M + N) * (K // fmt_block)
    return ab + (M * N * out_bytes if include_c else 0)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="mxfp4_8192")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def cpu_baseline_gemm(a, b, K, budget_s=12.0):
    """The oracle (quantise + FP64 GEMM) on a slab of the 8192^3 workload: a
    few rows of A against a few rows of B, sized to roughly `budget_s` seconds;
    reported in TFLOP/s of the full problem's arithmetic."""
    import oracle
    rows = 8
    t0 = time.perf_counter()
    ra = oracle.quantize(a[:rows], oracle.FMT_MXFP4)
    rb = oracle.quantize(b[:rows], oracle.FMT_MXFP4)
    oracle.gemm(ra[0], ra[1], rb[0], rb[1], rows, rows, K, oracle.FMT_MXFP4)
    dt = time.perf_counter() - t0
    cols = int(max(8, min(4096, rows * budget_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    ra = oracle.quantize(a[:64], oracle.FMT_MXFP4)
    rb = oracle.quantize(b[:cols], oracle.FMT_MXFP4)
    oracle.gemm(ra[0], ra[1], rb[0], rb[1], 64, cols, K, oracle.FMT_MXFP4)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": gemm_flops(64, cols, K) / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "oracle MXFP4 quantise of 64 rows of A and %d rows of B plus FP64 GEMM 64x%dx%d "
                      "(%.1f s)" % (cols, cols, K, dt)}


def bench_mxfp4_8192(args, torch, fp4):
    import synth
    n = 8192
    a, b = synth.mxfp4_8192(n)
    cpu = None if args.no_cpu_baseline else cpu_baseline_gemm(a, b, n)
    qa = [fp4.quantize(torch.from_numpy(a).cuda(), fp4.MXFP4)]
    qb = [fp4.quantize(torch.from_numpy(b).cuda(), fp4.MXFP4)]
    del a, b
    for _ in range(ROTATE - 1):
        qa.append(fp4.Quantized(qa[0].codes.clone(), qa[0].scales.clone(), None, fp4.MXFP4, n, n))
        qb.append(fp4.Quantized(qb[0].codes.clone(), qb[0].scales.clone(), None, fp4.MXFP4, n, n))
    C = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        fp4.gemm(qa[i % ROTATE], qb[i % ROTATE], out=C)

    return step, cpu, dict(M=n, N=n, K=n)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import block_scaled_fp4_03_amd as fp4
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload != "mxfp4_8192":
        raise SystemExit("unknown workload " + args.workload)
    step, cpu, shp = bench_mxfp4_8192(args, torch, fp4)
    M, N, K = shp["M"], shp["N"], shp["K"]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = gemm_flops(M, N, K)
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "FP4 GEMM TFLOPS & % MXFP4 MFMA peak; decode-shape HBM GB/s & % peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": "mxfp4_gemm_8192x8192x8192", "M": M, "N": N, "K": K, "out": "bf16",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP4_TFLOPS, 4), "traffic": None,
                     "kernel": "gemm_mx_kernel"},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

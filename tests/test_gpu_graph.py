"""Quantise + GEMM steps captured in a HIP graph: every replay (with eager work
and synchronisations in between) must reproduce the eager result bit for bit,
and the eager result must agree with the oracle.  The NVFP4 steps include the
tensor-amax reduction, which keeps a self-resetting counter in the workspace,
so a replay that saw a stale counter would differ."""
import numpy as np
import pytest

import synth
from gpu_helpers import assert_gemm_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _capture(step, n):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            step()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, out, ref, eager_noise):
    import torch
    for rep in range(4):
        out.zero_()
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), "replay %d differs from eager" % rep


@pytest.mark.parametrize("M,K", [(1, 2048), (8, 2048), (32, 2048), (32, 8192)])
def test_graph_nvfp4_decode(orc, M, K):
    """Quantise X + decode GEMV captured in a graph and replayed; (32, 8192)
    takes the one-launch quantiser whose workgroups exchange the maximum
    through the workspace (512 KB of X), which every replay must leave zero."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    N = 1024
    w = synth.gaussian(2, (N, K), std=0.02, bernoulli=0.001)
    x = synth.to_bf16_bits(synth.gaussian(202 + M, (M, K)))
    say("graph nvfp4 decode M=%d N=%d K=%d" % (M, N, K))
    qw = fp4.quantize(to_dev(w), fp4.NVFP4)
    xd = to_dev(x)
    qx = fp4.quantize(xd, fp4.NVFP4)
    wsq = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, M, 0, K)
    wsg = fp4.workspace(fp4.OP_GEMM, fp4.NVFP4, M, N, K)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        fp4.quantize(xd, fp4.NVFP4, ws=wsq, out=qx)
        fp4.gemm(qx, qw, out=C, ws=wsg)

    step()
    torch.cuda.synchronize()
    ref = C.clone()
    rx = orc.quantize(x, orc.FMT_NVFP4)
    rw = orc.quantize(w, orc.FMT_NVFP4)
    np.testing.assert_array_equal(to_host(qx.codes), rx[0])
    Cref, T = orc.gemm(rx[0], rx[1], rw[0], rw[1], M, N, K, orc.FMT_NVFP4, tsA=rx[3], tsB=rw[3])
    assert_gemm_close(orc, to_host(C), Cref, T, True, "eager decode M=%d" % M)

    g = _capture(step, 3)
    other = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    _replay_and_check(g, C, ref, lambda: fp4.gemm(fp4.quantize(other, fp4.NVFP4), qw))


@pytest.mark.parametrize("M", [1, 8])
def test_graph_nvfp4_fused_decode(orc, M):
    """The one-kernel decode step (activation quantised inside) under graph
    replay; its result equals the two-call path's bits."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    N, K = 1024, 2048
    w = synth.gaussian(3, (N, K), std=0.02, bernoulli=0.001)
    x = synth.to_bf16_bits(synth.gaussian(203 + M, (M, K)))
    say("graph fused decode M=%d N=%d K=%d" % (M, N, K))
    qw = fp4.quantize(to_dev(w), fp4.NVFP4)
    xd = to_dev(x)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        fp4.gemm_nvfp4_act(xd, qw, out=C)

    step()
    torch.cuda.synchronize()
    ref = C.clone()
    C2 = fp4.gemm(fp4.quantize(xd, fp4.NVFP4), qw, out_dtype=torch.bfloat16)
    assert torch.equal(ref.view(torch.int16), C2.view(torch.int16))
    g = _capture(step, 3)
    other = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    _replay_and_check(g, C, ref, lambda: fp4.gemm_nvfp4_act(other, qw))


def test_graph_mxfp4_small(orc):
    import block_scaled_fp4_03_amd as fp4
    import torch
    a, b = synth.mxfp4_256()
    say("graph mxfp4 256^3")
    xa, xb = to_dev(a), to_dev(b)
    qa, qb = fp4.quantize(xa, fp4.MXFP4), fp4.quantize(xb, fp4.MXFP4)
    C = torch.empty((256, 256), dtype=torch.float32, device="cuda")

    def step():
        fp4.quantize(xa, fp4.MXFP4, out=qa)
        fp4.quantize(xb, fp4.MXFP4, out=qb)
        fp4.gemm(qa, qb, out=C)

    step()
    torch.cuda.synchronize()
    ref = C.clone()
    ra, rb = orc.quantize(a, orc.FMT_MXFP4), orc.quantize(b, orc.FMT_MXFP4)
    Cref, T = orc.gemm(ra[0], ra[1], rb[0], rb[1], 256, 256, 256, orc.FMT_MXFP4)
    assert_gemm_close(orc, to_host(C), Cref, T, False, "eager 256^3")

    g = _capture(step, 2)
    other = torch.randn(256, 256, device="cuda")
    _replay_and_check(g, C, ref, lambda: fp4.gemm(fp4.quantize(other, fp4.MXFP4), qb))


def test_graph_w4a8_step(orc):
    """BF16 activations -> MXFP8, times MXFP4 weights (fp4_gemm_w4a8) with
    bias and ReLU, captured twice in one graph; every replay equals the eager
    result, which is checked against the oracle's exact values (grid data:
    every product fits the matrix core's window and every sum is exact)."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    M, N, K = 96, 320, 512
    g = synth.rng(71)
    a = ((g.integers(0, 16, (M, K)) * 0.25) * np.where(g.random((M, K)) < 0.5, -1, 1)).astype(np.float32)
    a[:, ::32] = 3.75
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    w = (grid[g.integers(0, 8, (N, K))] * np.where(g.random((N, K)) < 0.5, -1, 1)).astype(np.float32)
    w[:, ::32] = 6.0
    bias = (g.integers(-64, 64, N) * 0.25).astype(np.float32)
    say("graph w4a8")
    xa = to_dev(synth.to_bf16_bits(a))
    qw = fp4.quantize(to_dev(w), fp4.MXFP4)
    qa = fp4.quantize(xa, fp4.MXFP8)
    bd = to_dev(bias)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        fp4.quantize(xa, fp4.MXFP8, out=qa)
        fp4.gemm_w4a8(qa, qw, bias=bd, act=fp4.ACT_RELU, out=C)

    step()
    torch.cuda.synchronize()
    ref = C.clone()
    ra = orc.quantize(synth.to_bf16_bits(a), orc.FMT_MXFP8)
    rw = orc.quantize(w, orc.FMT_MXFP4)
    Cref, _ = orc.gemm_mixed(ra[0], ra[1], orc.FMT_MXFP8, rw[0], rw[1], orc.FMT_MXFP4, M, N, K)
    np.testing.assert_array_equal(to_host(C), orc.epilogue(Cref, bias, orc.ACT_RELU))

    gr = _capture(step, 2)
    other = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    _replay_and_check(gr, C, ref, lambda: fp4.gemm_w4a8(fp4.quantize(other, fp4.MXFP8), qw))


def test_graph_grouped_moe_step(orc):
    """The MoE step at a small size -- BF16 tokens -> MXFP4, then the grouped
    GEMM with its workspace (two kernels: the copy of the routed rows into
    expert order, the GEMM) -- captured twice in one graph; every replay
    equals the eager result, which is checked against the oracle."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    counts = np.array([70, 0, 257, 3, 33])
    E, N, K, T_rows = counts.size, 264, 544, 120
    row_idx, off = synth.moe_routing(counts, tokens=T_rows, seed=21)
    x = synth.to_bf16_bits(synth.gaussian(22, (T_rows, K)))
    say("graph grouped moe step")
    xd = to_dev(x)
    qx = fp4.quantize(xd, fp4.MXFP4)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, fp4.fp4_scale_bytes(0, N, K)), dtype=torch.uint8, device="cuda")
    wsr = []
    for e in range(E):
        w = synth.gaussian(23 + e, (N, K), std=0.02)
        fp4.quantize(to_dev(w), 0, out=fp4.Quantized(codes[e], scales[e], None, 0, N, K))
        wsr.append(w)
    total = int(off[-1])
    ri, go = torch.from_numpy(row_idx).cuda(), torch.from_numpy(off).cuda()
    ws = torch.empty(fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, 0, total, N, K, E), dtype=torch.uint8,
                     device="cuda")
    C = torch.empty((total, N), dtype=torch.float32, device="cuda")

    def step():
        fp4.quantize(xd, fp4.MXFP4, out=qx)
        fp4.gemm_grouped(qx, ri, go, codes, scales, N, K, 0, out=C, ws=ws)

    step()
    torch.cuda.synchronize()
    ref = C.clone()
    rx = orc.quantize(x, orc.FMT_MXFP4)
    B = to_host(codes).reshape(-1)
    sB = to_host(scales).reshape(-1)
    rows = np.repeat(np.arange(total), N)
    cols = np.tile(np.arange(N), total)
    Cref, T = orc.gemm_grouped_sampled(rx[0], rx[1], T_rows, row_idx, off, B, sB, N, K, orc.FMT_MXFP4, rows, cols)
    assert_gemm_close(orc, to_host(C).reshape(-1), Cref, T, False, "eager grouped")

    g = _capture(step, 2)
    other = torch.randn(T_rows, K, device="cuda")
    _replay_and_check(g, C, ref, lambda: fp4.gemm_grouped(fp4.quantize(other, fp4.MXFP4), ri, go, codes, scales, N,
                                                          K, 0, ws=ws, out_dtype=torch.float32))

"""The oracle's quantiser and matrix product pinned to what the pages fix:

  * the glossary's worked example (Ultralytics "FP4", "How FP4 works"): its
    printed mean absolute errors, reproduced from the same seed-0 vector;
  * the error ordering whole-tensor > 32-block > 16-block in every mode;
  * block max mapped to 6, power-of-two MXFP4 scales, NVFP4 two-level scales
    (NVFP4 video transcript);
  * the GEMM as FP32-accumulated product of scaled operands ("Rubin FP4 GEMM
    deep dive", §3.1, §4.2): closed forms on hand-built operands and numpy's
    matmul of dequantised operands on small shapes.
"""
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_mae():
    out = {}
    with open(os.path.join(GOLDEN, "page_mae.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                b, v = line.split()
                out[int(b)] = float(v)
    return out


def test_page_worked_example_reproduced(orc):
    x = synth.page_vector()
    assert x.size == 4096
    for block, printed in _page_mae().items():
        got = orc.block_mae(x, block, orc.MAE_PAGE)
        assert round(got, 4) == printed, (block, got, printed)


def test_nvfp4_whole_tensor_block_equals_page_recipe(orc):
    # One block holding the whole tensor: its E4M3 scale is 448 and
    # 448 * s_t = amax/6, so the two-level recipe collapses to the page's.
    x = synth.page_vector()
    assert round(orc.block_mae(x, 4096, orc.MAE_NVFP4), 4) == _page_mae()[4096]


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("which", ["page", "mxfp4_256"])
def test_error_falls_as_blocks_shrink(orc, mode, which):
    x = synth.page_vector() if which == "page" else synth.mxfp4_256_vector()
    e = [orc.block_mae(x, b, mode) for b in (4096, 32, 16)]
    assert e[0] > e[1] > e[2], e


def _grid():
    return np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _codes_unpacked(codes):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def _canon_from_tiled(orc, fmt, scales, rows, K):
    KB = K // orc.block_size(fmt)
    return np.array([[scales[orc.scale_offset(fmt, rows, K, r, b)] for b in range(KB)] for r in range(rows)],
                    np.uint8)


@pytest.mark.parametrize("fmt", [0, 2])
def test_mxfp4_scales_are_powers_of_two_and_max_maps_near_6(orc, fmt):
    x = synth.gaussian(11, (64, 256), every=97)
    codes, scales, canon, ts = orc.quantize(x, fmt)
    assert ts == 1.0
    np.testing.assert_array_equal(_canon_from_tiled(orc, fmt, scales, 64, 256), canon)
    c = _codes_unpacked(codes).reshape(64, 8, 32)
    blocks = x.reshape(64, 8, 32)
    amax = np.abs(blocks).max(axis=2)
    e = canon.astype(np.int64) - 127
    # the decoded scale is a power of two and the block max lands on 4 or 6
    ymax = amax / np.ldexp(1.0, e)
    if fmt == 0:
        assert np.all((ymax > 3.0) & (ymax <= 6.0))
    else:
        assert np.all((ymax >= 4.0) & (ymax < 8.0))
    imax = np.abs(blocks).argmax(axis=2)
    cmax = np.take_along_axis(c & 7, imax[..., None], axis=2)[..., 0]
    # the block max rounds to 3, 4 or 6 (ceil rule, y in (3, 6]) or 4 or 6
    # (floor rule, y in [4, 8) saturating at 6)
    assert np.all(cmax >= (5 if fmt == 0 else 6))
    # an amax of exactly 6*2^j gives scale 2^j and code 7
    x2 = np.zeros((1, 32), np.float32)
    x2[0, 5] = np.float32(6.0 * 2.0 ** -3)
    x2[0, 7] = -0.1
    codes2, _, canon2, _ = orc.quantize(x2, fmt)
    assert canon2[0, 0] == 127 - 3
    assert _codes_unpacked(codes2)[0, 5] == 7


def test_nvfp4_block_max_gets_code_7(orc):
    x = synth.row_scaled_gaussian(12, 64, 512)
    codes, scales, canon, ts = orc.quantize(x, orc.FMT_NVFP4)
    assert ts == np.float32(np.abs(x).max()) / np.float32(2688.0)
    c = _codes_unpacked(codes).reshape(64, 32, 16)
    blocks = np.abs(x.reshape(64, 32, 16))
    imax = blocks.argmax(axis=2)
    cmax = np.take_along_axis(c & 7, imax[..., None], axis=2)[..., 0]
    normal = canon >= 8  # E4M3 exponent field > 0: relative error <= 2^-4
    assert normal.sum() > 1000
    assert np.all(cmax[normal] == 7)
    # the block that holds the tensor max gets the largest finite E4M3 scale
    r, k = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert canon[r, k // 16] == 0x7E


def test_nvfp4_quantizer_steps_with_torch_e4m3(orc):
    """Per block: r = (amax/6)/s_t in FP32, E4M3 by torch's cast, divisor
    d = E4M3(r)*s_t in FP32, code = nearest grid point of |x|/d."""
    import torch
    x = synth.gaussian(13, (32, 128), std=0.3, every=41)
    codes, scales, canon, ts = orc.quantize(x, orc.FMT_NVFP4)
    f32 = np.float32
    amax_t = np.abs(x).max()
    assert ts == f32(amax_t) / f32(2688.0)
    blocks = x.reshape(32, 8, 16)
    amax = np.abs(blocks).max(axis=2).astype(f32)
    r = (amax / f32(6.0)) / f32(ts)
    sb = torch.from_numpy(r).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(canon, sb.view(torch.uint8).numpy())
    d = sb.to(torch.float32).numpy() * f32(ts)
    y = (np.abs(blocks) / d[..., None]).astype(f32)
    dist = np.abs(y[..., None].astype(np.float64) - _grid())
    srt = np.sort(dist, axis=-1)
    tie = srt[..., 0] == srt[..., 1]
    ref = np.argmin(dist, axis=-1)
    got = (_codes_unpacked(codes).reshape(32, 8, 16) & 7)
    assert not tie.any()
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_quantized_value_is_nearest_grid_point(orc, fmt):
    x = synth.gaussian(14, (16, 512), every=33)
    codes, scales, canon, ts = orc.quantize(x, fmt)
    bs = orc.block_size(fmt)
    deq = orc.dequantize(codes, scales, 1.0, fmt, 16, 512).astype(np.float64)
    if fmt == 1:
        s = np.array([[orc.e4m3_value(b) for b in row] for row in canon]) * ts
    else:
        s = np.ldexp(1.0, canon.astype(np.int64) - 127)
    s = np.repeat(s, bs, axis=1)
    grid = _grid()
    # the chosen magnitude is at least as close to |x|/s as any grid point
    y = np.abs(x.astype(np.float64)) / s
    chosen = np.abs(deq) / (s / (ts if fmt == 1 else 1.0))
    best = np.abs(y[..., None] - grid).min(axis=-1)
    assert np.all(np.abs(chosen - y) <= best + 1e-12 * np.maximum(1, y))
    # sign is the input's sign bit
    signs = (_codes_unpacked(codes) >> 3).astype(bool)
    np.testing.assert_array_equal(signs, np.signbit(x))


def test_dequantize_is_grid_times_scale(orc):
    x = synth.gaussian(15, (8, 64))
    codes, scales, canon, _ = orc.quantize(x, orc.FMT_MXFP4)
    c = _codes_unpacked(codes)
    grid = _grid()
    ref = np.where(c >= 8, -1.0, 1.0) * grid[c & 7] * np.repeat(np.ldexp(1.0, canon.astype(np.int64) - 127), 32,
                                                                  axis=1)
    np.testing.assert_array_equal(orc.dequantize(codes, scales, 1.0, 0, 8, 64), ref.astype(np.float32))
    bf = orc.dequantize(codes, scales, 1.0, 0, 8, 64, out_bf16=True)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bf), ref.astype(np.float32))  # exact in BF16


def test_nvfp4_dequantize_applies_tensor_scale_once(orc):
    x = synth.gaussian(16, (4, 64), std=5.0)
    codes, scales, canon, ts = orc.quantize(x, orc.FMT_NVFP4)
    c = _codes_unpacked(codes)
    v = np.where(c >= 8, -1.0, 1.0) * _grid()[c & 7] * np.repeat(
        np.array([[orc.e4m3_value(b) for b in row] for row in canon]), 16, axis=1)
    ref = (v.astype(np.float32) * np.float32(ts)).astype(np.float32)  # exact product, one FP32 rounding
    np.testing.assert_array_equal(orc.dequantize(codes, scales, ts, 1, 4, 64), ref)


def test_zero_and_negative_zero(orc):
    x = np.zeros((2, 32), np.float32)
    x[1, 3] = -0.0
    for fmt in (0, 1, 2):
        codes, scales, canon, ts = orc.quantize(x, fmt)
        assert np.all(canon == 0)
        c = _codes_unpacked(codes)
        assert c[1, 3] == 8 and np.all(np.delete(c.reshape(-1), 32 + 3) == 0)
        if fmt == 1:
            assert ts == 1.0


def test_bf16_input_is_its_fp32_value(orc):
    x = synth.to_bf16_bits(synth.gaussian(17, (8, 128), every=50))
    xf = synth.bf16_bits_to_f32(x)
    for fmt in (0, 1):
        a = orc.quantize(x, fmt)
        b = orc.quantize(xf, fmt)
        for u, v in zip(a[:3], b[:3]):
            np.testing.assert_array_equal(u, v)
        assert a[3] == b[3]


# ---- matrix product ------------------------------------------------------
def _pack(codes4):
    codes4 = np.asarray(codes4, np.uint8)
    return (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)


def _scales_const(orc, fmt, rows, K, byte):
    s = np.zeros(orc.scale_bytes(fmt, rows, K), np.uint8)
    for r in range(rows):
        for b in range(K // orc.block_size(fmt)):
            s[orc.scale_offset(fmt, rows, K, r, b)] = byte
    return s


@pytest.mark.parametrize("fmt,unit", [(0, 127), (1, 0x38)])
def test_gemm_closed_forms(orc, fmt, unit):
    M, N, K = 3, 5, 256
    # all elements 6 (code 7), unit scales: C = 36*K
    A = _pack(np.full((M, K), 7))
    B = _pack(np.full((N, K), 7))
    sA = _scales_const(orc, fmt, M, K, unit)
    sB = _scales_const(orc, fmt, N, K, unit)
    C, T = orc.gemm(A, sA, B, sB, M, N, K, fmt)
    np.testing.assert_array_equal(C, np.full((M, N), 36.0 * K))
    np.testing.assert_array_equal(T, C)
    # tensor scales multiply the result
    C2, _ = orc.gemm(A, sA, B, sB, M, N, K, fmt, tsA=0.5, tsB=3.0)
    np.testing.assert_array_equal(C2, 1.5 * C)
    # alternating signs along K cancel exactly: +6 -6 +6 ...
    alt = np.tile(np.array([7, 15], np.uint8), (N, K // 2))
    C3, T3 = orc.gemm(A, sA, _pack(alt), sB, M, N, K, fmt)
    np.testing.assert_array_equal(C3, 0.0)
    np.testing.assert_array_equal(T3, 36.0 * K)
    # one-hot: A[1, 70] = 1.5 (code 3), B[4, 70] = -4 (code 14), scales 2^3, 2^-2
    a1 = np.zeros((M, K), np.uint8)
    b1 = np.zeros((N, K), np.uint8)
    a1[1, 70] = 3
    b1[4, 70] = 14
    if fmt == 0:
        sA1 = _scales_const(orc, fmt, M, K, 127 + 3)
        sB1 = _scales_const(orc, fmt, N, K, 127 - 2)
        want = 1.5 * -4.0 * 2.0 ** 3 * 2.0 ** -2
    else:
        sA1 = _scales_const(orc, fmt, M, K, 0x50)   # 2^3
        sB1 = _scales_const(orc, fmt, N, K, 0x2D)   # 1.625 * 2^-2
        want = 1.5 * -4.0 * 8.0 * 1.625 * 0.25
    C4, _ = orc.gemm(_pack(a1), sA1, _pack(b1), sB1, M, N, K, fmt)
    ref = np.zeros((M, N))
    ref[1, 4] = want
    np.testing.assert_array_equal(C4, ref)


def test_gemm_block_scale_doubling_adds_that_block(orc):
    fmt, M, N, K = 0, 2, 3, 128
    x = synth.gaussian(18, (M, K))
    w = synth.gaussian(19, (N, K))
    A, sA, cA, _ = orc.quantize(x, fmt)
    B, sB, _, _ = orc.quantize(w, fmt)
    C, _ = orc.gemm(A, sA, B, sB, M, N, K, fmt)
    off = orc.scale_offset(fmt, M, K, 1, 2)  # row 1, block 2 (K 64..95)
    sA2 = sA.copy()
    sA2[off] += 1
    C2, _ = orc.gemm(A, sA2, B, sB, M, N, K, fmt)
    deqA = orc.dequantize(A, sA, 1.0, fmt, M, K).astype(np.float64)
    deqB = orc.dequantize(B, sB, 1.0, fmt, N, K).astype(np.float64)
    part = deqA[1, 64:96] @ deqB[:, 64:96].T
    np.testing.assert_array_equal(C2[0], C[0])
    np.testing.assert_allclose(C2[1] - C[1], part, rtol=0, atol=1e-12 * np.abs(part).max())


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 7, 64), (8, 3, 128), (16, 16, 256)])
def test_gemm_equals_numpy_matmul_of_dequantised(orc, fmt, M, N, K):
    x = synth.gaussian(20 + M, (M, K), every=13)
    w = synth.gaussian(30 + N, (N, K), std=0.1)
    A, sA, _, tA = orc.quantize(x, fmt)
    B, sB, _, tB = orc.quantize(w, fmt)
    C, T = orc.gemm(A, sA, B, sB, M, N, K, fmt, tsA=tA, tsB=tB)
    dA = orc.dequantize(A, sA, 1.0, fmt, M, K).astype(np.float64)  # exact without tensor scale
    dB = orc.dequantize(B, sB, 1.0, fmt, N, K).astype(np.float64)
    ref = (dA @ dB.T) * tA * tB
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(T, (np.abs(dA) @ np.abs(dB).T) * tA * tB, rtol=1e-12, atol=1e-300)
    # sampled variant agrees element for element
    rows = np.array([0, M - 1, M // 2])
    cols = np.array([N - 1, 0, N // 2])
    Cs, Ts = orc.gemm_sampled(A, sA, B, sB, M, N, K, fmt, rows, cols, tsA=tA, tsB=tB)
    np.testing.assert_array_equal(Cs, C[rows, cols])
    np.testing.assert_array_equal(Ts, T[rows, cols])


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_equals_per_expert_gemm(orc, fmt):
    """The grouped oracle equals the dense oracle on each expert's gathered
    rows.  NVFP4: the gathered rows are quantised under the whole token
    matrix's tensor scale (so their codes and block scales are those of the
    whole matrix), and each expert's rows use that expert's tensor scale."""
    E, T_rows, N, K = 4, 24, 16, 96
    counts = np.array([5, 0, 17, 2])
    row_idx, off = synth.moe_routing(counts, tokens=T_rows, seed=1)
    x = synth.gaussian(40, (T_rows, K))
    A, sA, _, tsA = orc.quantize(x, fmt)
    Bs, sBs, tsBs = [], [], []
    for e in range(E):
        b, s, _, t = orc.quantize(synth.gaussian(50 + e, (N, K), std=0.02 * (1 + e)), fmt)
        Bs.append(b)
        sBs.append(s)
        tsBs.append(t)
    B = np.concatenate([b.reshape(-1) for b in Bs])
    sB = np.concatenate(sBs)
    for e in range(E):
        if counts[e] == 0:
            continue
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.repeat(np.arange(lo, hi), N)
        cols = np.tile(np.arange(N), hi - lo)
        C, _ = orc.gemm_grouped_sampled(A, sA, T_rows, row_idx, off, B, sB, N, K, fmt, rows, cols,
                                        tsA=tsA, tsB=tsBs[e])
        g = row_idx[lo:hi]
        Ag = orc.quantize(x[g], fmt, tensor_scale=tsA if fmt == 1 else None)
        Ce, _ = orc.gemm(Ag[0], Ag[1], Bs[e], sBs[e], len(g), N, K, fmt, tsA=tsA, tsB=tsBs[e])
        np.testing.assert_array_equal(C.reshape(hi - lo, N), Ce)


def test_tolerance_check_semantics(orc):
    Cref = np.array([1.0, -2.0, 0.0, 100.0])
    T = np.array([10.0, 10.0, 0.0, 1000.0])
    ok = orc.gemm_within_tolerance(np.array([1.0 + 9e-5, -2.0 - 1.1e-4, 0.0, 100.0]), Cref, T)
    np.testing.assert_array_equal(ok, [True, False, True, True])
    bf = orc.f32_to_bf16_bits(np.array([1.0, -2.0, 0.0, 100.0], np.float32))
    assert orc.gemm_within_tolerance(bf, Cref, T, out_bf16=True).all()
    bad = orc.f32_to_bf16_bits(np.array([1.0078125, -2.0, 0.0, 100.0], np.float32))
    np.testing.assert_array_equal(orc.gemm_within_tolerance(bad, Cref, T, out_bf16=True),
                                  [False, True, True, True])


def test_epilogue_bias_relu_hand_case(orc):
    """Epilogue ("Rubin FP4 GEMM deep dive" §3.2, §4.2): + bias per column,
    ReLU, one rounding to FP32 -- checked on values worked out by hand."""
    C = np.array([[1.5, -2.0, 0.0], [-0.0, 3.0, -0.5]])
    b = np.array([0.25, -1.0, 0.5], np.float32)
    np.testing.assert_array_equal(orc.epilogue(C, b, orc.ACT_NONE), [[1.75, -3.0, 0.5], [0.25, 2.0, 0.0]])
    out = orc.epilogue(C, b, orc.ACT_RELU)
    np.testing.assert_array_equal(out, [[1.75, 0.0, 0.5], [0.25, 2.0, 0.0]])
    assert not np.signbit(out).any()                      # ReLU gives +0, never -0
    # Without bias -0 passes through unchanged (no addition); ReLU turns it into +0.
    z = np.array([[-0.0, -3.0]])
    assert np.signbit(orc.epilogue(z, None, orc.ACT_NONE)[0, 0])
    assert not np.signbit(orc.epilogue(z, None, orc.ACT_RELU)).any()
    # With a bias of +0, -0 + 0 = +0 (IEEE round to nearest).
    assert not np.signbit(orc.epilogue(z, np.zeros(2, np.float32), orc.ACT_NONE)[0, 0])


def test_epilogue_rounds_once_to_fp32(orc):
    """The sum is formed in FP64 and rounded to FP32 once: 1 + 2^-24 + 2^-40
    lies above the midpoint between 1 and 1 + 2^-23, so it rounds up (rounding
    to FP32 first would land exactly on the midpoint and round to even, 1)."""
    C = np.array([[1.0 + 2.0 ** -24 + 2.0 ** -40, 1.0 + 2.0 ** -24]])
    out = orc.epilogue(C, None, orc.ACT_NONE)
    assert out[0, 0] == np.float32(1.0 + 2.0 ** -23)
    assert out[0, 1] == np.float32(1.0)                   # exact midpoint: ties to even
    b = np.array([2.0 ** -40, 0.0], np.float32)
    out = orc.epilogue(np.array([[1.0 + 2.0 ** -24, 5.0]]), b, orc.ACT_NONE)
    assert out[0, 0] == np.float32(1.0 + 2.0 ** -23)      # the bias tips the midpoint up


def test_epilogue_rejects_wrong_bias_length(orc):
    with pytest.raises(ValueError):
        orc.epilogue(np.zeros((2, 3)), np.zeros(2, np.float32))


# ---- stochastic rounding (NVFP4 video transcript, the training recipe's
# fourth part: 0.3 rounds to 1 with probability 30%, to 0 otherwise) --------
def _u64(v):
    return np.array([np.uint64(int(x) & 0xFFFFFFFFFFFFFFFF) for x in v], dtype=np.uint64)


@pytest.mark.parametrize("counter,key", [([1, 0, 0, 0], [0, 0]), ([6, 0, 0, 0], [7, 0]),
                                         ([123456789, 2 ** 63 + 5, 77, 2 ** 64 - 1], [2 ** 64 - 3, 99]),
                                         ([2 ** 40, 3, 2 ** 62, 9], [0x243F6A8885A308D3, 0x13198A2E03707344])])
def test_philox_matches_numpy(orc, counter, key):
    """The oracle's Philox4x64-10 equals numpy's Philox bit generator, which
    advances its counter before each block (so counter - 1 is passed)."""
    c = _u64(counter)
    before = c.copy()
    before[0] -= np.uint64(1)
    ref = np.random.Philox(counter=before, key=_u64(key)).random_raw(4)
    np.testing.assert_array_equal(orc.philox4x64_10(c, key), ref)


def test_sr_word_layout(orc):
    seed = 0x0123456789ABCDEF
    for i in range(24):
        blk = orc.philox4x64_10([i // 8, 0, 0, 0], [seed, 0])
        w = int(blk[(i % 8) // 2])
        assert orc.sr_word(seed, i) == ((w >> 32) if i % 2 else (w & 0xFFFFFFFF))


def test_sr_mag_exact_probability(orc):
    """Round up iff (r >> 8) < f * 2^24 for y = lo + f (hi - lo): on grid points
    never, above 6 saturate; otherwise exactly ceil(f 2^24) of the 2^24 words."""
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for c, g in enumerate(grid):
        for r in (0, 1 << 8, 0x80000000, 0xFFFFFFFF):
            assert orc.e2m1_sr_mag(g, r) == c
    assert orc.e2m1_sr_mag(6.5, 0) == 7 and orc.e2m1_sr_mag(1e30, 0xFFFFFFFF) == 7
    for lo in range(7):
        glo, ghi = grid[lo], grid[lo + 1]
        for f in (0.25, 0.3, 0.5, 0.75, 2.0 ** -20):
            y = np.float32(glo + f * (ghi - glo))
            n = (float(y) - glo) / (ghi - glo) * 2 ** 24          # exact: y - lo and hi - lo are exact
            k_up = int(np.ceil(n)) - 1                            # largest u index that still rounds up
            assert orc.e2m1_sr_mag(y, k_up << 8) == lo + 1
            assert orc.e2m1_sr_mag(y, (k_up + 1) << 8) == lo
            assert orc.e2m1_sr_mag(y, 0xFF) == lo + 1             # u = 0: up for any y > lo


def test_sr_transcript_example(orc):
    """The transcript's example: 0.3 where the representable neighbours are 0
    and 1 (an MXFP4 block whose maximum 12 gives scale 2, grid step 1 near 0)
    becomes 1 in about 30% of the seeds and 0 otherwise; the mean is 0.3."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 12.0
    x[0, 1:] = 0.3
    vals = []
    for seed in range(4000):
        c, s, _, _ = orc.quantize(x, orc.FMT_MXFP4, sr_seed=seed)
        v = orc.dequantize(c, s, 1.0, orc.FMT_MXFP4, 1, 32)[0, 1:]
        assert set(np.unique(v)) <= {0.0, 1.0}
        vals.append(v)
    p = np.concatenate(vals).mean()
    assert abs(p - 0.3) < 4 * np.sqrt(0.3 * 0.7 / (4000 * 31))


def _neighbours(orc, x, canon, ts, fmt):
    """The two grid points bracketing each element, as signed values: MXFP4
    divisor 2^(byte - 127); NVFP4 divisor E4M3(byte) * s_t (FP32)."""
    bs = orc.block_size(fmt)
    if fmt == orc.FMT_NVFP4:
        e4 = np.array([orc.e4m3_value(int(b)) for b in canon.reshape(-1)], np.float32).reshape(canon.shape)
        d = (e4 * np.float32(ts)).astype(np.float32)
    else:
        d = np.ldexp(np.float32(1), canon.astype(np.int32) - 127).astype(np.float32)
    d = np.repeat(d, bs, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(d > 0, np.abs(x) / d, 0).astype(np.float32)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    lo_i = np.clip(np.searchsorted(grid, y, side="right") - 1, 0, 7)
    hi_i = np.minimum(lo_i + 1, 7)
    hi_i = np.where(grid[lo_i] == y, lo_i, hi_i)
    sgn = np.where(np.signbit(x), -1.0, 1.0)
    scale = d.astype(np.float64)
    return sgn * grid[lo_i] * scale, sgn * grid[hi_i] * scale, sgn * np.minimum(np.abs(x), 6.0 * scale)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_sr_unbiased_and_scales_unchanged(orc, fmt):
    """Every stochastic value is one of the element's two grid neighbours,
    the scales equal the deterministic quantiser's, and over n seeds the mean
    lies within 4 sigma (sigma <= (hi - lo) / (2 sqrt n)) of x -- of x clipped
    to 6 x divisor where the block scale lets an element saturate (the OCP
    rule, or an E4M3 block scale rounded down)."""
    rows, K = 4, 64
    x = synth.gaussian(61, (rows, K))
    c0, s0, canon, ts0 = orc.quantize(x, fmt)
    lo, hi, clipped = _neighbours(orc, x, canon, ts0, fmt)
    n = 400
    acc = np.zeros((rows, K))
    for seed in range(n):
        c, s, _, ts = orc.quantize(x, fmt, sr_seed=seed * 7919 + 1)
        np.testing.assert_array_equal(s, s0)
        assert ts == ts0
        d = orc.dequantize(c, s, ts, fmt, rows, K).astype(np.float64)
        tol = np.abs(hi) * 2.0 ** -20 + 1e-30
        assert (np.minimum(np.abs(d - lo), np.abs(d - hi)) <= tol).all()
        acc += d
    mean = acc / n
    sigma = np.abs(hi - lo) / (2 * np.sqrt(n))
    assert (np.abs(mean - clipped) <= 4 * sigma + np.abs(clipped) * 2.0 ** -20 + 1e-30).all()


def test_sr_reproducible_and_seed_dependent(orc):
    x = synth.gaussian(62, (8, 128))
    a = orc.quantize(x, orc.FMT_NVFP4, sr_seed=5)
    b = orc.quantize(x, orc.FMT_NVFP4, sr_seed=5)
    c = orc.quantize(x, orc.FMT_NVFP4, sr_seed=6)
    np.testing.assert_array_equal(a[0], b[0])
    assert (a[0] != c[0]).any()


# ---- random Hadamard transform and 2-D weight scaling (NVFP4 video
# transcript, the training recipe's third and second parts) ----------------
def test_rht_equals_hadamard_matrix_times_signs(orc):
    """On integer inputs every butterfly sum is exact, so the oracle's FP32
    transform equals (1/4) H16 D x computed with scipy's Hadamard matrix, bit
    for bit; D holds the signs of the columns' Philox words."""
    from scipy.linalg import hadamard
    seed = 424242
    g = synth.rng(90)
    x = g.integers(-50, 50, (5, 64)).astype(np.float32)
    y = orc.rht16(x, seed)
    H = hadamard(16).astype(np.float64)
    d = np.array([-1.0 if orc.sr_word(seed, k) >> 31 else 1.0 for k in range(64)])
    ref = np.concatenate([(0.25 * (H @ (d[16 * b:16 * b + 16] * x[:, 16 * b:16 * b + 16]).T)).T
                          for b in range(4)], axis=1)
    np.testing.assert_array_equal(y, ref.astype(np.float32))
    assert (d > 0).any() and (d < 0).any()


def test_rht_keeps_norms_and_dot_products(orc):
    a = synth.gaussian(91, (4, 256))
    b = synth.gaussian(92, (6, 256))
    ta, tb = orc.rht16(a, 7), orc.rht16(b, 7)
    np.testing.assert_allclose((ta.astype(np.float64) ** 2).sum(1), (a.astype(np.float64) ** 2).sum(1), rtol=1e-6)
    np.testing.assert_allclose(ta.astype(np.float64) @ tb.T.astype(np.float64),
                               a.astype(np.float64) @ b.T.astype(np.float64), rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("fmt", [0, 2])
def test_rht_lowers_quantisation_error_with_outliers(orc, fmt):
    """The transcript's point: with one large value per block the block scale
    is set by the outlier; after the transform the error (same norm in both
    domains, the transform being orthogonal) is smaller.  Holds for MXFP4's
    32-value power-of-two blocks; NVFP4's 16-value E4M3 blocks already place a
    lone outlier well, and there the transform raised the error on every
    outlier density tried (1.1-2.1x)."""
    x = synth.gaussian(93, (64, 512))
    x[:, ::16] *= np.float32(30.0)
    y = orc.rht16(x, 3)

    def err(v):
        c, s, _, ts = orc.quantize(v, fmt)
        return float(((orc.dequantize(c, s, ts, fmt, *v.shape).astype(np.float64) - v) ** 2).sum())

    assert err(y) < 0.7 * err(x)


def test_2d_scales_make_w_and_wt_quantise_alike(orc):
    """2-D scaling: W and W^T dequantise to transposes of each other exactly
    (same 16 x 16 patches, same tensor scale); with 1 x 16 blocks they do not."""
    w = synth.gaussian(94, (48, 64), std=0.02, bernoulli=0.01)
    wt = np.ascontiguousarray(w.T)
    c, s, _, ts = orc.quantize(w, orc.FMT_NVFP4, two_d=True)
    ct, st, _, tst = orc.quantize(wt, orc.FMT_NVFP4, two_d=True)
    assert ts == tst
    d = orc.dequantize(c, s, ts, orc.FMT_NVFP4, 48, 64)
    dt = orc.dequantize(ct, st, tst, orc.FMT_NVFP4, 64, 48)
    np.testing.assert_array_equal(d, dt.T)
    c1, s1, _, _ = orc.quantize(w, orc.FMT_NVFP4)
    c1t, s1t, _, _ = orc.quantize(wt, orc.FMT_NVFP4)
    assert not np.array_equal(orc.dequantize(c1, s1, ts, orc.FMT_NVFP4, 48, 64),
                              orc.dequantize(c1t, s1t, ts, orc.FMT_NVFP4, 64, 48).T)


def test_2d_patch_rows_share_scales(orc):
    w = synth.gaussian(95, (40, 96))          # 40 rows: patch groups of 16, 16 and 8 rows
    _, _, canon, _ = orc.quantize(w, orc.FMT_NVFP4, two_d=True)
    for r0 in (0, 16, 32):
        grp = canon[r0:min(r0 + 16, 40)]
        assert (grp == grp[0]).all()
    # the patch scale is the 1-D scale of the patch's largest block
    _, _, canon1, _ = orc.quantize(w, orc.FMT_NVFP4)
    np.testing.assert_array_equal(canon[32], canon1[32:40].max(axis=0))

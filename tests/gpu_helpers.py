"""Shared helpers of the GPU parity tests: moving seeded host inputs to the
device and results back, and comparing them with the oracle."""
import sys

import numpy as np


def say(msg):
    """Name the case before each GPU step, flushed, so a fault can be placed."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def to_dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:  # BF16 bit patterns
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def to_host(t):
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_gemm_close(orc, C, Cref, T, out_bf16, what=""):
    ok = orc.gemm_within_tolerance(C, Cref, T, out_bf16=out_bf16)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        c = orc.bf16_bits_to_f32(C) if out_bf16 else C
        lines = ["%s: %d / %d outside 1e-5*sum|ab|" % (what, (~ok).sum(), ok.size)]
        for i in idx:
            i = tuple(i)
            lines.append("  at %s: got %r ref %r T %r" % (i, float(c[i]), float(Cref[i]), float(T[i])))
        raise AssertionError("\n".join(lines))


def _f32_down(x):
    """Largest float32 <= x (float64 array)."""
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(-np.inf)), f)


def _f32_up(x):
    """Smallest float32 >= x (float64 array)."""
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f)


def _signed_order(codes):
    """E2M1 codes in the order of their values: -6 < ... < -0.5 < -0 < +0 <
    0.5 < ... < 6 (the oracle's encoder copies the sign, so -0 is its own code)."""
    codes = codes.astype(np.int64)
    mag = codes & 7
    return np.where(codes & 8, -mag - 1, mag)


def _oracle_codes(orc, y):
    """The oracle's E2M1 code of each float32 y: its magnitude code, sign copied."""
    y = np.asarray(y, np.float32)
    mag = orc.e2m1_encode_mag(np.abs(y)).astype(np.int64)
    return mag | (np.signbit(y).astype(np.int64) << 3)


def assert_fp4_output_valid(orc, codes, scales, lo, hi, rows, M, N, ocp, what):
    """codes, scales: the GPU's MXFP4 output (M x N/2 codes, tiled scales);
    rows: the output rows to check; lo, hi (len(rows) x N, float64): each
    element's interval of acceptable FP32 epilogue values.  The oracle's
    exponent rule is non-decreasing in the block maximum, and its E2M1 code is
    non-decreasing (in signed order) in the scaled value, so the outputs some
    v in [lo, hi] gives are exactly those between the ends' outputs."""
    R = len(rows)
    lo32, hi32 = _f32_down(lo), _f32_up(hi)
    absmin = np.where((lo32 <= 0) & (hi32 >= 0), np.float32(0), np.minimum(np.abs(lo32), np.abs(hi32)))
    absmax = np.maximum(np.abs(lo32), np.abs(hi32))
    amax_lo = absmin.reshape(R, N // 32, 32).max(axis=2)
    amax_hi = absmax.reshape(R, N // 32, 32).max(axis=2)
    e_lo = orc.mx_exponent(amax_lo.astype(np.float32), ocp).reshape(R, N // 32)
    e_hi = orc.mx_exponent(amax_hi.astype(np.float32), ocp).reshape(R, N // 32)
    sb = np.array([[scales[orc.scale_offset(0, M, N, int(r), b)] for b in range(N // 32)] for r in rows],
                  np.int64)
    e = sb - 127
    bad = (e < e_lo) | (e > e_hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d / %d scale bytes outside the oracle's; block %s byte %d, allowed "
                             "exponents [%d, %d]" % (what, bad.sum(), bad.size, i, sb[i], e_lo[i], e_hi[i]))
    # Codes: v * 2^-e is exact in FP32 (a power of two; any underflow lands
    # far below E2M1's 0.25 and cannot change a code).
    scale = np.ldexp(np.float64(1.0), -np.repeat(e, 32, axis=1))
    c_lo = _signed_order(_oracle_codes(orc, (lo32.astype(np.float64) * scale).astype(np.float32)))
    c_hi = _signed_order(_oracle_codes(orc, (hi32.astype(np.float64) * scale).astype(np.float32)))
    packed = codes[rows].astype(np.int64)
    got = np.empty((R, N), np.int64)
    got[:, 0::2] = packed & 15
    got[:, 1::2] = packed >> 4
    g = _signed_order(got)
    bad = (g < c_lo) | (g > c_hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d / %d codes outside the oracle's; at %s code %d, allowed order [%d, %d], "
                             "interval [%r, %r]" % (what, bad.sum(), bad.size, i, got[i], c_lo[i], c_hi[i],
                                                    float(lo[i]), float(hi[i])))


def assert_nvfp4_output_valid(orc, codes, scales, lo, hi, rows, M, N, s_t, what):
    """The NVFP4 counterpart of assert_fp4_output_valid, under the given tensor
    scale s_t (FP32): the oracle's block byte E4M3((amax / 6) / s_t) is
    non-decreasing in the block maximum, and its code of |x| / d (d =
    E4M3value(byte) * s_t, FP32; a zero byte gives magnitude 0), sign copied,
    is non-decreasing in x in signed order; so the outputs some v in
    [lo, hi] gives are exactly those between the ends' outputs."""
    R = len(rows)
    st = np.float32(s_t)
    lo32, hi32 = _f32_down(lo), _f32_up(hi)
    absmin = np.where((lo32 <= 0) & (hi32 >= 0), np.float32(0), np.minimum(np.abs(lo32), np.abs(hi32)))
    absmax = np.maximum(np.abs(lo32), np.abs(hi32))
    nb = N // 16
    amax_lo = absmin.reshape(R, nb, 16).max(axis=2).astype(np.float32)
    amax_hi = absmax.reshape(R, nb, 16).max(axis=2).astype(np.float32)
    sb_lo = orc.e4m3_encode((amax_lo / np.float32(6.0)) / st).astype(np.int64)
    sb_hi = orc.e4m3_encode((amax_hi / np.float32(6.0)) / st).astype(np.int64)
    sb = np.array([[scales[orc.scale_offset(1, M, N, int(r), b)] for b in range(nb)] for r in rows], np.int64)
    bad = (sb < sb_lo) | (sb > sb_hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d / %d scale bytes outside the oracle's; block %s byte %d, allowed [%d, %d]"
                             % (what, bad.sum(), bad.size, i, sb[i], sb_lo[i], sb_hi[i]))
    d = (np.array([orc.e4m3_value(int(b)) for b in range(256)], np.float32)[np.repeat(sb, 16, axis=1)] * st)
    d = d.astype(np.float32)
    zero = np.repeat(sb == 0, 16, axis=1)

    def code(x):
        with np.errstate(divide="ignore", invalid="ignore"):
            y = np.where(zero, np.float32(0), np.abs(x) / np.where(zero, np.float32(1), d)).astype(np.float32)
        return _signed_order(_oracle_codes(orc, np.copysign(y, x)))

    c_lo, c_hi = code(lo32), code(hi32)
    packed = codes[rows].astype(np.int64)
    got = np.empty((R, N), np.int64)
    got[:, 0::2] = packed & 15
    got[:, 1::2] = packed >> 4
    g = _signed_order(got)
    bad = (g < c_lo) | (g > c_hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d / %d codes outside the oracle's; at %s code %d, allowed order [%d, %d], "
                             "interval [%r, %r]" % (what, bad.sum(), bad.size, i, got[i], c_lo[i], c_hi[i],
                                                    float(lo[i]), float(hi[i])))

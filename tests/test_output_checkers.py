"""The acceptance checkers the GPU tests use, run on the CPU against the
oracle's own results: they accept every output the oracle gives for a value
inside the acceptance interval, and reject planted mistakes (a code or a
scale byte moved off the oracle's)."""
import numpy as np
import pytest

import synth
from gpu_helpers import assert_fp4_output_valid, assert_nvfp4_output_valid


def _case(orc, seed, M=64, N=256, K=512, act=1):
    a = synth.gaussian(seed, (M, K), every=509)
    b = synth.gaussian(seed + 1, (N, K), std=0.05, bernoulli=0.002)
    ra, rb = orc.quantize(a, 0), orc.quantize(b, 0)
    Cref, T = orc.gemm(ra[0], ra[1], rb[0], rb[1], M, N, K, 0)
    bias = (0.5 * synth.gaussian(seed + 2, (N,))).astype(np.float32)
    lo, hi = Cref - 1e-5 * T + bias, Cref + 1e-5 * T + bias
    lo, hi = lo - np.abs(lo) * 2.0 ** -23, hi + np.abs(hi) * 2.0 ** -23
    if act:
        lo, hi = np.maximum(lo, 0.0), np.maximum(hi, 0.0)
    return Cref, T, bias, lo, hi


@pytest.mark.parametrize("ocp", [False, True])
@pytest.mark.parametrize("act", [0, 1])
def test_fp4_checker_accepts_oracle_values_in_the_interval(orc, ocp, act):
    M, N = 64, 256
    Cref, T, bias, lo, hi = _case(orc, 30 + act, act=act)
    g = np.random.default_rng(1)
    for pick in ("mid", "lo", "hi", "random"):
        if pick == "mid":
            v = orc.epilogue(Cref, bias, act)
        else:
            t = {"lo": 0.0, "hi": 1.0}.get(pick)
            w = g.random(lo.shape) if t is None else np.full(lo.shape, t)
            v = (lo + w * (hi - lo)).astype(np.float32)
            v = np.clip(v, lo.astype(np.float32), hi.astype(np.float32))
            v = np.where(v.astype(np.float64) < lo, np.nextafter(v, np.float32(np.inf)), v)
            v = np.where(v.astype(np.float64) > hi, np.nextafter(v, np.float32(-np.inf)), v)
        codes, scales, _, _ = orc.quantize(np.ascontiguousarray(v, np.float32), 2 if ocp else 0)
        assert_fp4_output_valid(orc, codes, scales, lo, hi, np.arange(M), M, N, ocp, pick)


def test_fp4_checker_rejects_planted_mistakes(orc):
    M, N = 64, 256
    Cref, T, bias, lo, hi = _case(orc, 40)
    v = orc.epilogue(Cref, bias, 1)
    codes, scales, _, _ = orc.quantize(v, 0)
    # A code moved two grid steps up (beyond any rounding the interval allows).
    bad = codes.copy()
    r, c = 5, 17
    nib = (bad[r, c] & 15) & 7
    new = min(nib + 2, 7) if nib < 6 else nib - 2
    bad[r, c] = (bad[r, c] & 0xF0) | new
    with pytest.raises(AssertionError, match="codes"):
        assert_fp4_output_valid(orc, bad, scales, lo, hi, np.arange(M), M, N, False, "planted code")
    # A scale byte one binade up.
    bad_s = scales.copy()
    off = orc.scale_offset(0, M, N, 9, 3)
    bad_s[off] += 1
    with pytest.raises(AssertionError, match="scale bytes"):
        assert_fp4_output_valid(orc, codes, bad_s, lo, hi, np.arange(M), M, N, False, "planted scale")
    # -0 where ReLU gives +0.
    zr, zc = np.argwhere(v == 0)[0]
    bad = codes.copy()
    sh = 4 * (zc & 1)
    bad[zr, zc // 2] |= np.uint8(8 << sh)
    with pytest.raises(AssertionError, match="codes"):
        assert_fp4_output_valid(orc, bad, scales, lo, hi, np.arange(M), M, N, False, "planted -0")


def _nv_ts(orc, Cref, bias, act):
    v = orc.epilogue(Cref, bias, act)
    return float(orc.nvfp4_tensor_scale(np.float32(np.abs(v).max())))


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("ts_kind", ["own", "small", "large"])
def test_nvfp4_checker_accepts_oracle_values_in_the_interval(orc, act, ts_kind):
    M, N = 64, 256
    Cref, T, bias, lo, hi = _case(orc, 50 + act, act=act)
    ts = {"own": _nv_ts(orc, Cref, bias, act), "small": 2.0 ** -14, "large": 0.37}[ts_kind]
    g = np.random.default_rng(2)
    for pick in ("mid", "lo", "hi", "random"):
        if pick == "mid":
            v = orc.epilogue(Cref, bias, act)
        else:
            t = {"lo": 0.0, "hi": 1.0}.get(pick)
            w = g.random(lo.shape) if t is None else np.full(lo.shape, t)
            v = (lo + w * (hi - lo)).astype(np.float32)
            v = np.where(v.astype(np.float64) < lo, np.nextafter(v, np.float32(np.inf)), v)
            v = np.where(v.astype(np.float64) > hi, np.nextafter(v, np.float32(-np.inf)), v)
        codes, scales, _, _ = orc.quantize(np.ascontiguousarray(v, np.float32), 1, tensor_scale=ts)
        assert_nvfp4_output_valid(orc, codes, scales, lo, hi, np.arange(M), M, N, ts, pick)


def test_nvfp4_checker_rejects_planted_mistakes(orc):
    M, N = 64, 256
    Cref, T, bias, lo, hi = _case(orc, 60)
    v = orc.epilogue(Cref, bias, 1)
    ts = _nv_ts(orc, Cref, bias, 1)
    codes, scales, _, _ = orc.quantize(v, 1, tensor_scale=ts)
    bad = codes.copy()
    r, c = 7, 21
    nib = (bad[r, c] & 15) & 7
    new = min(nib + 2, 7) if nib < 6 else nib - 2
    bad[r, c] = (bad[r, c] & 0xF0) | new
    with pytest.raises(AssertionError, match="codes"):
        assert_nvfp4_output_valid(orc, bad, scales, lo, hi, np.arange(M), M, N, ts, "planted code")
    # An E4M3 block scale two steps up (beyond what the interval's maxima give).
    bad_s = scales.copy()
    off = orc.scale_offset(1, M, N, 11, 5)
    bad_s[off] += 2
    with pytest.raises(AssertionError, match="scale bytes"):
        assert_nvfp4_output_valid(orc, codes, bad_s, lo, hi, np.arange(M), M, N, ts, "planted scale")
    # The right codes checked under another tensor scale: the bytes no longer fit.
    with pytest.raises(AssertionError, match="scale bytes"):
        assert_nvfp4_output_valid(orc, codes, scales, lo, hi, np.arange(M), M, N, ts * 2.0, "wrong s_t")

"""fp4_quantize_noalloc (the entry point for callers that cannot allocate)
against fp4_quantize with a caller-given workspace, through the C ABI: the
same codes, scales and tensor scale bit for bit, on two calls in a row (the
second on a smaller input), so the library-held scratch is left clean by the
first call; plus the paths that need no scratch (small NVFP4 input, a given
tensor scale, MXFP4)."""
import numpy as np
import pytest

import synth
from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _q_alloc_free(fp4, torch, x, fmt, rows, K, dt, ts=None):
    codes = torch.empty(rows * (K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty(fp4.fp4_scale_bytes(fmt, rows, K), dtype=torch.uint8, device="cuda")
    t = ts.clone() if ts is not None else torch.empty(1, dtype=torch.float32, device="cuda")
    flags = fp4.TS_GIVEN if ts is not None else 0
    rc = fp4.fp4_quantize_noalloc(x.data_ptr(), fmt, codes.data_ptr(), scales.data_ptr(),
                                  t.data_ptr() if fmt == fp4.NVFP4 else None, rows, K, dt, flags,
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fp4.fp4_status_string(rc)
    return codes, scales, t


def _q_with_ws(fp4, torch, x, fmt, rows, K, dt, ts=None):
    codes = torch.empty(rows * (K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty(fp4.fp4_scale_bytes(fmt, rows, K), dtype=torch.uint8, device="cuda")
    t = ts.clone() if ts is not None else torch.empty(1, dtype=torch.float32, device="cuda")
    flags = fp4.TS_GIVEN if ts is not None else 0
    ws = torch.zeros(64, dtype=torch.uint8, device="cuda")
    rc = fp4.fp4_quantize(x.data_ptr(), fmt, codes.data_ptr(), scales.data_ptr(),
                          t.data_ptr() if fmt == fp4.NVFP4 else None, rows, K, dt, flags, ws.data_ptr(), ws.numel(),
                          torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fp4.fp4_status_string(rc)
    return codes, scales, t


# (rows, K, dtype, fmt): the first two NVFP4 cases exceed 256 KB of input, so
# the tensor maximum goes through the scratch; the second is smaller than
# the first.
CASES = [(777, 4096, "bf16", 1), (300, 1024, "f32", 1), (37, 2048, "bf16", 1), (96, 512, "f32", 0),
         (5000, 256, "bf16", 1)]


@pytest.mark.parametrize("order", [0, 1])
def test_noalloc_equals_workspace_path(orc, order):
    import block_scaled_fp4_03_amd as fp4
    import torch
    cases = CASES if order == 0 else CASES[::-1]
    for i, (rows, K, dt, fmt) in enumerate(cases):
        xh = synth.gaussian(700 + i, (rows, K), std=0.3, bernoulli=0.002)
        if dt == "bf16":
            xh = synth.to_bf16_bits(xh)
        x = to_dev(xh)
        dcode = fp4.BF16 if dt == "bf16" else fp4.F32
        say("noalloc %d x %d %s fmt %d (call %d)" % (rows, K, dt, fmt, i))
        c1, s1, t1 = _q_alloc_free(fp4, torch, x, fmt, rows, K, dcode)
        c0, s0, t0 = _q_with_ws(fp4, torch, x, fmt, rows, K, dcode)
        np.testing.assert_array_equal(to_host(c1), to_host(c0))
        np.testing.assert_array_equal(to_host(s1), to_host(s0))
        if fmt == fp4.NVFP4:
            assert to_host(t1)[0] == to_host(t0)[0]
            r = orc.quantize(xh, fmt)
            assert to_host(t1)[0] == np.float32(r[3])
            np.testing.assert_array_equal(to_host(c1).reshape(rows, K // 2), r[0])
            np.testing.assert_array_equal(to_host(s1), r[1])
        # A given tensor scale takes no scratch either way.
        if fmt == fp4.NVFP4:
            g = torch.tensor([0.0125], dtype=torch.float32, device="cuda")
            c1, s1, _ = _q_alloc_free(fp4, torch, x, fmt, rows, K, dcode, ts=g)
            c0, s0, _ = _q_with_ws(fp4, torch, x, fmt, rows, K, dcode, ts=g)
            np.testing.assert_array_equal(to_host(c1), to_host(c0))
            np.testing.assert_array_equal(to_host(s1), to_host(s0))


def test_noalloc_back_to_back_without_sync(orc):
    """Calls queued back to back on one stream, no host sync between them:
    each finds the scratch cleared by the one before."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    xs = [synth.to_bf16_bits(synth.gaussian(750 + i, (r, 2048), std=s)) for i, (r, s) in
          enumerate([(512, 1.0), (256, 40.0), (129, 0.01)])]
    outs = []
    for i, xh in enumerate(xs):
        say("noalloc back-to-back call %d rows %d" % (i, xh.shape[0]))
        outs.append(_q_alloc_free(fp4, torch, to_dev(xh), fp4.NVFP4, xh.shape[0], 2048, fp4.BF16))
    torch.cuda.synchronize()
    for xh, (c, s, t) in zip(xs, outs):
        r = orc.quantize(xh, fp4.NVFP4)
        assert to_host(t)[0] == np.float32(r[3])
        np.testing.assert_array_equal(to_host(c).reshape(xh.shape[0], 1024), r[0])
        np.testing.assert_array_equal(to_host(s), r[1])

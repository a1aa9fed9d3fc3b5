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

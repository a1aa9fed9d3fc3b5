"""bench.py's algorithmic counts against the figures the deep dive prints
("Rubin FP4 GEMM deep dive" §5.1 and §2.3; tests/golden/page_arithmetic.txt).
The page rounds: its intensity 8155 is 1.37e11 / 16.8e6, the exact codes-only
value is 8192; the check allows the page's own rounding (0.5%)."""
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.txt")


def _page():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


def test_section_5_1_intensity():
    p = _page()
    n = 4096
    flops = bench.gemm_flops(n, n, n)
    assert flops == 2 * n ** 3
    assert flops == pytest.approx(p["s51_flops"], rel=0.005)
    codes = 2 * n * n * 0.5                                   # A and B codes, no scales, no C
    assert codes == pytest.approx(p["s51_bytes"], rel=0.005)
    assert flops / codes == 8192
    assert flops / codes == pytest.approx(p["s51_intensity"], rel=0.005)
    # with the block scales (1 byte per 32 values) and without C, as bench.py counts operands
    ai = bench.arithmetic_intensity(n, n, n, block=32, include_c=False)
    assert ai == pytest.approx(2 * n ** 3 / (2 * (n * n * 0.5 + n * n / 32)))
    assert ai < flops / codes


def test_section_2_3_weight_bytes():
    p = _page()
    n = 10000
    fp4_codes = n * n * 0.5
    assert fp4_codes == pytest.approx(p["s23_fp4_bytes"], rel=0.01)
    assert 2 * n * n == pytest.approx(p["s23_fp16_bytes"], rel=0.01)
    # bench.py's operand bytes add the scales: 1/32 byte per value for MXFP4
    assert bench.fp4_operand_bytes(n, n, 32) == fp4_codes + n * (n // 32)


def test_headline_bytes_and_flops():
    """The 8192^3 counts the roofline uses: 205,520,896 algorithmic bytes
    (codes + scales of A and B, BF16 C) and 1.0995e12 flop."""
    n = 8192
    assert bench.gemm_bytes(n, n, n) == 205520896
    assert bench.gemm_flops(n, n, n) == 1099511627776

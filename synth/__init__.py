"""Seeded synthetic inputs for the FP4 block-scaled quantise / GEMM workloads.

This module only draws numbers: Gaussian operands with outliers, per-row
scales, MoE routing.  It holds none of the quantisation or matrix-product
arithmetic, so that both the HIP path and the CPU oracle can be fed the same
bits from it.

Distributions follow the worked example of the Ultralytics glossary "FP4"
("How FP4 works": a seed-0 N(0,1) vector of 4096 values with every 512th value
multiplied by 20) and the workloads the library is measured on:

  mxfp4_256      A, B 256x256 FP32 N(0,1), flat index % 512 == 0 times 20.
  nvfp4_decode   W 8192x8192 N(0, 0.02^2) with a Bernoulli(0.001) mask times
                 20; X Mx8192 BF16 N(0,1), M in {1, 8, 32}.
  mxfp4_8192     A, B 8192x8192 N(0,1) with a Bernoulli(0.002) mask times 20.
  nvfp4_mlp      A 4096x4096 BF16, W 14336x4096; row i ~ N(0, s_i^2) with
                 s_i = 10^U(-2, 0) (log-uniform in [0.01, 1]).
  mxfp4_moe      32 experts, W_e 5760x2880 (N x K) N(0, 0.02^2); 16384 tokens
                 x 2880 BF16 N(0,1); top-4 routing with Zipf(1.2) expert
                 popularity (seed 0).

Every generator uses numpy's PCG64 with a fixed seed; BF16 data is the
round-to-nearest-even cast of the FP32 draw (torch's CPU cast), returned as
uint16 bit patterns.
"""
import numpy as np

OUTLIER_MULT = 20.0


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x):
    """FP32 -> BF16 (round to nearest even) bit patterns, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def page_vector():
    """The glossary's worked-example input: torch.manual_seed(0);
    torch.randn(4096); every 512th value (index 0, 512, ...) times 20."""
    import torch
    g = torch.Generator().manual_seed(0)
    x = torch.randn(4096, generator=g)
    x[::512] *= 20
    return x.numpy().astype(np.float32)


def gaussian(seed, shape, std=1.0, every=None, bernoulli=None, mult=OUTLIER_MULT):
    """N(0, std^2) FP32 with outliers: either every `every`-th flat index
    (starting at 0) or a Bernoulli(`bernoulli`) mask, multiplied by `mult`."""
    g = rng(seed)
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    flat = x.reshape(-1)
    if every is not None:
        flat[::every] *= np.float32(mult)
    if bernoulli is not None:
        mask = g.random(flat.size, dtype=np.float32) < bernoulli
        flat[mask] *= np.float32(mult)
    return x


def row_scaled_gaussian(seed, rows, cols, lo_exp=-2.0, hi_exp=0.0):
    """Row i ~ N(0, s_i^2), s_i = 10^U(lo_exp, hi_exp)."""
    g = rng(seed)
    s = np.power(10.0, g.uniform(lo_exp, hi_exp, rows)).astype(np.float32)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    x *= s[:, None]
    return x


# ---- the measured workloads -------------------------------------------------
def mxfp4_256():
    """(A, B) FP32 256x256, every 512th flat element x20; seed 1."""
    g_a = gaussian(1, (256, 256), every=512)
    g_b = gaussian(101, (256, 256), every=512)
    return g_a, g_b


def mxfp4_256_vector():
    """A 4096-vector of the same law as mxfp4_256's operands (seed 1001)."""
    return gaussian(1001, (4096,), every=512)


def nvfp4_decode_weight(N=8192, K=8192):
    return gaussian(2, (N, K), std=0.02, bernoulli=0.001)


def nvfp4_decode_act(M, K=8192, seed=202):
    return to_bf16_bits(gaussian(seed + M, (M, K)))


def mxfp4_8192(n=8192):
    return gaussian(3, (n, n), bernoulli=0.002), gaussian(303, (n, n), bernoulli=0.002)


def nvfp4_mlp(M=4096, N=14336, K=4096):
    """(A bf16 bits MxK, W fp32 NxK)."""
    return to_bf16_bits(row_scaled_gaussian(4, M, K)), row_scaled_gaussian(404, N, K)


# ---- MoE routing ------------------------------------------------------------
def zipf_counts(E=32, total=65536, cap=16384, a=1.2, seed=0):
    """Per-expert row counts: z = Zipf(a) draws (one per expert, seed 0),
    a largest-remainder apportionment of `total` proportional to z, each count
    capped at `cap` with the overflow handed to the remaining experts in
    proportion to their weights."""
    z = np.random.default_rng(seed).zipf(a, E).astype(np.float64)
    counts = np.zeros(E, np.int64)
    free = np.ones(E, bool)
    remaining = total
    while remaining > 0:
        w = np.where(free, z, 0.0)
        share = remaining * w / w.sum()
        base = np.floor(share).astype(np.int64)
        rem = remaining - base.sum()
        order = np.argsort(-(share - base), kind="stable")
        base[order[:rem]] += 1
        counts += base
        over = np.maximum(counts - cap, 0)
        counts -= over
        free &= counts < cap
        remaining = int(over.sum())
    return counts


def moe_routing(counts, tokens=16384, seed=5):
    """Slots laid out expert after expert; slot i holds token perm[i % tokens]
    for a seeded permutation, so a token never meets the same expert twice as
    long as every count is <= tokens.  Returns (row_idx int32[total],
    group_off int32[E+1])."""
    counts = np.asarray(counts, np.int64)
    off = np.zeros(counts.size + 1, np.int64)
    off[1:] = np.cumsum(counts)
    perm = rng(seed).permutation(tokens)
    row_idx = perm[np.arange(off[-1]) % tokens]
    return row_idx.astype(np.int32), off.astype(np.int32)


def mxfp4_moe_act(tokens=16384, K=2880):
    return to_bf16_bits(gaussian(5, (tokens, K)))


def mxfp4_moe_weights(E=32, N=5760, K=2880, experts=None):
    """Expert weights, one independent seed per expert so a subset can be drawn."""
    ids = range(E) if experts is None else experts
    return [gaussian(5000 + e, (N, K), std=0.02) for e in ids]

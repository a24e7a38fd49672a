"""Seeded synthetic inputs for the ternary projection workloads.

This module only draws random numbers and stores them in the dtypes the
workloads use (int8 trits, binary16 scale bits, bfloat16 sign and activation
bits, int32 token ids).  It holds none of the projection's arithmetic (no
packing, no transform, no dequantisation): the oracle and the HIP path each
take these arrays and do their own work on them.

Workload shapes follow the 27B Ternary Bonsai model ([tensorsharp] §4.4:
hidden 5120, FFN 17408, vocabulary 248320; Hadamard block 1024 from
[ninfer-skill] §6).  Real weights are not available; these draws stand in for
them (value recipes below).
"""

import numpy as np

BF16_ONE = 0x3F80
BF16_MINUS_ONE = 0xBF80


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def trits_uniform(rng, n, k):
    """iid uniform over {-1, 0, +1}."""
    return rng.integers(-1, 2, size=(n, k), dtype=np.int8)


def trits_sparse(rng, n, k, p_zero=0.4, chunk_rows=4096):
    """P(0) = p_zero, P(-1) = P(+1) = (1 - p_zero) / 2."""
    out = np.empty((n, k), dtype=np.int8)
    p_neg = p_zero + (1.0 - p_zero) / 2.0
    for r0 in range(0, n, chunk_rows):
        u = rng.random((min(chunk_rows, n - r0), k), dtype=np.float32)
        t = np.zeros(u.shape, dtype=np.int8)
        t[(u >= p_zero) & (u < p_neg)] = -1
        t[u >= p_neg] = 1
        out[r0:r0 + u.shape[0]] = t
    return out


def scale_bits_uniform(rng, n, groups, lo, hi):
    """fp16 bits of U[lo, hi) draws (float64 rounded to nearest fp16)."""
    return rng.uniform(lo, hi, size=(n, groups)).astype(np.float16).view(np.uint16)


def scale_bits_lognormal(rng, n, groups, mu=-4.0, sigma=0.5):
    """fp16 bits of exp(N(mu, sigma)) draws."""
    return rng.lognormal(mu, sigma, size=(n, groups)).astype(np.float16).view(np.uint16)


def sign_bits(rng, k):
    """bf16 bits of an iid +-1 (p = 1/2) sign table of length k."""
    s = rng.integers(0, 2, size=k)
    return np.where(s == 1, BF16_ONE, BF16_MINUS_ONE).astype(np.uint16)


def activations_f32(rng, rows, k):
    return rng.standard_normal((rows, k), dtype=np.float32)


def activations_bf16_bits(rng, rows, k):
    return f32_to_bf16_bits(activations_f32(rng, rows, k))


def norm_weight_bits(rng, k):
    """bf16 bits of a norm weight near one: 1 + 0.1 * N(0, 1)."""
    return f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32))


def token_ids(rng, count, n):
    return rng.integers(0, n, size=count, dtype=np.int64).astype(np.int32)


def groups_of(k):
    return -(-k // 128)


# name -> description; seeds are the config numbers.
CONFIGS = {
    1: "tiny PQ2_0_G128 projection N=256 K=1024, fp32 activation",
    2: "FFN gate/up decode GEMV PQ2_0_G128 N=17408 K=5120, batch 1 bf16",
    3: "FFN down decode GEMV PTQ1_0_G128 N=5120 K=17408, batch 1/4/8 bf16",
    4: "output head PQ2_0_G128 N=248320 K=5120 batch 1 + 64-row embedding",
    5: "prefill GEMM 2048x5120 bf16 x PQ2_0_G128 N=17408",
}


def make_config(cfg, n=None, k=None, rows=None):
    """Draw one workload's inputs.  ``n``/``k``/``rows`` shrink the shape for
    fast tests while keeping the config's value recipe.

    Draw order is fixed: trits, scales, signs, activations, token ids.
    Returns a dict with keys fmt, n, k, trits, scale_bits, sign_bits, x
    (float32 array, or uint16 bf16 bits), x_dtype ('f32' or 'bf16') and, for
    config 4, ids.
    """
    rng = np.random.default_rng(cfg)
    if cfg == 1:
        fmt, n0, k0, r0 = "PQ2_0_G128", 256, 1024, 1
    elif cfg == 2:
        fmt, n0, k0, r0 = "PQ2_0_G128", 17408, 5120, 1
    elif cfg == 3:
        fmt, n0, k0, r0 = "PTQ1_0_G128", 5120, 17408, 8
    elif cfg == 4:
        fmt, n0, k0, r0 = "PQ2_0_G128", 248320, 5120, 1
    elif cfg == 5:
        fmt, n0, k0, r0 = "PQ2_0_G128", 17408, 5120, 2048
    else:
        raise ValueError("configs are 1..5")
    n = n0 if n is None else n
    k = k0 if k is None else k
    rows = r0 if rows is None else rows
    g = groups_of(k)
    if cfg in (1, 4):
        trits = trits_uniform(rng, n, k)
    else:
        trits = trits_sparse(rng, n, k)
    if cfg == 1:
        scales = scale_bits_uniform(rng, n, g, 0.005, 0.05)
    elif cfg == 4:
        scales = scale_bits_uniform(rng, n, g, 0.01, 0.04)
    else:
        scales = scale_bits_lognormal(rng, n, g)
    signs = sign_bits(rng, k)
    if cfg == 1:
        x, xdt = activations_f32(rng, rows, k), "f32"
    else:
        x, xdt = activations_bf16_bits(rng, rows, k), "bf16"
    out = dict(cfg=cfg, fmt=fmt, n=n, k=k, trits=trits, scale_bits=scales,
               sign_bits=signs, x=x, x_dtype=xdt)
    if cfg == 4:
        out["ids"] = token_ids(rng, 64, n)
    return out

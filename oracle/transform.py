"""Signed blockwise Walsh-Hadamard transform in float64 (oracle; test only).

[tensorsharp] §4.2: for a projection input x each block computes
H(D.x)/sqrt(block_size), with D the stored diagonal of +-1 signs and H the
unnormalised Hadamard matrix; embedding rows take the reverse order
D.(H.x)/sqrt(block_size).  The block size is 1024 ([ninfer-skill] §6
constants; [ninfer-v3] §8 ``hadamard_signs``: per 1024-element block,
multiply by the signs first, then apply the normalised Sylvester
Walsh-Hadamard transform).  "Sylvester" fixes the natural (not sequency)
ordering: H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]].

The transform is the dense matrix product, block by block, in float64.
"""

import numpy as np

BLOCK = 1024
INV_SQRT_BLOCK = 1.0 / 32.0  # 1/sqrt(1024), an exact power of two


def sylvester_hadamard(size):
    """Dense unnormalised Sylvester Hadamard matrix of order ``size``."""
    if size < 1 or size & (size - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < size:
        h = np.block([[h, h], [h, -h]])
    return h


_H_CACHE = {}


def hadamard_1024():
    if BLOCK not in _H_CACHE:
        _H_CACHE[BLOCK] = sylvester_hadamard(BLOCK)
    return _H_CACHE[BLOCK]


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_bits_to_f64(bits):
    """binary16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _check(x, d):
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    d = np.asarray(d, dtype=np.float64).reshape(-1)
    if x.shape[1] % BLOCK:
        raise ValueError("width must be a multiple of 1024")
    if d.shape[0] != x.shape[1]:
        raise ValueError("sign table must have one entry per column")
    return x, d


def forward(x, d):
    """Rows of x -> per block H(D.x)/32.  x: [rows, K]; d: [K] of +-1."""
    x, d = _check(x, d)
    h = hadamard_1024()
    out = np.empty_like(x)
    for b0 in range(0, x.shape[1], BLOCK):
        sl = slice(b0, b0 + BLOCK)
        dx = d[sl] * x[:, sl]               # D.x  (row-wise)
        out[:, sl] = (h @ dx.T).T * INV_SQRT_BLOCK   # H.(D.x) / 32
    return out


def inverse(x, d):
    """Rows of x -> per block D.(H.x)/32 (the inverse of :func:`forward`)."""
    x, d = _check(x, d)
    h = hadamard_1024()
    out = np.empty_like(x)
    for b0 in range(0, x.shape[1], BLOCK):
        sl = slice(b0, b0 + BLOCK)
        hx = (h @ x[:, sl].T).T             # H.x
        out[:, sl] = d[sl] * hx * INV_SQRT_BLOCK
    return out


def block_l1_over_32(x):
    """Per element, ||block of x containing it||_1 / 32 (the scale that the
    acceptance bound of a transform output uses: sum_j |H_ij d_j x_j| / 32)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    out = np.empty_like(x)
    for b0 in range(0, x.shape[1], BLOCK):
        sl = slice(b0, b0 + BLOCK)
        out[:, sl] = np.abs(x[:, sl]).sum(axis=1, keepdims=True) * INV_SQRT_BLOCK
    return out

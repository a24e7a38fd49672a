"""Lossless expansion of the ternary formats into 2-bit G64 blocks
(oracle; test infrastructure only).

[tensorsharp] §4.1: a loader that cannot run the private ternary types
expands their blocks, without requantising, into the upstream 2-bit block
type, and pays for it in memory (about 6% more for PQ2_0 and 29% more for
PTQ1_0, repeated in §8).  The target block follows [gguf-explainer] §4.3's
Q2_0 dequantisation: a binary16 multiplier ``d`` and packed codes, weight j of
a block at byte j/4, bits 2*(j%4), value (code - 1) * d; [ninfer-v3] §6.1
names the same codec q2_g64_fp16 (offset codes 0..3 for -1..2, groups of 64,
a binary16 multiplier).

Readings (the pages leave these open):
* a block holds 64 weights and is 18 bytes, [d (2 bytes, little-endian)]
  then [16 code bytes].  The explainer's listing sets its block size to 256
  (66 bytes, 2.0625 bits per weight), which would make the expansion smaller
  than PQ2_0's 2.125 bits, contradicting both quoted overheads; 64-weight
  blocks give 2.25 bits per weight, i.e. +5.9% over PQ2_0 and +28.6% over
  PTQ1_0, as quoted, and match the q2_g64_fp16 name.  The multiplier comes
  first as in the PQ2_0 GGUF block ([ninfer-skill] §4);
* the stream is row-major: row r holds blocks r*B .. r*B + B - 1 with
  B = k_pad / 64; block 2g and 2g + 1 of a row carry the two halves of the
  128-weight group g and both take that group's scale;
* weights past k up to k_pad are trit 0 (code 1), as in the planes;
* a stored value that is not a trit (a PQ2_0 code 3, which decodes to +2, or
  a PTQ1_0 byte beyond the digit range, decoded by the digit arithmetic) is
  carried over as its decoded value: the 2-bit code 3 also means +2, so the
  expansion keeps every decoded value, ternary or not.
"""

import numpy as np

from .codec import unpack_rowsplit
from .geometry import align_up

BLOCK_WEIGHTS = 64
BLOCK_BYTES = 18
GROUP = 128


def blocks_per_row(k):
    return align_up(k, GROUP) // BLOCK_WEIGHTS


def expanded_bytes(n, k):
    """Size of the expanded stream of an n x k matrix."""
    return n * blocks_per_row(k) * BLOCK_BYTES


def expand(fmt, n, k, payload):
    """Row-split planes of either ternary format -> the G64 block stream.

    The planes are decoded to trits and scales first ([ninfer-skill] §3 plane
    addressing, the format's code rule); every 128-weight group then becomes
    two blocks with the group's scale, so no value changes.
    """
    vals, scale_bits = unpack_rowsplit(fmt, n, k, payload)
    nb = blocks_per_row(k)
    codes = (vals.astype(np.int32) + 1).reshape(n, nb, 16, 4)
    qs = (codes[..., 0] | (codes[..., 1] << 2) | (codes[..., 2] << 4) | (codes[..., 3] << 6))
    d = np.repeat(scale_bits.astype(np.uint32), 2, axis=1)  # group g -> blocks 2g, 2g+1
    out = np.zeros((n, nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0] = d & 0xFF
    out[:, :, 1] = d >> 8
    out[:, :, 2:] = qs.astype(np.uint8)
    return out.reshape(-1)


def dequantize(stream, n, k):
    """G64 block stream -> float64 W[n, k_pad] by the block rule: value of
    weight j = (code_j - 1) * d with code_j = (qs[j // 4] >> 2*(j % 4)) & 3."""
    nb = blocks_per_row(k)
    blocks = np.asarray(stream, dtype=np.uint8)
    if blocks.size != n * nb * BLOCK_BYTES:
        raise ValueError("block stream stores %d bytes; layout requires %d"
                         % (blocks.size, n * nb * BLOCK_BYTES))
    blocks = blocks.reshape(n, nb, BLOCK_BYTES)
    d_bits = blocks[:, :, 0].astype(np.uint16) | (blocks[:, :, 1].astype(np.uint16) << 8)
    d = d_bits.view(np.float16).astype(np.float64)
    qs = blocks[:, :, 2:].astype(np.int32)
    codes = np.stack([(qs >> (2 * i)) & 3 for i in range(4)], axis=-1)  # [n, nb, 16, 4]
    vals = codes.reshape(n, nb, BLOCK_WEIGHTS) - 1
    return (vals * d[:, :, None]).reshape(n, nb * BLOCK_WEIGHTS)


def project(stream, n, k, xrot):
    """y[b, r] = sum_j W[r, j] * x'[b, j] over the expanded stream, float64.
    xrot: [batch, k_pad] (or [batch, k], zero-extended)."""
    w = dequantize(stream, n, k)
    xr = np.zeros((xrot.shape[0], w.shape[1]), dtype=np.float64)
    xr[:, :xrot.shape[1]] = xrot
    return xr @ w.T

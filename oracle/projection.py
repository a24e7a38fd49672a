"""Dequantisation, projection and embedding rows in float64 (oracle; test only).

The weight of row n, column 128g+j is trit * scale[n, g] ([gguf-explainer]
§4.3: value = (code - 1) * d with one fp16 scale per group; [ninfer-skill]
§2/§3: one binary16 scale per 128-weight group).  A projection multiplies the
stored matrix by the transformed input ([ninfer-v3] §8: the use multiplies
the stored matrix by hadamard_transform(input, signs) instead of the raw
input; [tensorsharp] §4.4: every low-bit projection rotates its input, the
head takes the forward transform after the final norm, the embedding row
takes the inverse transform).

Everything is the plain definition: y[b, n] = sum_j W[n, j] * x'[b, j].
"""

import numpy as np

from . import codec, transform
from .geometry import row_split_geometry

# Acceptance: |gpu - oracle| <= REL * sum_j |w_nj * x'_j| + ABS per output.
REL = 1e-3
ABS = 1e-5


def dequantize(fmt, n, k, payload, rows=None):
    """Payload -> dense float64 W[rows, k_pad] (all rows when rows is None)."""
    vals, scale_bits = codec.unpack_rowsplit(fmt, n, k, payload)
    if rows is not None:
        vals = vals[rows]
        scale_bits = scale_bits[rows]
    scale = transform.fp16_bits_to_f64(scale_bits)            # [r, G]
    w = vals.astype(np.float64).reshape(vals.shape[0], -1, codec.GROUP)
    w = w * scale[:, :, None]
    return w.reshape(vals.shape[0], -1)


def dequantize_trits(trits, scale_bits):
    """Generated trits [n, k] and scale bits [n, G] -> W[n, k] in float64."""
    trits = np.asarray(trits)
    n, k = trits.shape
    scale = transform.fp16_bits_to_f64(scale_bits)
    col_group = np.arange(k) // codec.GROUP
    return trits.astype(np.float64) * scale[:, col_group]


def project(w, xrot):
    """y[b, n] = sum_j W[n, j] x'[b, j]; W: [N, K'], x': [B, K] with K <= K'."""
    xrot = np.atleast_2d(np.asarray(xrot, dtype=np.float64))
    w = w[:, :xrot.shape[1]]
    return xrot @ w.T


def bound(w, xrot):
    """Per-output acceptance bound REL * sum_j |W[n,j] x'[b,j]| + ABS."""
    xrot = np.atleast_2d(np.asarray(xrot, dtype=np.float64))
    w = w[:, :xrot.shape[1]]
    return REL * (np.abs(xrot) @ np.abs(w).T) + ABS


def project_payload(fmt, n, k, payload, xrot, rows=None, chunk=4096):
    """Projection straight from the payload, chunked over rows so that large
    matrices never hold a dense float64 copy.  Returns (y, bound) with shape
    [B, len(rows)]."""
    xrot = np.atleast_2d(np.asarray(xrot, dtype=np.float64))
    rows = np.arange(n) if rows is None else np.asarray(rows)
    ys, bs = [], []
    for c0 in range(0, rows.size, chunk):
        r = rows[c0:c0 + chunk]
        w = dequantize(fmt, n, k, payload, rows=r)
        ys.append(project(w, xrot))
        bs.append(bound(w, xrot))
    if not ys:
        empty = np.zeros((xrot.shape[0], 0))
        return empty, empty
    return np.concatenate(ys, axis=1), np.concatenate(bs, axis=1)


def project_scalar(fmt, n, k, payload, xrot):
    """Unpack-and-dot with plain loops, for tiny shapes only.

    For each output row, walk the groups, decode the group's bytes with the
    scalar group decoder, take the scale's binary16 bits from the scale plane,
    and accumulate trit * scale * x' in float64.
    """
    geo = row_split_geometry(fmt, n, k)
    data = bytes(np.asarray(payload, dtype=np.uint8))
    xrot = np.atleast_2d(np.asarray(xrot, dtype=np.float64))
    groups = geo["groups_per_row"]
    bpg, hpg = geo["base_bytes_per_group"], geo["high_bytes_per_group"]
    out = np.zeros((xrot.shape[0], n))
    for row in range(n):
        for g in range(groups):
            b = geo["base_offset"] + row * geo["base_row_bytes"] + g * bpg
            base = data[b:b + bpg]
            if fmt == "PQ2_0_G128":
                vals = codec.pq2_decode_group(base)
            else:
                h = geo["high_offset"] + row * geo["high_row_bytes"] + g * hpg
                vals = codec.ptq1_decode_group(base, data[h:h + hpg])
            s = geo["scale_offset"] + row * geo["scale_row_bytes"] + 2 * g
            sbits = data[s] | (data[s + 1] << 8)
            scale = float(np.array([sbits], dtype=np.uint16).view(np.float16)[0])
            for bi in range(xrot.shape[0]):
                acc = 0.0
                for j in range(codec.GROUP):
                    col = g * codec.GROUP + j
                    if col < xrot.shape[1]:
                        acc += vals[j] * float(xrot[bi, col])
                out[bi, row] += scale * acc
    return out


def projection(fmt, n, k, payload, x, signs):
    """End to end: y = W . H(D.x)/32 (x: [B, K] float64, signs: [K])."""
    xrot = transform.forward(x, signs)
    return project_payload(fmt, n, k, payload, xrot)


def embed_rows_inverse(fmt, n, k, payload, ids, signs):
    """Embedding rows: out[i] = D.(H.W[ids[i]])/32 blockwise, float64.

    Also returns the acceptance scale per element (block L1 norm of the
    dequantised row over 32)."""
    ids = np.asarray(ids).reshape(-1)
    if ids.size and (ids.min() < 0 or ids.max() >= n):
        raise IndexError("token id out of range")
    w = dequantize(fmt, n, k, payload, rows=ids)[:, :k]
    return transform.inverse(w, signs), transform.block_l1_over_32(w)

"""Ternary group codecs and row-split plane packing (oracle; test only).

PQ2_0_G128 code semantics: [gguf-explainer] §4.3 -- weight j of a group sits
in byte j/4 at bit offset 2*(j%4) (least significant pair first) and its value
is (code - 1) times the group scale, i.e. codes 0,1,2,3 mean -1,0,+1,+2.  The
byte-permute table of §4.4 (bytes FF,00,01,02 = -1,0,1,2 indexed by the code)
states the same mapping.  Plane bytes are the GGUF block bytes copied verbatim
([ninfer-skill] §4 block <-> plane slices), so the 32 base bytes of a group
are exactly those ``qs`` bytes.

PTQ1_0_G128 trit packing: the pages give only the byte budget (24 base bytes,
2 high bytes per 128-weight group, [ninfer-skill] §2/§3), not the bit order.
This project's convention (parity of it is pinned to the convention itself,
not to the pages): digit u = trit + 1 in {0,1,2};
  base byte b (0 <= b < 24) = sum_{i<5} u[5b+i] * 3**i   (trits 0..119)
  high byte h (0 <= h < 2)  = sum_{i<4} u[120+4h+i] * 3**i (trits 120..127)
and decoding takes digit i of byte v as (v // 3**i) % 3.

Plane addressing: each plane is row-major over (row, group); the base bytes
of (row n, group g) start at base_offset + n*base_row_bytes + g*base_bytes,
high bytes at high_offset + n*high_row_bytes + g*high_bytes, and the scale is
a little-endian binary16 at scale_offset + n*scale_row_bytes + 2*g
([ninfer-skill] §3 per-row byte counts and the per-format scale-start table).
Padding bytes between planes are zero; trits past k up to k_pad are 0.
"""

import numpy as np

from .geometry import FORMATS, row_split_geometry

GROUP = 128

# [gguf-explainer] §4.3: value of each 2-bit code (00=-1, 01=0, 10=+1, 11=+2).
PQ2_CODE_VALUE = (-1, 0, 1, 2)


# ---------------------------------------------------------------- scalar ---
def pq2_encode_group(trits):
    """128 trits in {-1,0,1} -> 32 bytes (code = trit + 1, LSB pair first)."""
    assert len(trits) == GROUP
    out = bytearray(32)
    for j, t in enumerate(trits):
        t = int(t)
        if t not in (-1, 0, 1):
            raise ValueError("trit out of range: %d" % t)
        out[j // 4] |= (t + 1) << (2 * (j % 4))
    return bytes(out)


def pq2_decode_group(base):
    """32 bytes -> 128 values in {-1,0,1,2} ([gguf-explainer] §4.3 rule)."""
    assert len(base) == 32
    vals = []
    for j in range(GROUP):
        code = (base[j // 4] >> (2 * (j % 4))) & 0x03
        vals.append(PQ2_CODE_VALUE[code])
    return vals


def ptq1_encode_group(trits):
    """128 trits -> (24 base bytes, 2 high bytes) by the radix-3 convention."""
    assert len(trits) == GROUP
    u = []
    for t in trits:
        t = int(t)
        if t not in (-1, 0, 1):
            raise ValueError("trit out of range: %d" % t)
        u.append(t + 1)
    base = bytearray(24)
    for b in range(24):
        v = 0
        for i in range(5):
            v += u[5 * b + i] * 3 ** i
        base[b] = v
    high = bytearray(2)
    for h in range(2):
        v = 0
        for i in range(4):
            v += u[120 + 4 * h + i] * 3 ** i
        high[h] = v
    return bytes(base), bytes(high)


def ptq1_decode_group(base, high):
    """(24 base bytes, 2 high bytes) -> 128 trits (digit i = v//3**i % 3, -1)."""
    assert len(base) == 24 and len(high) == 2
    vals = []
    for b in range(24):
        for i in range(5):
            vals.append((base[b] // 3 ** i) % 3 - 1)
    for h in range(2):
        for i in range(4):
            vals.append((high[h] // 3 ** i) % 3 - 1)
    return vals


# ------------------------------------------------------------ vectorised ---
def _pad_trits(trits, k_pad):
    n, k = trits.shape
    if k == k_pad:
        return np.ascontiguousarray(trits, dtype=np.int8)
    out = np.zeros((n, k_pad), dtype=np.int8)
    out[:, :k] = trits
    return out


def pack_rowsplit(fmt, trits, scale_bits):
    """Encode an [n, k] trit matrix and [n, G] fp16 scale bits into planes.

    Returns the payload as a uint8 array of exactly ``payload_bytes`` bytes.
    """
    trits = np.asarray(trits)
    n, k = trits.shape
    geo = row_split_geometry(fmt, n, k)
    groups = geo["groups_per_row"]
    scale_bits = np.asarray(scale_bits, dtype=np.uint16)
    if scale_bits.shape != (n, groups):
        raise ValueError("scale_bits must have shape (n, groups_per_row)")
    if trits.size and (trits.min() < -1 or trits.max() > 1):
        raise ValueError("trits must lie in {-1, 0, 1}")
    u = _pad_trits(trits, geo["k_pad"]).astype(np.int32) + 1
    u = u.reshape(n, groups, GROUP)
    payload = np.zeros(geo["payload_bytes"], dtype=np.uint8)
    if fmt == "PQ2_0_G128":
        q = u.reshape(n, groups, 32, 4)
        base = q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)
        high = None
    else:
        w5 = np.array([1, 3, 9, 27, 81], dtype=np.int32)
        w4 = np.array([1, 3, 9, 27], dtype=np.int32)
        base = (u[:, :, :120].reshape(n, groups, 24, 5) * w5).sum(axis=-1)
        high = (u[:, :, 120:].reshape(n, groups, 2, 4) * w4).sum(axis=-1)
    b0 = geo["base_offset"]
    payload[b0:b0 + geo["base_bytes"]] = base.astype(np.uint8).reshape(-1)
    if high is not None:
        h0 = geo["high_offset"]
        payload[h0:h0 + geo["high_bytes"]] = high.astype(np.uint8).reshape(-1)
    s0 = geo["scale_offset"]
    # little-endian binary16: low byte first
    sb = scale_bits.astype(np.uint32)
    scale_le = np.stack([sb & 0xFF, sb >> 8], axis=-1).astype(np.uint8)
    payload[s0:s0 + geo["scale_bytes"]] = scale_le.reshape(-1)
    return payload


def plane_arrays(fmt, n, k, payload):
    """Return (base [n,G,bpg], high [n,G,hpg] or None, scale_bits [n,G])."""
    geo = row_split_geometry(fmt, n, k)
    payload = np.asarray(payload, dtype=np.uint8)
    if payload.size != geo["payload_bytes"]:
        raise ValueError("payload stores %d bytes; layout requires %d"
                         % (payload.size, geo["payload_bytes"]))
    groups = geo["groups_per_row"]
    bpg = geo["base_bytes_per_group"]
    hpg = geo["high_bytes_per_group"]
    b0, h0, s0 = geo["base_offset"], geo["high_offset"], geo["scale_offset"]
    base = payload[b0:b0 + geo["base_bytes"]].reshape(n, groups, bpg)
    high = None
    if hpg:
        high = payload[h0:h0 + geo["high_bytes"]].reshape(n, groups, hpg)
    s = payload[s0:s0 + geo["scale_bytes"]].reshape(n, groups, 2)
    scale_bits = s[..., 0].astype(np.uint16) | (s[..., 1].astype(np.uint16) << 8)
    return base, high, scale_bits


def unpack_rowsplit(fmt, n, k, payload):
    """Decode planes -> (values [n, k_pad] int8 in {-1,0,1,2}, scale_bits).

    A PQ2_0 code 3 decodes to +2 and a PTQ1_0 byte above 242 (base) or 80
    (high) decodes by the digit arithmetic; neither is a ternary value, and
    callers that need strict ternary data check the result.
    """
    base, high, scale_bits = plane_arrays(fmt, n, k, payload)
    groups = base.shape[1]
    if fmt == "PQ2_0_G128":
        b = base.astype(np.int16)
        codes = np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=-1)
        vals = codes.reshape(n, groups * GROUP) - 1
    else:
        b = base.astype(np.int32)
        h = high.astype(np.int32)
        dig_b = np.stack([(b // 3 ** i) % 3 for i in range(5)], axis=-1)
        dig_h = np.stack([(h // 3 ** i) % 3 for i in range(4)], axis=-1)
        vals = np.concatenate([dig_b.reshape(n, groups, 120),
                               dig_h.reshape(n, groups, 8)], axis=-1)
        vals = vals.reshape(n, groups * GROUP) - 1
    return vals.astype(np.int8), scale_bits


# ------------------------------------------------- block <-> plane slices ---
# [ninfer-skill] §4: per format, the (start, stop) byte ranges of one GGUF
# block that go to the base, high and scale planes (None: no such plane).
BLOCK_BYTES = {"PTQ1_0_G128": 28, "PQ2_0_G128": 34}
BLOCK_PLANE_SLICES = {
    "PTQ1_0_G128": ((0, 24), (24, 26), (26, 28)),
    "PQ2_0_G128": ((2, 34), (None, None), (0, 2)),
}


def planes_to_blocks(fmt, n, k, payload):
    """Row-split planes -> the contiguous GGUF block stream (row by row)."""
    base, high, scale_bits = plane_arrays(fmt, n, k, payload)
    groups = base.shape[1]
    blocks = np.zeros((n, groups, BLOCK_BYTES[fmt]), dtype=np.uint8)
    (b_lo, b_hi), (h_lo, h_hi), (s_lo, s_hi) = BLOCK_PLANE_SLICES[fmt]
    blocks[:, :, b_lo:b_hi] = base
    if h_lo is not None:
        blocks[:, :, h_lo:h_hi] = high
    blocks[:, :, s_lo] = (scale_bits & 0xFF).astype(np.uint8)
    blocks[:, :, s_lo + 1] = (scale_bits >> 8).astype(np.uint8)
    return blocks.reshape(-1)


def blocks_to_planes(fmt, n, k, blocks):
    """GGUF block stream -> row-split payload (the exact inverse)."""
    geo = row_split_geometry(fmt, n, k)
    groups = geo["groups_per_row"]
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(n, groups, BLOCK_BYTES[fmt])
    (b_lo, b_hi), (h_lo, h_hi), (s_lo, s_hi) = BLOCK_PLANE_SLICES[fmt]
    payload = np.zeros(geo["payload_bytes"], dtype=np.uint8)
    b0, h0, s0 = geo["base_offset"], geo["high_offset"], geo["scale_offset"]
    payload[b0:b0 + geo["base_bytes"]] = blocks[:, :, b_lo:b_hi].reshape(-1)
    if h_lo is not None:
        payload[h0:h0 + geo["high_bytes"]] = blocks[:, :, h_lo:h_hi].reshape(-1)
    payload[s0:s0 + geo["scale_bytes"]] = blocks[:, :, s_lo:s_hi].reshape(-1)
    return payload

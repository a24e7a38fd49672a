"""Row-split plane geometry (oracle; test infrastructure only).

Follows [ninfer-skill] §2 (the two ternary formats as
(group_size, base_bytes, high_bytes)) and §3 (the row-split geometry
derivation and the order of the 16 fields of the record), with align_up as
defined in [ninfer-v3] (round up to a multiple).
"""

from collections import OrderedDict

# [ninfer-skill] §2: TernaryFormat(name, group_size, base_bytes, high_bytes).
FORMATS = {
    "PQ2_0_G128": (128, 32, 0),
    "PTQ1_0_G128": (128, 24, 2),
}

# [ninfer-skill] §6 constants table: GGUF tensor type ids.
GGUF_TYPE = {"PQ2_0_G128": 142, "PTQ1_0_G128": 143}

# [ninfer-skill] §1 alignment constants.
PLANE_ALIGNMENT = 256
K_ALIGNMENT = 128
SCALE_BYTES = 2  # one binary16 per group ([ninfer-skill] §3)

# [ninfer-skill] §3: field order of RowSplitGeometry.
FIELDS = (
    "n", "k", "k_pad", "groups_per_row", "base_bytes_per_group",
    "high_bytes_per_group", "base_row_bytes", "high_row_bytes",
    "scale_row_bytes", "base_offset", "base_bytes", "high_offset",
    "high_bytes", "scale_offset", "scale_bytes", "payload_bytes",
)


def align_up(value, alignment):
    """Smallest multiple of ``alignment`` that is >= ``value``."""
    return -(-value // alignment) * alignment


def row_split_geometry(fmt, n, k):
    """Return the 16-field geometry of an [n, k] ternary matrix.

    [ninfer-skill] §3: the shape must be rank 2 with positive dimensions;
    k_pad = align_up(k, 128); groups = k_pad / 128; per-row bytes of each
    plane are groups times the per-group bytes (2 for the scale); the base
    plane starts at 0, the high plane at align_up(base_bytes, 256) (kept even
    when it is empty), the scale plane at high_offset +
    align_up(high_bytes, 256), and the payload ends after the scale plane.
    """
    if fmt not in FORMATS:
        raise ValueError("unknown numeric format: %r" % (fmt,))
    if not (isinstance(n, int) and isinstance(k, int)) or n <= 0 or k <= 0:
        raise ValueError("shape must be rank 2 with positive dimensions")
    group, base_pg, high_pg = FORMATS[fmt]
    k_pad = align_up(k, K_ALIGNMENT)
    groups = k_pad // group
    base_row = groups * base_pg
    high_row = groups * high_pg
    scale_row = groups * SCALE_BYTES
    base_offset = 0
    base_bytes = n * base_row
    high_offset = align_up(base_bytes, PLANE_ALIGNMENT)
    high_bytes = n * high_row
    scale_offset = high_offset + align_up(high_bytes, PLANE_ALIGNMENT)
    scale_bytes = n * scale_row
    payload = scale_offset + scale_bytes
    values = (n, k, k_pad, groups, base_pg, high_pg, base_row, high_row,
              scale_row, base_offset, base_bytes, high_offset, high_bytes,
              scale_offset, scale_bytes, payload)
    return OrderedDict(zip(FIELDS, values))

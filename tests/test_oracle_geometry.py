"""Oracle geometry pinned to the sizes the pages print and to closed forms."""

import pytest

from oracle.geometry import FIELDS, FORMATS, GGUF_TYPE, row_split_geometry
from oracle.codec import BLOCK_BYTES, BLOCK_PLANE_SLICES
from conftest import load_golden

G = load_golden("geometry_pages.json")


@pytest.mark.parametrize("case", G["payload_bytes"])
def test_printed_vocab_payload(case):
    geo = row_split_geometry(case["fmt"], case["n"], case["k"])
    assert geo["payload_bytes"] == case["payload_bytes"]


def test_printed_per_row_bytes():
    # [ninfer-skill] §3: value_z (12288, 5120) and query_key (7168, 5120)
    # store n*1360 bytes in PQ2_0 (base 1280 + scales 80 per row).
    per_row = G["per_row_bytes_k5120"]["PQ2_0_G128"]
    for n in G["example_rows"].values():
        geo = row_split_geometry("PQ2_0_G128", n, 5120)
        assert geo["payload_bytes"] == n * per_row
    # PTQ1_0: the page prints 1088, which contradicts its own vocabulary
    # total; the reading is 1120 = 278118400 / 248320 = 40 * 28.
    assert 278118400 // 248320 == 1120 != G["per_row_bytes_k5120"]["PTQ1_0_G128_as_printed"]
    for n in G["example_rows"].values():
        geo = row_split_geometry("PTQ1_0_G128", n, 5120)
        assert geo["payload_bytes"] == n * 1120


@pytest.mark.parametrize("k,groups", [(5120, 40), (6144, 48), (17408, 136), (1024, 8)])
def test_groups_per_row(k, groups):
    for fmt in FORMATS:
        assert row_split_geometry(fmt, 7, k)["groups_per_row"] == groups
    if str(k) in G["groups_per_row"]:
        assert G["groups_per_row"][str(k)] == groups


def test_pq2_empty_high_plane():
    # [ninfer-skill] §3: the high offset is computed even when high_bytes is
    # 0, so PQ2_0 keeps an empty high plane and scale_offset == high_offset.
    for n, k in [(1, 128), (3, 1000), (17408, 5120), (248320, 5120)]:
        geo = row_split_geometry("PQ2_0_G128", n, k)
        assert geo["high_bytes"] == 0 and geo["high_row_bytes"] == 0
        assert geo["scale_offset"] == geo["high_offset"]


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_scale_start_table(fmt):
    # [ninfer-skill] §3 table: the scale plane starts at rows*groups*32
    # (PQ2_0) or rows*groups*26 (PTQ1_0) -- whenever the planes before it are
    # whole multiples of 256 bytes, as for every model width.
    per_group = G["scale_start_bytes_per_group"][fmt]
    for n, k in [(248320, 5120), (12288, 5120), (6144, 6144), (5120, 17408)]:
        geo = row_split_geometry(fmt, n, k)
        assert geo["scale_offset"] == n * geo["groups_per_row"] * per_group


def test_block_sizes_and_slices():
    # [ninfer-skill] §4: GGML_BLOCK and BLOCK_PLANE_SLICES agree with the
    # per-group plane bytes of §2/§3 (base + high + 2-byte scale).
    for fmt, (group, base, high) in FORMATS.items():
        assert group == 128
        assert base + high + 2 == BLOCK_BYTES[fmt] == G["block_bytes"][fmt]
        (b0, b1), (h0, h1), (s0, s1) = BLOCK_PLANE_SLICES[fmt]
        assert b1 - b0 == base and s1 - s0 == 2
        assert (h1 - h0 if h0 is not None else 0) == high
    assert GGUF_TYPE == G["gguf_type"]


def test_field_order_and_workload_sizes():
    assert len(FIELDS) == 16 and FIELDS[0] == "n" and FIELDS[-1] == "payload_bytes"
    # Worked by hand:
    # 256 x 1024 PQ2_0: 8 groups; base 256*256 = 65536; scales 256*16 = 4096.
    assert row_split_geometry("PQ2_0_G128", 256, 1024)["payload_bytes"] == 69632
    # 17408 x 5120 PQ2_0: base 17408*1280 = 22282240; scales 17408*80.
    assert row_split_geometry("PQ2_0_G128", 17408, 5120)["payload_bytes"] == 23674880
    # 5120 x 17408 PTQ1_0: 136 groups; base 5120*3264 = 16711680;
    # high 5120*272 = 1392640 at 16711680; scales at 18104320.
    geo = row_split_geometry("PTQ1_0_G128", 5120, 17408)
    assert (geo["base_bytes"], geo["high_offset"], geo["high_bytes"],
            geo["scale_offset"], geo["payload_bytes"]) == (
        16711680, 16711680, 1392640, 18104320, 19496960)


def test_ragged_k_and_alignment():
    # k = 1000 pads to 1024; 3 rows of PTQ1_0: base 3*8*24 = 576 -> high at
    # 768; high 3*16 = 48 -> scales at 768 + 256 = 1024; payload 1024 + 48.
    geo = row_split_geometry("PTQ1_0_G128", 3, 1000)
    assert geo["k_pad"] == 1024 and geo["groups_per_row"] == 8
    assert geo["high_offset"] == 768 and geo["scale_offset"] == 1024
    assert geo["payload_bytes"] == 1072
    for fmt in FORMATS:
        for n, k in [(1, 1), (5, 129), (33, 4000)]:
            geo = row_split_geometry(fmt, n, k)
            assert geo["high_offset"] % 256 == 0 and geo["scale_offset"] % 256 == 0


@pytest.mark.parametrize("bad", [("Q4_0", 4, 128), ("PQ2_0_G128", 0, 128),
                                 ("PQ2_0_G128", 4, 0), ("PTQ1_0_G128", -1, 128)])
def test_rejects_bad_arguments(bad):
    with pytest.raises(ValueError):
        row_split_geometry(*bad)

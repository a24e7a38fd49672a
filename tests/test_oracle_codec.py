"""Oracle codecs pinned to the pages' code rule, brute force and invariants."""

import itertools

import numpy as np
import pytest

from oracle import codec
from oracle.geometry import row_split_geometry
from conftest import load_golden
import synth

PQ = load_golden("pq2_codes.json")
PT = load_golden("ptq1_convention.json")


def test_pq2_lut_from_page():
    # [gguf-explainer] §4.4: the bytes of 0x020100FF, indexed by the code,
    # are the restored values -1, 0, 1, 2 (little-endian byte order).
    word = int(PQ["lut_dword"], 16)
    lut = [int(np.array([(word >> (8 * c)) & 0xFF], dtype=np.uint8).view(np.int8)[0])
           for c in range(4)]
    assert lut == PQ["lut_values_by_code"] == list(codec.PQ2_CODE_VALUE)


@pytest.mark.parametrize("case", PQ["bytes"])
def test_pq2_worked_bytes(case):
    b = int(case["byte"], 16)
    vals = codec.pq2_decode_group(bytes([b]) * 32)
    assert vals[:4] == case["values"] and vals[4:8] == case["values"]


def test_pq2_all_bytes_brute_force():
    # Every byte value decodes to 4 codes; those without code 3 re-encode to
    # the same byte; code 3 decodes to +2 and cannot be encoded.
    n_ternary = 0
    for b in range(256):
        vals = codec.pq2_decode_group(bytes([b]) * 32)[:4]
        codes = [(b >> (2 * i)) & 3 for i in range(4)]
        assert vals == [c - 1 for c in codes]
        if 3 in codes:
            assert 2 in vals
            with pytest.raises(ValueError):
                codec.pq2_encode_group(vals * 32)
        else:
            n_ternary += 1
            assert codec.pq2_encode_group(vals * 32) == bytes([b]) * 32
    assert n_ternary == 81


@pytest.mark.parametrize("case", PT["base"])
def test_ptq1_worked_base_bytes(case):
    trits = case["trits"] * 24 + [0] * 8
    base, high = codec.ptq1_encode_group(trits)
    assert base == bytes([case["byte"]]) * 24 and high == bytes([40, 40])


@pytest.mark.parametrize("case", PT["high"])
def test_ptq1_worked_high_bytes(case):
    trits = [0] * 120 + case["trits"] * 2
    base, high = codec.ptq1_encode_group(trits)
    assert high == bytes([case["byte"]]) * 2 and base == bytes([121]) * 24


def test_ptq1_bijections_brute_force():
    # 3^5 = 243 five-trit tuples <-> base bytes 0..242, and 3^4 = 81 four-trit
    # tuples <-> high bytes 0..80, one to one.
    seen = {}
    for tup in itertools.product((-1, 0, 1), repeat=5):
        base, _ = codec.ptq1_encode_group(list(tup) * 24 + [0] * 8)
        assert base[0] not in seen
        seen[base[0]] = tup
        assert tuple(codec.ptq1_decode_group(base, bytes([40, 40]))[:5]) == tup
    assert sorted(seen) == list(range(243))
    seen_h = set()
    for tup in itertools.product((-1, 0, 1), repeat=4):
        _, high = codec.ptq1_encode_group([0] * 120 + list(tup) * 2)
        seen_h.add(high[0])
        assert tuple(codec.ptq1_decode_group(bytes([121]) * 24, high)[120:124]) == tup
    assert sorted(seen_h) == list(range(81))


def test_ptq1_division_identity():
    # floor(v/3) == (v*171) >> 9 for every byte value: the exact
    # multiply-shift a decoder may use in place of a division.
    for v in range(256):
        assert v // 3 == (v * 171) >> 9


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("n,k", [(1, 128), (5, 1024), (7, 1000), (3, 2176)])
def test_pack_matches_scalar_groups_and_roundtrips(fmt, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    trits = synth.trits_uniform(rng, n, k)
    g = synth.groups_of(k)
    sb = synth.scale_bits_uniform(rng, n, g, 0.01, 0.04)
    payload = codec.pack_rowsplit(fmt, trits, sb)
    geo = row_split_geometry(fmt, n, k)
    assert payload.size == geo["payload_bytes"]
    pad = np.zeros((n, geo["k_pad"]), dtype=np.int8)
    pad[:, :k] = trits
    data = payload.tobytes()
    for r in range(n):
        for gi in range(g):
            grp = list(pad[r, 128 * gi:128 * gi + 128])
            b = geo["base_offset"] + r * geo["base_row_bytes"] + gi * geo["base_bytes_per_group"]
            s = geo["scale_offset"] + r * geo["scale_row_bytes"] + 2 * gi
            if fmt == "PQ2_0_G128":
                assert data[b:b + 32] == codec.pq2_encode_group(grp)
            else:
                h = geo["high_offset"] + r * geo["high_row_bytes"] + 2 * gi
                assert (data[b:b + 24], data[h:h + 2]) == codec.ptq1_encode_group(grp)
            assert data[s] | (data[s + 1] << 8) == sb[r, gi]
    vals, sb2 = codec.unpack_rowsplit(fmt, n, k, payload)
    assert np.array_equal(vals, pad) and np.array_equal(sb2, sb)
    # Padding between planes is zero.
    gaps = [(geo["base_bytes"], geo["high_offset"]),
            (geo["high_offset"] + geo["high_bytes"], geo["scale_offset"])]
    for lo, hi in gaps:
        assert not payload[lo:hi].any()


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("k", [5120, 6144, 17408])
def test_block_plane_exact_inverse(fmt, k):
    # [ninfer-skill] §4: the slices reproduce block_to_planes, their lengths
    # sum to the block size and planes_to_block is the exact inverse.
    n = 3
    rng = np.random.default_rng(k)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = codec.pack_rowsplit(fmt, trits, sb)
    blocks = codec.planes_to_blocks(fmt, n, k, payload)
    assert blocks.size == n * (k // 128) * codec.BLOCK_BYTES[fmt]
    assert np.array_equal(codec.blocks_to_planes(fmt, n, k, blocks), payload)
    # PQ2_0 blocks carry the scale first, PTQ1_0 blocks last ([ninfer-skill] §3).
    blk = blocks.reshape(n, -1, codec.BLOCK_BYTES[fmt])
    s_lo = 0 if fmt == "PQ2_0_G128" else 26
    bits = blk[:, :, s_lo].astype(np.uint16) | (blk[:, :, s_lo + 1].astype(np.uint16) << 8)
    assert np.array_equal(bits, sb)


def test_wrong_scale_offset_trap():
    # [ninfer-skill] §3: reading PTQ1_0 scales at rows*groups*base_bytes
    # (inside the high plane) gives plausible-looking but wrong numbers; the
    # geometry's scale_offset gives the stored scales back exactly.
    n, k = 64, 5120
    rng = np.random.default_rng(7)
    trits = synth.trits_sparse(rng, n, k)
    g = synth.groups_of(k)
    sb = synth.scale_bits_lognormal(rng, n, g)
    payload = codec.pack_rowsplit("PTQ1_0_G128", trits, sb)
    geo = row_split_geometry("PTQ1_0_G128", n, k)
    right = payload[geo["scale_offset"]:geo["scale_offset"] + 2 * n * g].view(np.uint16)
    assert np.array_equal(right.reshape(n, g), sb)
    wrong_at = n * g * 24
    wrong = payload[wrong_at:wrong_at + 2 * n * g].view(np.uint16)
    assert not np.array_equal(wrong.reshape(n, g), sb)
    med = float(np.median(right.view(np.float16).astype(np.float64)))
    assert 0.01 < med < 0.03    # healthy scale statistics (median near e^-4)


def test_pack_rejects_bad_input():
    with pytest.raises(ValueError):
        codec.pack_rowsplit("PQ2_0_G128", np.full((2, 128), 2, np.int8),
                            np.zeros((2, 1), np.uint16))
    with pytest.raises(ValueError):
        codec.pack_rowsplit("PQ2_0_G128", np.zeros((2, 128), np.int8),
                            np.zeros((2, 2), np.uint16))
    with pytest.raises(ValueError):
        codec.plane_arrays("PQ2_0_G128", 2, 128, np.zeros(10, np.uint8))

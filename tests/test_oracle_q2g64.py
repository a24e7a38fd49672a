"""G64 expansion oracle pinned to the pages' overheads, the code table,
hand-computed blocks and exact equality of the dequantised values."""

import numpy as np
import pytest

from oracle import codec, q2g64, projection as P
from oracle.geometry import row_split_geometry
from conftest import load_golden
import synth

FMTS = ["PQ2_0_G128", "PTQ1_0_G128"]
GOLD = load_golden("q2g64_blocks.json")
CODES = load_golden("pq2_codes.json")


@pytest.mark.parametrize("fmt,n,k,percent", [
    # [tensorsharp] §4.1 and §8: the expansion needs about 6% more memory
    # for PQ2_0 and about 29% more for PTQ1_0.
    ("PQ2_0_G128", 17408, 5120, 6),
    ("PQ2_0_G128", 248320, 5120, 6),
    ("PTQ1_0_G128", 5120, 17408, 29),
    ("PTQ1_0_G128", 248320, 5120, 29),
])
def test_overhead_matches_pages(fmt, n, k, percent):
    payload = row_split_geometry(fmt, n, k)["payload_bytes"]
    assert round(100 * (q2g64.expanded_bytes(n, k) / payload - 1)) == percent


def test_bits_per_weight():
    # 2 bits per code plus a 16-bit multiplier per 64 weights
    assert q2g64.BLOCK_BYTES * 8 / q2g64.BLOCK_WEIGHTS == 2.25
    assert q2g64.expanded_bytes(3, 1000) == 3 * 16 * 18  # k_pad = 1024


def _golden_trits():
    n, k = GOLD["n"], GOLD["k"]
    trits = np.zeros((n, k), np.int8)
    for j, t in GOLD["nonzero_trits_row0"].items():
        trits[0, int(j)] = t
    trits[1, :] = GOLD["row1_trit"]
    sb = np.array(GOLD["scale_bits"], np.uint16).reshape(n, 1)
    return trits, sb


@pytest.mark.parametrize("fmt", FMTS)
def test_hand_computed_stream(fmt):
    trits, sb = _golden_trits()
    payload = codec.pack_rowsplit(fmt, trits, sb)
    out = q2g64.expand(fmt, GOLD["n"], GOLD["k"], payload)
    want = bytes.fromhex("".join(GOLD["stream_hex"]).replace(" ", ""))
    assert out.tobytes() == want


def test_hand_computed_stream_dequantises_to_trits():
    trits, sb = _golden_trits()
    want = bytes.fromhex("".join(GOLD["stream_hex"]).replace(" ", ""))
    w = q2g64.dequantize(np.frombuffer(want, np.uint8), GOLD["n"], GOLD["k"])
    assert np.array_equal(w[0], trits[0].astype(np.float64))
    assert np.array_equal(w[1], 2.0 * trits[1].astype(np.float64))


@pytest.mark.parametrize("case", CODES["bytes"])
def test_block_code_table_from_page(case):
    # [gguf-explainer] §4.3: codes 00, 01, 10, 11 mean -1, 0, +1, +2 times d
    block = bytes([0x00, 0x38]) + bytes([int(case["byte"], 16)]) * 16  # d = 0.5
    w = q2g64.dequantize(np.frombuffer(block * 2, np.uint8), 1, 128)[0]
    assert list(w[:4] * 2) == case["values"]
    assert np.array_equal(w.reshape(32, 4) * 2, np.tile(case["values"], (32, 1)))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,seed", [(7, 1024, 1), (3, 5120, 2), (5, 1000, 3), (1, 128, 4)])
def test_lossless(fmt, n, k, seed):
    # [tensorsharp] §4.1: the represented values are kept, no requantisation
    rng = np.random.default_rng(seed)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = codec.pack_rowsplit(fmt, trits, sb)
    stream = q2g64.expand(fmt, n, k, payload)
    assert stream.size == q2g64.expanded_bytes(n, k)
    assert np.array_equal(q2g64.dequantize(stream, n, k), P.dequantize(fmt, n, k, payload))
    # both formats holding the same trits expand to the same bytes
    other = FMTS[1 - FMTS.index(fmt)]
    assert np.array_equal(stream, q2g64.expand(other, n, k, codec.pack_rowsplit(other, trits, sb)))


def test_single_weight_positions():
    # one nonzero trit at every position of a 256-weight row lands in block
    # j // 64, byte 2 + (j % 64) // 4, bits 2 * (j % 4), with code 2
    n, k = 1, 256
    sb = np.array([[0x3C00, 0x4400]], np.uint16)
    for j in range(k):
        trits = np.zeros((n, k), np.int8)
        trits[0, j] = 1
        stream = q2g64.expand("PQ2_0_G128", n, k, codec.pack_rowsplit("PQ2_0_G128", trits, sb))
        blocks = stream.reshape(4, 18)
        for b in range(4):
            assert blocks[b, 0] == 0 and blocks[b, 1] == (0x3C if b < 2 else 0x44)
        byte = blocks[j // 64, 2 + (j % 64) // 4]
        assert (byte >> (2 * (j % 4))) & 3 == 2
        assert np.count_nonzero(blocks[:, 2:] != 0x55) == 1


@pytest.mark.parametrize("fmt,byte", [("PQ2_0_G128", 0xFF), ("PTQ1_0_G128", 0xFF)])
def test_non_ternary_values_kept(fmt, byte):
    # PQ2_0 code 3 decodes to +2 and a PTQ1_0 byte past 242 by the digit
    # arithmetic; the 2-bit block keeps the decoded value either way
    n, k = 2, 256
    sb = np.full((n, 2), 0x3C00, np.uint16)
    payload = codec.pack_rowsplit(fmt, np.zeros((n, k), np.int8), sb).copy()
    payload[0] = byte
    w = q2g64.dequantize(q2g64.expand(fmt, n, k, payload), n, k)
    assert np.array_equal(w, P.dequantize(fmt, n, k, payload))
    if fmt == "PQ2_0_G128":
        assert list(w[0, :4]) == [2.0] * 4


def test_projection_equals_plane_projection():
    rng = np.random.default_rng(5)
    n, k = 9, 2048
    trits = synth.trits_uniform(rng, n, k)
    sb = synth.scale_bits_uniform(rng, n, synth.groups_of(k), 0.01, 0.04)
    payload = codec.pack_rowsplit("PTQ1_0_G128", trits, sb)
    xrot = rng.standard_normal((2, k))
    y = q2g64.project(q2g64.expand("PTQ1_0_G128", n, k, payload), n, k, xrot)
    y_ref, _ = P.project_payload("PTQ1_0_G128", n, k, payload, xrot)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)

"""C-ABI library on the CPU: exports, geometry, host packer, validation.

The host packer and geometry are compared bit-exactly with the oracle's own
independent implementation.  Device entry points are only called with
arguments that fail validation, which returns before any HIP call.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import codec as ocodec
from oracle.geometry import row_split_geometry

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "tq.h")
FMTS = ["PQ2_0_G128", "PTQ1_0_G128"]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    lib = tq.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(tq.EXPORTS) == names
    assert re.match(r"^\d+\.\d+\.\d+$", tq.version())


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 1), (3, 127), (5, 128), (7, 1000), (256, 1024),
                                 (17408, 5120), (5120, 17408), (248320, 5120), (12288, 6144)])
def test_geometry_matches_oracle(fmt, n, k):
    assert tq.geometry(fmt, n, k) == dict(row_split_geometry(fmt, n, k))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_packer_bit_exact_on_workload_recipes(cfg):
    c = synth.make_config(cfg, n=48, k=None if cfg != 4 else 5120)
    payload = tq.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
    expect = ocodec.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
    assert np.array_equal(payload, expect)
    vals, sb, bad = tq.unpack_rowsplit(c["fmt"], c["n"], c["k"], payload)
    ovals, osb = ocodec.unpack_rowsplit(c["fmt"], c["n"], c["k"], expect)
    assert np.array_equal(vals, ovals) and np.array_equal(sb, osb) and bad == 0


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 128), (9, 1000), (4, 2176), (2, 130)])
def test_packer_random_shapes(fmt, n, k):
    rng = np.random.default_rng(n * 7919 + k)
    trits = synth.trits_uniform(rng, n, k)
    sb = synth.scale_bits_uniform(rng, n, synth.groups_of(k), 0.01, 0.04)
    assert np.array_equal(tq.pack_rowsplit(fmt, trits, sb), ocodec.pack_rowsplit(fmt, trits, sb))


def test_unpack_reports_non_ternary_codes():
    # PQ2_0 code 3 decodes to +2 and is counted; PTQ1_0 bytes above 242
    # (base) or 80 (high) are counted.
    n, k = 2, 128
    p = tq.pack_rowsplit("PQ2_0_G128", np.zeros((n, k), np.int8), np.full((n, 1), 0x3C00, np.uint16))
    p[0] = 0xFF
    vals, _, bad = tq.unpack_rowsplit("PQ2_0_G128", n, k, p)
    assert bad == 4 and vals[0, :4].tolist() == [2, 2, 2, 2]
    ovals, _ = ocodec.unpack_rowsplit("PQ2_0_G128", n, k, p)
    assert np.array_equal(vals, ovals)
    p = tq.pack_rowsplit("PTQ1_0_G128", np.zeros((n, k), np.int8), np.full((n, 1), 0x3C00, np.uint16))
    geo = tq.geometry("PTQ1_0_G128", n, k)
    p[0] = 250
    p[geo["high_offset"]] = 81
    vals, _, bad = tq.unpack_rowsplit("PTQ1_0_G128", n, k, p)
    ovals, _ = ocodec.unpack_rowsplit("PTQ1_0_G128", n, k, p)
    assert bad == 2 and np.array_equal(vals, ovals)


def expect_error(status, fn, *args):
    with pytest.raises(tq.TQError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_host_errors():
    msg = expect_error(2, tq.geometry, 99, 4, 128)
    assert "unknown numeric format" in msg
    expect_error(5, tq.geometry, "PQ2_0_G128", 0, 128)
    expect_error(5, tq.geometry, "PQ2_0_G128", 4, -1)
    # sizes that would wrap 64-bit arithmetic are refused, not wrapped
    for fmt in FMTS:
        msg = expect_error(5, tq.geometry, fmt, 1 << 62, 1 << 20)
        assert "too large" in msg
        expect_error(5, tq.geometry, fmt, (1 << 40) + 1, 1 << 25)
    # the largest accepted payload is bounded by 2^62 bytes
    g = tq.geometry("PQ2_0_G128", 1 << 30, 1 << 20)
    assert g["payload_bytes"] < (1 << 63)
    bad = np.full((2, 128), 2, np.int8)
    expect_error(8, tq.pack_rowsplit, "PQ2_0_G128", bad, np.zeros((2, 1), np.uint16))
    # payload size mismatch: message in the pages' style
    L = tq.lib()
    trits = np.zeros((2, 128), np.int8)
    sb = np.zeros((2, 1), np.uint16)
    buf = np.zeros(10, np.uint8)
    st = L.tq_pack_rowsplit(142, 2, 128, trits.ctypes.data, sb.ctypes.data, buf.ctypes.data, 10)
    assert st == 3
    assert "stores 10 bytes; layout requires 260" in L.tq_last_error().decode()


DEV = 1 << 20      # a 256-byte aligned stand-in address; never dereferenced


def test_device_entry_validation_without_gpu():
    L = tq.lib()
    pb = tq.geometry("PQ2_0_G128", 64, 1024)["payload_bytes"]
    # wrong payload size
    assert L.tq_gemv_rowsplit(DEV, pb + 1, 142, 64, 1024, DEV, 0, 1, 1024, DEV, 64, None) == 3
    # misaligned payload
    assert L.tq_gemv_rowsplit(DEV + 16, pb, 142, 64, 1024, DEV, 0, 1, 1024, DEV, 64, None) == 4
    # batch out of range, k not a multiple of 128
    assert L.tq_gemv_rowsplit(DEV, pb, 142, 64, 1024, DEV, 0, 9, 1024, DEV, 64, None) == 5
    pb2 = tq.geometry("PQ2_0_G128", 64, 1000)["payload_bytes"]
    assert L.tq_gemv_rowsplit(DEV, pb2, 142, 64, 1000, DEV, 0, 1, 1000, DEV, 64, None) == 5
    # leading dimensions, null pointers, bad dtype, misaligned activations
    assert L.tq_gemv_rowsplit(DEV, pb, 142, 64, 1024, DEV, 0, 1, 512, DEV, 64, None) == 1
    assert L.tq_gemv_rowsplit(DEV, pb, 142, 64, 1024, None, 0, 1, 1024, DEV, 64, None) == 1
    assert L.tq_gemv_rowsplit(DEV, pb, 142, 64, 1024, DEV, 7, 1, 1024, DEV, 64, None) == 1
    assert L.tq_gemv_rowsplit(DEV, pb, 142, 64, 1024, DEV + 8, 0, 1, 1024, DEV, 64, None) == 4
    # transform: k must be a multiple of 1024; inverse flag; null signs
    assert L.tq_hadamard_signed(DEV, 0, 1, 1536, 1536, DEV, 0, DEV, 0, 1536, None) == 5
    assert L.tq_hadamard_signed(DEV, 0, 1, 1024, 1024, DEV, 2, DEV, 0, 1024, None) == 1
    assert L.tq_hadamard_signed(DEV, 0, 1, 1024, 1024, None, 0, DEV, 0, 1024, None) == 1
    assert L.tq_hadamard_signed(DEV, 0, 1, 1024, 1024, DEV, 0, DEV, 1, 1024, None) == 1  # in-place dtype change
    assert L.tq_hadamard_signed(DEV, 0, -1, 1024, 1024, DEV, 0, DEV, 0, 1024, None) == 5
    # GEMM dtypes and shapes
    assert L.tq_gemm_rowsplit(DEV, pb, 142, 64, 1024, DEV, 0, 4, 1024, DEV, 0, 64, None) == 1
    assert L.tq_gemm_rowsplit(DEV, pb, 142, 64, 1024, DEV, 2, 4, 1024, DEV, 2, 64, None) == 1
    assert L.tq_gemm_rowsplit(DEV, pb, 143, 64, 1024, DEV, 2, 4, 1024, DEV, 0, 64, None) == 3
    # GEMM limits: k <= 2^20 (shape), ldx < 2^22 (argument)
    kb = (1 << 20) + 128
    pbk = tq.geometry("PQ2_0_G128", 64, kb)["payload_bytes"]
    assert L.tq_gemm_rowsplit(DEV, pbk, 142, 64, kb, DEV, 2, 4, kb, DEV, 0, 64, None) == 5
    assert L.tq_gemm_rowsplit(DEV, pb, 142, 64, 1024, DEV, 2, 4, 1 << 22, DEV, 0, 64, None) == 1
    # fused transform + GEMV: k multiple of 1024, null signs, then the
    # requests the one-launch kernel does not cover (PTQ1_0, batch > 1)
    f = L.tq_rotated_gemv_rowsplit
    pb4 = tq.geometry("PQ2_0_G128", 64, 1152)["payload_bytes"]
    assert f(DEV, pb4, 142, 64, 1152, DEV, 0, 1, 1152, DEV, DEV, 64, None) == 5
    assert f(DEV, pb, 142, 64, 1024, DEV, 0, 1, 1024, None, DEV, 64, None) == 1
    assert f(DEV, pb, 142, 64, 1024, DEV, 0, 9, 1024, DEV, DEV, 64, None) == 5
    assert f(DEV, pb, 142, 64, 1024, DEV + 8, 0, 1, 1024, DEV, DEV, 64, None) == 4
    assert f(DEV, pb, 142, 64, 1024, DEV, 0, 2, 1024, DEV, DEV, 64, None) == 6
    pt = tq.geometry("PTQ1_0_G128", 64, 1024)["payload_bytes"]
    assert f(DEV, pt, 143, 64, 1024, DEV, 0, 1, 1024, DEV, DEV, 64, None) == 6
    assert b"tq_hadamard_signed then tq_gemv_rowsplit" in L.tq_last_error()
    # embedding: k must be a multiple of 1024
    pb3 = tq.geometry("PQ2_0_G128", 64, 1152)["payload_bytes"]
    assert L.tq_embed_rows_inverse(DEV, pb3, 142, 64, 1152, DEV, 4, DEV, DEV, 1152, None, None) == 5
    assert L.tq_embed_rows_inverse(DEV, pb, 142, 64, 1024, DEV, -1, DEV, DEV, 1024, None, None) == 5
    # decode hook: unknown format
    assert L.tq_decode_rowsplit(DEV, pb, 141, 64, 1024, DEV, 1, DEV, DEV, None) == 2
    # a validation failure leaves a message
    assert L.tq_decode_rowsplit(DEV, pb, 141, 64, 1024, DEV, 1, DEV, DEV, None) == 2
    assert b"unknown numeric format" in L.tq_last_error()


def test_stream_read_validation_without_gpu():
    L = tq.lib()
    assert L.tq_stream_read(None, 1024, DEV, None) == 1
    assert L.tq_stream_read(DEV, 1024, None, None) == 1
    assert L.tq_stream_read(DEV, 0, DEV, None) == 5
    assert L.tq_stream_read(DEV, 1000, DEV, None) == 5
    assert L.tq_stream_read(DEV, 1 << 41, DEV, None) == 5
    assert L.tq_stream_read(DEV + 8, 1024, DEV, None) == 4
    assert L.tq_stream_read(DEV, 1024, DEV + 2, None) == 4

"""Grouped head order entry points on the CPU: argument validation only
(arguments that fail validation return before any HIP call)."""

import ternary_quantized_amd as tq

DEV = 1 << 20      # a 256-byte aligned stand-in address; never dereferenced


def test_grouped_transform_validation_without_gpu():
    L = tq.lib()
    f = L.tq_hadamard_signed_grouped
    k = 6144
    assert f(DEV, 0, 1, k, k, 3, 16, 64, DEV, DEV * 8, 0, k, None) == 5     # product != k
    assert f(DEV, 0, 1, k, k, 3, 16, 0, DEV, DEV * 8, 0, k, None) == 5      # head_dim 0
    assert f(DEV, 0, 1, 6000, 6000, 3, 16, 125, DEV, DEV * 8, 0, 6000, None) == 5
    assert f(DEV, 0, 1, 3072, 3072, 1, 3, 1000, DEV, DEV * 8, 0, 3072, None) == 5  # not /16
    assert f(DEV, 0, 1, k, k, 0, 16, 384, DEV, DEV * 8, 0, k, None) == 5     # tiles 0
    assert f(DEV, 0, 1, k, k, 3, 16, 128, None, DEV * 8, 0, k, None) == 1   # signs
    assert f(DEV, 0, 1, k, k, 3, 16, 128, DEV, DEV, 0, k, None) == 1        # in place
    assert b"overlap" in L.tq_last_error()
    assert f(DEV + 8, 0, 1, k, k, 3, 16, 128, DEV, DEV * 8, 0, k, None) == 4
    assert f(DEV, 0, 0, k, k, 3, 16, 128, DEV, DEV, 0, k, None) == 0        # no rows: no-op


def test_grouped_fused_validation_without_gpu():
    L = tq.lib()
    f = L.tq_rotated_gemv_rowsplit_grouped
    n, k = 64, 6144
    pb = tq.geometry("PQ2_0_G128", n, k)["payload_bytes"]
    assert f(DEV, pb, 142, n, k, DEV, 1, 1, k, 3, 16, 64, DEV, DEV, n, None) == 5
    assert f(DEV, pb + 1, 142, n, k, DEV, 1, 1, k, 3, 16, 128, DEV, DEV, n, None) == 3
    assert f(DEV, pb, 142, n, k, DEV, 1, 1, k, 3, 16, 128, None, DEV, n, None) == 1
    assert f(DEV, pb, 142, n, k, DEV, 1, 2, k, 3, 16, 128, DEV, DEV, n, None) == 6
    pt = tq.geometry("PTQ1_0_G128", n, k)["payload_bytes"]
    assert f(DEV, pt, 143, n, k, DEV, 1, 1, k, 3, 16, 128, DEV, DEV, n, None) == 6
    assert b"tq_hadamard_signed_grouped then tq_gemv_rowsplit" in L.tq_last_error()

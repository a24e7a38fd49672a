"""G64 block-stream entry points on the CPU: sizes against the oracle and
argument validation (device entry points are only called with arguments that
fail validation, which returns before any HIP call)."""

import pytest

import ternary_quantized_amd as tq
from oracle import q2g64

DEV = 1 << 20      # a 256-byte aligned stand-in address; never dereferenced


@pytest.mark.parametrize("n,k", [(1, 1), (3, 127), (5, 1000), (17408, 5120), (5120, 17408),
                                 (248320, 5120)])
def test_g64_bytes_matches_oracle(n, k):
    assert tq.g64_bytes(n, k) == q2g64.expanded_bytes(n, k)


def test_expand_validation_without_gpu():
    L = tq.lib()
    n, k = 64, 1024
    pb = tq.geometry("PQ2_0_G128", n, k)["payload_bytes"]
    gb = tq.g64_bytes(n, k)
    f = L.tq_expand_g64
    assert f(DEV, pb + 1, 142, n, k, DEV * 4, gb, None) == 3          # payload size
    assert f(DEV, pb, 142, n, k, DEV * 4, gb - 18, None) == 3         # stream size
    assert b"block stream stores" in L.tq_last_error()
    assert f(DEV, pb, 141, n, k, DEV * 4, gb, None) == 2              # format
    assert f(DEV + 16, pb, 142, n, k, DEV * 4, gb, None) == 4         # payload alignment
    assert f(DEV, pb, 142, n, k, DEV * 4 + 4, gb, None) == 4          # stream alignment
    assert f(DEV, pb, 142, n, k, None, gb, None) == 1                 # null stream
    assert f(DEV, pb, 142, n, k, DEV + 256, gb, None) == 1            # overlap
    assert f(DEV, pb, 142, 0, k, DEV * 4, gb, None) == 5              # shape


def test_gemv_validation_without_gpu():
    L = tq.lib()
    f = L.tq_gemv_g64
    n, k = 64, 5120
    gb = tq.g64_bytes(n, k)
    assert f(DEV, gb + 1, n, k, DEV, 0, 1, k, DEV, n, None) == 3      # size
    assert f(DEV, tq.g64_bytes(n, 1152), n, 1152, DEV, 0, 1, 1152, DEV, n, None) == 5
    big = 18 * 1024
    assert f(DEV, tq.g64_bytes(n, big), n, big, DEV, 0, 1, big, DEV, n, None) == 5
    assert f(DEV, gb, n, k, DEV, 7, 1, k, DEV, n, None) == 1          # dtype
    assert f(DEV, gb, n, k, DEV, 0, 1, k - 8, DEV, n, None) == 1      # ldx
    assert f(DEV, gb, n, k, None, 0, 1, k, DEV, n, None) == 1         # null x
    assert f(DEV + 4, gb, n, k, DEV, 0, 1, k, DEV, n, None) == 4      # blocks alignment
    assert f(DEV, gb, n, k, DEV + 8, 0, 1, k, DEV, n, None) == 4      # x alignment
    assert f(DEV, gb, n, k, DEV, 0, 0, k, DEV, n, None) == 5          # batch 0
    assert f(DEV, gb, n, k, DEV, 0, 2, k, DEV, n, None) == 6          # batch 2: not covered
    assert b"batch 1 only" in L.tq_last_error()

"""Helpers for the GPU parity tests: device copies of the seeded inputs and
the element-wise acceptance check against the oracle."""

import sys

import numpy as np

import ternary_quantized_amd as tq
from oracle import transform as T


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def payload_dev(torch, fmt, trits, scale_bits):
    return dev(torch, tq.pack_rowsplit(fmt, trits, scale_bits))


def signs_dev(torch, sign_bits):
    return dev(torch, np.asarray(sign_bits, np.uint16).view(np.int16))


def x_dev(torch, x, xdt):
    """Activations on the device: float32 as is, bf16/f16 from bit patterns."""
    if xdt == "f32":
        return dev(torch, np.asarray(x, np.float32))
    t = dev(torch, np.asarray(x, np.uint16).view(np.int16))
    return t.view(torch.bfloat16 if xdt == "bf16" else torch.float16)


def x_f64(x, xdt):
    if xdt == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if xdt == "bf16":
        return T.bf16_bits_to_f64(x)
    return T.fp16_bits_to_f64(x)


def to_f64(torch, t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_within(got, expect, bound, what):
    got = np.asarray(got, np.float64)
    d = np.abs(got - expect)
    ratio = float((d / bound).max()) if d.size else 0.0
    say("%s: %d outputs, max |err|/bound = %.3g" % (what, d.size, ratio))
    bad = np.argwhere(~(d <= bound))
    assert bad.size == 0, "%s: %d outputs out of bound, first at %s: got %r expect %r bound %r" % (
        what, len(bad), bad[0], got[tuple(bad[0])], expect[tuple(bad[0])], bound[tuple(bad[0])])
    return ratio


def pq2_b1_kernel(n, k):
    """Which kernel the library runs for a batch-1 PQ2_0 product of n rows of
    k weights, by its shape rule: "f4", the matrix-core kernel (rows of a
    multiple of 1024 weights up to 8192, at least 2^29 weights), else "dot",
    the dot-product kernels."""
    if k >= 1024 and k % 1024 == 0 and k <= 8192 and n * k >= 1 << 29:
        return "f4"
    return "dot"

"""GPU parity of every device entry point against the oracle, through the C ABI.

Inputs are the seeded synthetic recipes at sizes the oracle finishes in
seconds; shapes span several tiles plus ragged tails.  The bar: bit-exact for
decoded codes and scale bits and for integer-valued cases; otherwise, per
output, |gpu - oracle| <= 1e-3 * sum_j |w_j x'_j| + 1e-5 (projections) or
1e-3 * ||block||_1 / 32 + 1e-5 plus the output dtype's rounding (transforms).
"""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import codec, projection as P, transform as T
from gpu_util import (assert_within, dev, payload_dev, say, signs_dev, to_f64, x_dev, x_f64)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROUND = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
TORCH_DT = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def rand_x(rng, rows, k, xdt, scale=1.0):
    x = (rng.standard_normal((rows, k)) * scale).astype(np.float32)
    if xdt == "f32":
        return x
    if xdt == "bf16":
        return synth.f32_to_bf16_bits(x)
    return x.astype(np.float16).view(np.uint16)


# ------------------------------------------------------------- transform ---
@pytest.mark.parametrize("inverse", [0, 1])
def test_hadamard_basis_vectors_bit_exact(inverse):
    rng = np.random.default_rng(1)
    k = 2048
    sbits = synth.sign_bits(rng, k)
    d = T.bf16_bits_to_f64(sbits)
    x = np.zeros((k, k), np.float32)
    x[np.arange(k), np.arange(k)] = 1.0
    say("hadamard basis k=%d inverse=%d" % (k, inverse))
    y = tq.hadamard_signed(x_dev(torch, x, "f32"), signs_dev(torch, sbits), inverse=bool(inverse))
    torch.cuda.synchronize()
    expect = (T.inverse if inverse else T.forward)(x.astype(np.float64), d)
    assert np.array_equal(to_f64(torch, y), expect)


@pytest.mark.parametrize("xdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("ydt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("inverse", [0, 1])
@pytest.mark.parametrize("rows,k", [(1, 1024), (7, 5120), (3, 17408)])
def test_hadamard_parity(xdt, ydt, inverse, rows, k):
    rng = np.random.default_rng(rows * k + inverse)
    sbits = synth.sign_bits(rng, k)
    x = rand_x(rng, rows, k, xdt, scale=3.0)
    say("hadamard %s->%s inverse=%d rows=%d k=%d" % (xdt, ydt, inverse, rows, k))
    y = tq.hadamard_signed(x_dev(torch, x, xdt), signs_dev(torch, sbits), inverse=bool(inverse),
                           out_dtype=getattr(torch, TORCH_DT[ydt]))
    torch.cuda.synchronize()
    xf = x_f64(x, xdt)
    d = T.bf16_bits_to_f64(sbits)
    expect = (T.inverse if inverse else T.forward)(xf, d)
    bound = 1e-3 * T.block_l1_over_32(xf) + 1e-5 + ROUND[ydt] * np.abs(expect)
    assert_within(to_f64(torch, y), expect, bound, "hadamard")


def test_hadamard_in_place_strided_and_stream():
    rng = np.random.default_rng(5)
    k, rows = 3072, 5
    sbits = synth.sign_bits(rng, k)
    x = rand_x(rng, rows, k, "f32")
    big = torch.zeros((rows, k + 64), dtype=torch.float32, device="cuda")
    big[:, :k] = x_dev(torch, x, "f32")
    view = big[:, :k]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tq.hadamard_signed(view, signs_dev(torch, sbits), out=view)
    s.synchronize()
    expect = T.forward(x.astype(np.float64), T.bf16_bits_to_f64(sbits))
    bound = 1e-3 * T.block_l1_over_32(x.astype(np.float64)) + 1e-5
    assert_within(to_f64(torch, view), expect, bound, "hadamard in-place")
    assert not big[:, k:].any()
    empty = torch.zeros((0, k), dtype=torch.float32, device="cuda")
    assert tq.hadamard_signed(empty, signs_dev(torch, sbits)).shape == (0, k)


@pytest.mark.parametrize("xdt,ydt,inverse,rows,k,in_place",
                         [("bf16", "f16", 0, 3001, 3072, False), ("f32", "f32", 1, 2500, 2048, True),
                          ("f16", "f16", 0, 4099, 1024, True)])
def test_hadamard_many_rows(xdt, ydt, inverse, rows, k, in_place):
    """Thousands of rows: one wave per 1024-element block, four per
    workgroup, so the grid ends in a partly filled last workgroup when the
    block count is not a multiple of four (3001 rows x 3 blocks); in place
    too."""
    rng = np.random.default_rng(rows + k)
    sbits = synth.sign_bits(rng, k)
    x = rand_x(rng, rows, k, xdt, scale=2.0)
    say("hadamard many rows %s->%s inverse=%d rows=%d k=%d in_place=%s" % (xdt, ydt, inverse, rows, k, in_place))
    xd = x_dev(torch, x, xdt)
    kw = dict(out=xd) if in_place else dict(out_dtype=getattr(torch, TORCH_DT[ydt]))
    y = tq.hadamard_signed(xd, signs_dev(torch, sbits), inverse=bool(inverse), **kw)
    torch.cuda.synchronize()
    xf = x_f64(x, xdt)
    expect = (T.inverse if inverse else T.forward)(xf, T.bf16_bits_to_f64(sbits))
    bound = 1e-3 * T.block_l1_over_32(xf) + 1e-5 + ROUND[ydt] * np.abs(expect)
    assert_within(to_f64(torch, y), expect, bound, "hadamard many rows")


# ------------------------------------------------------------ decode hook --
@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
def test_decode_bit_exact(fmt):
    rng = np.random.default_rng(11)
    n, k = 300, 1000
    trits = synth.trits_uniform(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = tq.pack_rowsplit(fmt, trits, sb)
    # plant non-ternary codes: the decode follows the digit/code arithmetic
    payload[5] = 0xFF if fmt == "PQ2_0_G128" else 250
    rows = np.array([0, 299, 17, 17, 150, -1, 300], np.int32)
    vals, sbits = tq.decode_rowsplit(dev(torch, payload), fmt, n, k, dev(torch, rows))
    torch.cuda.synchronize()
    ovals, osb = codec.unpack_rowsplit(fmt, n, k, payload)
    v = vals.cpu().numpy()
    s = sbits.cpu().numpy().view(np.uint16)
    assert np.array_equal(v[:5], ovals[rows[:5]]) and np.array_equal(s[:5], osb[rows[:5]])
    assert not v[5:].any() and not s[5:].any()


# ------------------------------------------------------------------ GEMV ---
def gemv_case(fmt, n, k, batch, xdt, seed, p_zero=0.4):
    rng = np.random.default_rng(seed)
    trits = synth.trits_sparse(rng, n, k, p_zero)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    xr = rand_x(rng, batch, k, xdt)
    payload = tq.pack_rowsplit(fmt, trits, sb)
    return payload, xr


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("n,k", [(1, 128), (7, 1024), (64, 2176), (1000, 5120), (33, 17408)])
@pytest.mark.parametrize("batch", [1, 2, 3, 5, 8])
def test_gemv_parity(fmt, n, k, batch):
    xdt = ["f32", "bf16", "f16"][(n + batch) % 3]
    payload, xr = gemv_case(fmt, n, k, batch, xdt, seed=n * 31 + k + batch)
    say("gemv %s n=%d k=%d batch=%d x=%s" % (fmt, n, k, batch, xdt))
    y = tq.gemv_rowsplit(dev(torch, payload), fmt, n, k, x_dev(torch, xr, xdt))
    torch.cuda.synchronize()
    expect, bound = P.project_payload(fmt, n, k, payload, x_f64(xr, xdt))
    assert_within(to_f64(torch, y), expect, bound, "gemv")


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("k", [1024, 4096, 11264, 17408])
@pytest.mark.parametrize("batch,xdt", [(2, "f16"), (5, "bf16"), (6, "f16"), (8, "bf16"), (7, "f16"),
                                       (8, "f32")])
def test_gemv_row_quads_batches(fmt, k, batch, xdt):
    """The row-quad MFMA GEMV at two to eight batch rows: with 16-bit
    activations five to eight rows run in one pass that decodes each weight
    once for two groups of four rows (every wave count and slot count of the
    split, partial second groups); fp32 activations run passes of four."""
    n = 1000 if k < 17408 else 333
    payload, xr = gemv_case(fmt, n, k, batch, xdt, seed=k + batch)
    say("gemv row quads %s n=%d k=%d batch=%d x=%s" % (fmt, n, k, batch, xdt))
    y = tq.gemv_rowsplit(dev(torch, payload), fmt, n, k, x_dev(torch, xr, xdt))
    torch.cuda.synchronize()
    expect, bound = P.project_payload(fmt, n, k, payload, x_f64(xr, xdt))
    assert_within(to_f64(torch, y), expect, bound, "gemv row quads")


@pytest.mark.parametrize("fmt,k", [("PQ2_0_G128", 65536), ("PQ2_0_G128", 25600), ("PTQ1_0_G128", 32768),
                                   ("PTQ1_0_G128", 24576)])
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
def test_gemv_longest_rows(fmt, k, batch):
    """The longest rows the GEMV accepts (k = 65536 for PQ2_0, 32768 for
    PTQ1_0) and the first rows past the row-quad kernel's reach, where the
    lane-team kernels take over."""
    n = 37
    xdt = ["f32", "bf16", "f16"][batch % 3]
    payload, xr = gemv_case(fmt, n, k, batch, xdt, seed=k + batch)
    say("gemv longest rows %s n=%d k=%d batch=%d x=%s" % (fmt, n, k, batch, xdt))
    y = tq.gemv_rowsplit(dev(torch, payload), fmt, n, k, x_dev(torch, xr, xdt))
    torch.cuda.synchronize()
    expect, bound = P.project_payload(fmt, n, k, payload, x_f64(xr, xdt))
    assert_within(to_f64(torch, y), expect, bound, "gemv longest rows")


# ------------------------------------------- fused transform + GEMV ---
@pytest.mark.parametrize("n,k", [(1, 1024), (77, 3072), (1000, 5120), (300, 11264)])
@pytest.mark.parametrize("xdt", ["f32", "bf16", "f16"])
def test_rotated_gemv_parity_and_equals_two_launches(n, k, xdt):
    """One launch = tq_hadamard_signed (binary16 out) then tq_gemv_rowsplit,
    bit for bit; and within the oracle's bound of W . H(D.x)/32 computed in
    float64 from the unrotated input."""
    rng = np.random.default_rng(n + k)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = tq.pack_rowsplit("PQ2_0_G128", trits, sb)
    x = rand_x(rng, 1, k, xdt, scale=3.0)
    sign_bits = synth.sign_bits(rng, k)
    say("rotated gemv n=%d k=%d x=%s" % (n, k, xdt))
    pd, xd, sd = dev(torch, payload), x_dev(torch, x, xdt), signs_dev(torch, sign_bits)
    y = tq.rotated_gemv_rowsplit(pd, "PQ2_0_G128", n, k, xd, sd)
    xr = tq.hadamard_signed(xd, sd, out_dtype=torch.float16)
    y2 = tq.gemv_rowsplit(pd, "PQ2_0_G128", n, k, xr)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    xrot = T.forward(x_f64(x, xdt), T.bf16_bits_to_f64(sign_bits))
    expect, bound = P.project_payload("PQ2_0_G128", n, k, payload, xrot)
    # x' is rounded to binary16 (relative 2^-11 per element) before the dot,
    # which stays inside the stated tolerance
    assert_within(to_f64(torch, y), expect, bound, "rotated gemv")


def test_rotated_gemv_unsupported_requests_enqueue_nothing():
    rng = np.random.default_rng(9)
    n, k = 64, 2048
    sign_bits = synth.sign_bits(rng, k)
    sd = signs_dev(torch, sign_bits)
    x = x_dev(torch, rand_x(rng, 2, k, "f16"), "f16")
    for fmt, batch in (("PTQ1_0_G128", 1), ("PQ2_0_G128", 2)):
        trits = synth.trits_sparse(rng, n, k)
        sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
        pd = dev(torch, tq.pack_rowsplit(fmt, trits, sb))
        out = torch.full((batch, n), 7.0, device="cuda")
        with pytest.raises(tq.TQError) as e:
            tq.rotated_gemv_rowsplit(pd, fmt, n, k, x[:batch], sd, out=out)
        assert e.value.status == 6
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
def test_gemv_integer_exact_and_deterministic(fmt):
    # scales 1.0 and integer activations in [-8, 8] (exact in binary16):
    # every partial sum is an integer below 2^24, so the result is exact.
    rng = np.random.default_rng(3)
    n, k = 777, 5120
    trits = synth.trits_uniform(rng, n, k)
    sb = np.full((n, k // 128), 0x3C00, np.uint16)
    payload = tq.pack_rowsplit(fmt, trits, sb)
    xi = rng.integers(-8, 9, size=(4, k)).astype(np.float32)
    pd, xd = dev(torch, payload), x_dev(torch, xi, "f32")
    y1 = tq.gemv_rowsplit(pd, fmt, n, k, xd)
    y2 = tq.gemv_rowsplit(pd, fmt, n, k, xd)
    torch.cuda.synchronize()
    expect = xi.astype(np.int64) @ trits.T.astype(np.int64)
    assert np.array_equal(y1.cpu().numpy(), expect.astype(np.float32))
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("n,k", [(40000, 2048), (40000, 5120), (3001, 11264), (9000, 13312),
                                 (7000, 17408)])
def test_gemv_batch1_multi_pass_integer_exact(n, k):
    """Batch-1 PQ2_0 rows over several passes of the persistent grid (and
    the last, partial one), alone and fused with the transform: scales 1.0
    and integer activations make every partial sum an exact integer."""
    rng = np.random.default_rng(n + k)
    trits = synth.trits_uniform(rng, n, k)
    sb = np.full((n, k // 128), 0x3C00, np.uint16)
    payload = tq.pack_rowsplit("PQ2_0_G128", trits, sb)
    xi = rng.integers(-8, 9, size=(1, k)).astype(np.float32)
    say("gemv batch 1 multi-pass n=%d k=%d" % (n, k))
    pd = dev(torch, payload)
    y = tq.gemv_rowsplit(pd, "PQ2_0_G128", n, k, x_dev(torch, xi, "f32"))
    if k > 11264:  # the one-launch step covers k <= 11264
        torch.cuda.synchronize()
        expect = (xi.astype(np.int64) @ trits.T.astype(np.int64)).astype(np.float32)
        assert np.array_equal(y.cpu().numpy(), expect)
        return
    # fused: the unrotated input D.(H.z)/32 (multiples of 1/32, exact in
    # fp32) rotates back to z exactly, so the fused step is integer-exact too
    sign_bits = synth.sign_bits(rng, k)
    xu = T.inverse(xi.astype(np.float64), T.bf16_bits_to_f64(sign_bits)).astype(np.float32)
    yf = tq.rotated_gemv_rowsplit(pd, "PQ2_0_G128", n, k, x_dev(torch, xu, "f32"),
                                  signs_dev(torch, sign_bits))
    torch.cuda.synchronize()
    expect = (xi.astype(np.int64) @ trits.T.astype(np.int64)).astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), expect)
    assert np.array_equal(yf.cpu().numpy(), expect)


def test_gemv_rows_of_four_pieces_past_the_pair_split():
    """Rows of four 4096-weight pieces run split over wave pairs while a
    pair needs at most eight passes; 41000 rows at k = 16384 need nine, so
    the launch falls back to one wave per row.  Integer data (scales 1.0,
    integer activations) make each row exact; a spread sample of rows,
    the first and last included, is checked against integer arithmetic."""
    n, k = 41000, 16384
    rng = np.random.default_rng(n + k)
    trits = synth.trits_uniform(rng, n, k)
    sb = np.full((n, k // 128), 0x3C00, np.uint16)
    payload = tq.pack_rowsplit("PQ2_0_G128", trits, sb)
    xi = rng.integers(-8, 9, size=(1, k)).astype(np.float32)
    say("gemv pair-split fallback n=%d k=%d" % (n, k))
    y = tq.gemv_rowsplit(dev(torch, payload), "PQ2_0_G128", n, k, x_dev(torch, xi, "f32"))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, n, 97), np.arange(n - 40, n)]))
    expect = (trits[rows].astype(np.int64) @ xi[0].astype(np.int64)).astype(np.float32)
    assert np.array_equal(y.cpu().numpy()[0, rows], expect)


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
def test_gemv_non_ternary_codes_follow_decode_arithmetic(fmt):
    n, k = 40, 1024
    payload, xr = gemv_case(fmt, n, k, 1, "f32", seed=9)
    payload[0:64] = 0xFF if fmt == "PQ2_0_G128" else 251
    y = tq.gemv_rowsplit(dev(torch, payload), fmt, n, k, x_dev(torch, xr, "f32"))
    torch.cuda.synchronize()
    expect, bound = P.project_payload(fmt, n, k, payload, x_f64(xr, "f32"))
    assert_within(to_f64(torch, y), expect, bound, "gemv non-ternary")


# ------------------------------------------------------------------ GEMM ---
@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (17, 200, 1024), (128, 384, 2048), (300, 130, 1152)])
@pytest.mark.parametrize("xdt,ydt", [("f16", "f32"), ("bf16", "f32"), ("f16", "bf16")])
def test_gemm_parity(fmt, m, n, k, xdt, ydt):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    x = rand_x(rng, m, k, xdt)
    payload = tq.pack_rowsplit(fmt, trits, sb)
    say("gemm %s m=%d n=%d k=%d x=%s y=%s" % (fmt, m, n, k, xdt, ydt))
    y = tq.gemm_rowsplit(dev(torch, payload), fmt, n, k, x_dev(torch, x, xdt),
                         out_dtype=getattr(torch, TORCH_DT[ydt]))
    torch.cuda.synchronize()
    expect, bound = P.project_payload(fmt, n, k, payload, x_f64(x, xdt))
    if xdt == "bf16":
        # bf16 input is rounded to binary16 before the product
        expect16, _ = P.project_payload(fmt, n, k, payload,
                                        x_f64(x_f64(x, xdt).astype(np.float16).view(np.uint16), "f16"))
        assert np.abs(expect16 - expect).max() <= (bound * 0.5).max()
    bound = bound + ROUND[ydt] * np.abs(expect)
    assert_within(to_f64(torch, y), expect, bound, "gemm")


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
def test_gemm_integer_exact_and_matches_gemv(fmt):
    rng = np.random.default_rng(4)
    m, n, k = 96, 320, 2048
    trits = synth.trits_uniform(rng, n, k)
    sb = np.full((n, k // 128), 0x3C00, np.uint16)
    payload = dev(torch, tq.pack_rowsplit(fmt, trits, sb))
    xi = rng.integers(-8, 9, size=(m, k)).astype(np.float16)
    xd = dev(torch, xi.view(np.uint16).view(np.int16)).view(torch.float16)
    y = tq.gemm_rowsplit(payload, fmt, n, k, xd)
    y2 = tq.gemm_rowsplit(payload, fmt, n, k, xd)
    yv = tq.gemv_rowsplit(payload, fmt, n, k, xd[:8].contiguous())
    torch.cuda.synchronize()
    expect = xi.astype(np.int64) @ trits.T.astype(np.int64)
    assert np.array_equal(y.cpu().numpy(), expect.astype(np.float32))
    assert torch.equal(y, y2)
    assert torch.equal(yv, y[:8])


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("case", ["xcd_split", "plain_split", "two_steps"])
def test_gemm_tail_split_integer_exact(case, fmt):
    """Tile counts just past a whole round of the device: the left-over
    256 x 256 tiles run as 128 x 64 sub-tiles.  Integer data make every
    output exact, so any tile or sub-tile mapping slip shows."""
    cus = _cus()
    if case == "xcd_split":      # tiles % 8 == 0, left-over tiles % 8 == 0
        tm = 8
        tn = (cus + cus // 8) // tm
        m, n, k = tm * 256 - 37, tn * 256 - 100, 256
    elif case == "plain_split":  # tile count not a multiple of 8
        tm = 7
        tn = -(-(cus + 3) // tm)
        m, n, k = tm * 256 - 5, tn * 256 - 17, 256
    else:                        # smallest k: two steps
        tm = 8
        tn = (cus + cus // 8) // tm
        m, n, k = tm * 256, tn * 256, 128
    rng = np.random.default_rng(len(case))
    trits = synth.trits_uniform(rng, n, k)
    sb = np.full((n, k // 128), 0x3C00, np.uint16)
    payload = dev(torch, tq.pack_rowsplit(fmt, trits, sb))
    xi = rng.integers(-8, 9, size=(m, k)).astype(np.float16)
    xd = dev(torch, xi.view(np.uint16).view(np.int16)).view(torch.float16)
    say("gemm tail split %s %s m=%d n=%d k=%d cus=%d" % (fmt, case, m, n, k, cus))
    y = tq.gemm_rowsplit(payload, fmt, n, k, xd)
    torch.cuda.synchronize()
    expect = xi.astype(np.float64) @ trits.T.astype(np.float64)  # exact: |sum| <= 2048
    got = y.cpu().numpy()
    bad = np.argwhere(got != expect.astype(np.float32))
    assert bad.size == 0, "first mismatches (row, col): %s" % bad[:5].tolist()


# ------------------------------------------------------------- embedding ---
@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("n,k", [(50, 1024), (300, 5120)])
def test_embed_parity_and_bad_ids(fmt, n, k):
    rng = np.random.default_rng(n + k)
    trits = synth.trits_uniform(rng, n, k)
    sb = synth.scale_bits_uniform(rng, n, k // 128, 0.01, 0.04)
    sbits = synth.sign_bits(rng, k)
    payload = tq.pack_rowsplit(fmt, trits, sb)
    ids = np.concatenate([rng.integers(0, n, 20), [0, n - 1, 3, 3]]).astype(np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = tq.embed_rows_inverse(dev(torch, payload), fmt, n, k, dev(torch, ids),
                                signs_dev(torch, sbits), err_word=err)
    torch.cuda.synchronize()
    expect, scale = P.embed_rows_inverse(fmt, n, k, payload, ids, T.bf16_bits_to_f64(sbits))
    assert_within(to_f64(torch, out), expect, 1e-3 * scale + 1e-5, "embed")
    assert int(err.item()) == 0
    bad = np.array([1, -5, n, 2], np.int32)
    out = tq.embed_rows_inverse(dev(torch, payload), fmt, n, k, dev(torch, bad),
                                signs_dev(torch, sbits), err_word=err)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert int(err.item()) == 1 and not o[1].any() and not o[2].any()
    e2, _ = P.embed_rows_inverse(fmt, n, k, payload, bad[[0, 3]], T.bf16_bits_to_f64(sbits))
    assert np.allclose(o[[0, 3]], e2, rtol=0, atol=1e-5)

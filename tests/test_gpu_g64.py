"""GPU parity of the 2-bit G64 expansion and of the GEMV over the expanded
stream, through the C ABI.

The bar: the expansion is bit-exact against the oracle's (every byte); the
GEMV is within |gpu - oracle| <= 1e-3 * sum_j |w_j x'_j| + 1e-5 per output,
exact for integer-valued cases, and bit-identical to the plane GEMV on the
same PQ2_0 data (same pieces, same arithmetic order, same scales).
"""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import codec, projection as P, q2g64
from gpu_util import assert_within, dev, pq2_b1_kernel, say, to_f64, x_dev, x_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FMTS = ["PQ2_0_G128", "PTQ1_0_G128"]


def rand_x(rng, k, xdt):
    x = rng.standard_normal((1, k)).astype(np.float32)
    if xdt == "f32":
        return x
    if xdt == "bf16":
        return synth.f32_to_bf16_bits(x)
    return x.astype(np.float16).view(np.uint16)


def case(fmt, n, k, seed, uniform=False):
    rng = np.random.default_rng(seed)
    trits = synth.trits_uniform(rng, n, k) if uniform else synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    return rng, trits, sb, tq.pack_rowsplit(fmt, trits, sb)


# -------------------------------------------------------------- expansion --
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 128), (3, 1000), (77, 5120), (300, 17408), (2, 384)])
def test_expand_bit_exact(fmt, n, k):
    _, _, _, payload = case(fmt, n, k, seed=n * 7 + k)
    say("expand %s n=%d k=%d" % (fmt, n, k))
    out = tq.expand_g64(dev(torch, payload), fmt, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), q2g64.expand(fmt, n, k, payload))


@pytest.mark.parametrize("fmt", FMTS)
def test_expand_keeps_non_ternary_values(fmt):
    n, k = 40, 1024
    _, _, _, payload = case(fmt, n, k, seed=3)
    payload[0:64] = 0xFF if fmt == "PQ2_0_G128" else 251
    g = tq.geometry(fmt, n, k)
    if fmt == "PTQ1_0_G128":
        payload[g["high_offset"]:g["high_offset"] + 8] = 200
    say("expand non-ternary %s" % fmt)
    out = tq.expand_g64(dev(torch, payload), fmt, n, k).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(out, q2g64.expand(fmt, n, k, payload))
    assert np.array_equal(q2g64.dequantize(out, n, k), P.dequantize(fmt, n, k, payload))


@pytest.mark.parametrize("fmt,n,k", [("PQ2_0_G128", 17408, 5120), ("PTQ1_0_G128", 5120, 17408)])
def test_expand_full_size(fmt, n, k):
    """The decode-step shapes at full size, every byte against the oracle."""
    _, _, _, payload = case(fmt, n, k, seed=11)
    say("expand full %s n=%d k=%d" % (fmt, n, k))
    out = tq.expand_g64(dev(torch, payload), fmt, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), q2g64.expand(fmt, n, k, payload))


# ------------------------------------------------------------------- GEMV --
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 1024), (7, 3072), (1000, 5120), (300, 11264), (5, 13312),
                                 (64, 16384), (33, 17408)])
def test_gemv_g64_parity(fmt, n, k):
    xdt = ["f32", "bf16", "f16"][(n + k // 1024) % 3]
    rng, _, _, payload = case(fmt, n, k, seed=n * 13 + k)
    xr = rand_x(rng, k, xdt)
    say("gemv g64 %s n=%d k=%d x=%s" % (fmt, n, k, xdt))
    blocks = tq.expand_g64(dev(torch, payload), fmt, n, k)
    y = tq.gemv_g64(blocks, n, k, x_dev(torch, xr, xdt))
    torch.cuda.synchronize()
    stream = q2g64.expand(fmt, n, k, payload)
    xf = x_f64(xr, xdt)
    expect = q2g64.project(stream, n, k, xf)
    bound = P.REL * (np.abs(xf) @ np.abs(q2g64.dequantize(stream, n, k)).T) + P.ABS
    assert_within(to_f64(torch, y), expect, bound, "gemv g64")


@pytest.mark.parametrize("n,k", [(40000, 5120), (6000, 17408), (40000, 1024)])
def test_gemv_g64_multi_pass_integer_exact(n, k):
    """Several passes of the persistent grid and a partial last one: scales
    1.0 and integer activations make every partial sum an exact integer."""
    rng = np.random.default_rng(n + k)
    trits = synth.trits_uniform(rng, n, k)
    sb = np.full((n, k // 128), 0x3C00, np.uint16)
    payload = tq.pack_rowsplit("PTQ1_0_G128", trits, sb)
    xi = rng.integers(-8, 9, size=(1, k)).astype(np.float32)
    say("gemv g64 multi-pass n=%d k=%d" % (n, k))
    blocks = tq.expand_g64(dev(torch, payload), "PTQ1_0_G128", n, k)
    y = tq.gemv_g64(blocks, n, k, x_dev(torch, xi, "f32"))
    torch.cuda.synchronize()
    expect = (xi.astype(np.int64) @ trits.T.astype(np.int64)).astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), expect)


@pytest.mark.parametrize("n,k", [(17408, 5120), (1000, 11264), (513, 2048)])
def test_gemv_g64_equals_plane_gemv(n, k):
    """On PQ2_0 data the G64 GEMV and the plane GEMV read the same codes and
    scales.  Where the plane GEMV runs the dot-product kernel both do the
    same arithmetic in the same order and the results are bit-identical;
    where it takes the matrix-core kernel, whose sums are grouped differently,
    both are held to the oracle's bound."""
    rng, _, _, payload = case("PQ2_0_G128", n, k, seed=n + 5 * k)
    xr = rand_x(rng, k, "f16")
    say("gemv g64 vs planes n=%d k=%d" % (n, k))
    pd = dev(torch, payload)
    xd = x_dev(torch, xr, "f16")
    y1 = tq.gemv_g64(tq.expand_g64(pd, "PQ2_0_G128", n, k), n, k, xd)
    y2 = tq.gemv_rowsplit(pd, "PQ2_0_G128", n, k, xd)
    torch.cuda.synchronize()
    if pq2_b1_kernel(n, k) == "dot":
        assert torch.equal(y1, y2)
    else:
        expect, bound = P.project_payload("PQ2_0_G128", n, k, payload, x_f64(xr, "f16"))
        assert_within(to_f64(torch, y1), expect, bound, "g64 n=%d k=%d" % (n, k))
        assert_within(to_f64(torch, y2), expect, bound, "planes n=%d k=%d" % (n, k))


def test_gemv_g64_rejects_batch_above_one():
    n, k = 8, 1024
    blocks = torch.zeros(tq.g64_bytes(n, k), dtype=torch.uint8, device="cuda")
    x = torch.zeros((2, k), dtype=torch.float16, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.gemv_g64(blocks, n, k, x)
    assert e.value.status == 6

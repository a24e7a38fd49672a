"""GPU parity of the transform in the grouped head order, alone and fused
with the decode GEMV (the GatedDeltaNet output projection), through the C ABI.

The bar: the head gather is index work, so the grouped transform equals the
plain transform of the gathered row bit for bit; both are within the
transform tolerance of the float64 oracle; the fused step is bit-identical
to the two launches and within the projection tolerance
|gpu - oracle| <= 1e-3 * sum_j |w_j x'_j| + 1e-5.
"""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import gdn, projection as P, transform as T
from gpu_util import assert_within, dev, say, signs_dev, to_f64, x_dev, x_f64

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


@pytest.mark.parametrize("xdt,ydt", [("f32", "f32"), ("bf16", "f16"), ("f16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("rows,order", [(1, (3, 16, 128)), (5, (3, 16, 128)), (3, (2, 8, 64)),
                                        (2, (4, 4, 192)), (7, (1, 24, 128))])
def test_grouped_transform_parity(xdt, ydt, rows, order):
    tiles, groups, hd = order
    k = tiles * groups * hd
    rng = np.random.default_rng(rows * 7 + k + tiles)
    sbits = synth.sign_bits(rng, k)
    x = rand_x(rng, rows, k, xdt, 2.0)
    say("grouped transform %s->%s rows=%d order=%s" % (xdt, ydt, rows, order))
    xd, sd = x_dev(torch, x, xdt), signs_dev(torch, sbits)
    y = tq.hadamard_signed_grouped(xd, sd, tiles, groups, hd, out_dtype=getattr(torch, TORCH_DT[ydt]))
    # the plain transform of the row gathered on the host side
    src = torch.tensor([gdn.perm_row(j, tiles, groups, hd) for j in range(k)], device="cuda")
    y2 = tq.hadamard_signed(xd[:, src].contiguous(), sd, out_dtype=getattr(torch, TORCH_DT[ydt]))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    xf = x_f64(x, xdt)
    expect = gdn.forward_grouped(xf, T.bf16_bits_to_f64(sbits), tiles, groups, hd)
    bound = 1e-3 * T.block_l1_over_32(gdn.gather(xf, tiles, groups, hd)) + 1e-5 + \
        ROUND[ydt] * np.abs(expect)
    assert_within(to_f64(torch, y), expect, bound, "grouped transform")


def test_grouped_one_tile_is_plain_transform():
    rng = np.random.default_rng(4)
    k = 6144
    sbits = synth.sign_bits(rng, k)
    x = rand_x(rng, 2, k, "bf16")
    xd, sd = x_dev(torch, x, "bf16"), signs_dev(torch, sbits)
    y1 = tq.hadamard_signed_grouped(xd, sd, 1, 48, 128)
    y2 = tq.hadamard_signed(xd, sd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def gdn_case(n, k, seed):
    rng = np.random.default_rng(seed)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = tq.pack_rowsplit("PQ2_0_G128", trits, sb)
    sbits = synth.sign_bits(rng, k)
    x = rand_x(rng, 1, k, "bf16")
    return payload, sbits, x


@pytest.mark.parametrize("n", [1, 333, 5120])
def test_grouped_fused_gemv(n):
    """The GatedDeltaNet output projection step (k = 6144, 48 value heads):
    one launch equals the grouped transform (binary16) then the GEMV, bit
    for bit, and both are within the projection tolerance."""
    k = 6144
    payload, sbits, x = gdn_case(n, k, seed=n + 1)
    say("grouped fused gemv n=%d" % n)
    pd, xd, sd = dev(torch, payload), x_dev(torch, x, "bf16"), signs_dev(torch, sbits)
    y = tq.rotated_gemv_rowsplit_grouped(pd, "PQ2_0_G128", n, k, xd, sd)
    xr = tq.hadamard_signed_grouped(xd, sd, out_dtype=torch.float16)
    y2 = tq.gemv_rowsplit(pd, "PQ2_0_G128", n, k, xr)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    xrot = gdn.forward_grouped(x_f64(x, "bf16"), T.bf16_bits_to_f64(sbits))
    expect, bound = P.project_payload("PQ2_0_G128", n, k, payload, xrot)
    assert_within(to_f64(torch, y), expect, bound, "grouped fused gemv")


def test_grouped_order_matters():
    """The same input without the gather gives a different result (the
    reorder is not the identity on the model's value heads)."""
    n, k = 64, 6144
    payload, sbits, x = gdn_case(n, k, seed=3)
    pd, xd, sd = dev(torch, payload), x_dev(torch, x, "bf16"), signs_dev(torch, sbits)
    y1 = tq.rotated_gemv_rowsplit_grouped(pd, "PQ2_0_G128", n, k, xd, sd)
    y2 = tq.rotated_gemv_rowsplit(pd, "PQ2_0_G128", n, k, xd, sd)
    torch.cuda.synchronize()
    assert not torch.allclose(y1, y2)

"""GPU parity with leading dimensions wider than the rows: activations read
through ldx > k, outputs written through ldy > n (GEMV at batch 1-8, both
formats, every kernel that serves them: the batch-1 wave kernel, the row-quad
kernel and the team kernel for rows beyond the others' reach), the prefill
GEMM with ldx > k and ldy > n for both output types, and the embedding with
ldo > k.  The columns between the row width and the leading dimension must be
left untouched.

Tolerance: the stated per-output bound 1e-3 * sum_j |w_j x'_j| + 1e-5 against
the float64 oracle (plus bf16 rounding of the GEMM's bf16 output, and the
block-L1 bound of the transform for the embedding rows)."""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import projection as P, transform as T
from gpu_util import assert_within, dev, say, signs_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SENTINEL = -12288.0  # exact in bf16, binary16 and fp32


def padded(shape, width, dtype, fill):
    """A [rows, width] buffer filled with `fill`; returns it and the
    [rows, shape[1]] view of its leading columns."""
    buf = torch.full((shape[0], width), fill, dtype=dtype, device="cuda")
    return buf, buf[:, :shape[1]]


def workload(fmt, n, k, seed):
    rng = np.random.default_rng(seed)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    return rng, tq.pack_rowsplit(fmt, trits, sb)


@pytest.mark.parametrize("fmt,n,k,batch", [
    ("PQ2_0_G128", 1000, 5120, 1),      # batch-1 wave kernel
    ("PQ2_0_G128", 777, 5120, 3),       # row-quad kernel
    ("PTQ1_0_G128", 640, 17408, 8),     # row-quad kernel, PTQ1_0
    ("PTQ1_0_G128", 300, 2048, 1),
    ("PQ2_0_G128", 130, 32768, 2),      # team kernel (rows beyond the row-quad kernel)
    ("PTQ1_0_G128", 96, 32768, 5),
])
def test_gemv_strided(fmt, n, k, batch):
    rng, payload = workload(fmt, n, k, n + k + batch)
    xr = (rng.standard_normal((batch, k))).astype(np.float16)
    ldx, ldy = k + 64, n + 5
    say("gemv strided %s n=%d k=%d batch=%d ldx=%d ldy=%d" % (fmt, n, k, batch, ldx, ldy))
    xbuf, xv = padded((batch, k), ldx, torch.float16, float("nan"))
    xv.copy_(torch.from_numpy(xr))
    ybuf, yv = padded((batch, n), ldy, torch.float32, SENTINEL)
    assert xv.stride(0) == ldx and yv.stride(0) == ldy
    tq.gemv_rowsplit(dev(torch, payload), fmt, n, k, xv, out=yv)
    torch.cuda.synchronize()
    y = ybuf.cpu().numpy()
    assert np.all(y[:, n:] == SENTINEL), "columns past n were written"
    expect, bound = P.project_payload(fmt, n, k, payload, xr.astype(np.float64))
    assert_within(y[:, :n].astype(np.float64), expect, bound, "gemv strided")


@pytest.mark.parametrize("fmt,ydt", [("PQ2_0_G128", torch.float32), ("PTQ1_0_G128", torch.bfloat16)])
def test_gemm_strided(fmt, ydt):
    n, k, m = 520, 3072, 300
    rng, payload = workload(fmt, n, k, 77 if ydt == torch.float32 else 78)
    xr = rng.standard_normal((m, k)).astype(np.float16)
    ldx, ldy = k + 8, n + 24
    say("gemm strided %s m=%d n=%d k=%d ldx=%d ldy=%d out=%s" % (fmt, m, n, k, ldx, ldy, ydt))
    xbuf, xv = padded((m, k), ldx, torch.float16, float("nan"))
    xv.copy_(torch.from_numpy(xr))
    ybuf, yv = padded((m, n), ldy, ydt, SENTINEL)
    tq.gemm_rowsplit(dev(torch, payload), fmt, n, k, xv, out_dtype=ydt, out=yv)
    torch.cuda.synchronize()
    y = ybuf.float().cpu().numpy().astype(np.float64)
    assert np.all(y[:, n:] == SENTINEL), "columns past n were written"
    expect, bound = P.project_payload(fmt, n, k, payload, xr.astype(np.float64))
    if ydt == torch.bfloat16:
        bound = bound + 2.0 ** -8 * np.abs(expect)
    assert_within(y[:, :n], expect, bound, "gemm strided")


def test_embed_strided():
    fmt, n, k = "PQ2_0_G128", 4096, 5120
    rng, payload = workload(fmt, n, k, 91)
    sbits = synth.sign_bits(rng, k)
    ids = synth.token_ids(rng, 40, n)
    ldo = k + 48
    say("embed strided n=%d k=%d ldo=%d" % (n, k, ldo))
    obuf, ov = padded((ids.size, k), ldo, torch.float32, SENTINEL)
    tq.embed_rows_inverse(dev(torch, payload), fmt, n, k, dev(torch, ids), signs_dev(torch, sbits),
                          out=ov)
    torch.cuda.synchronize()
    o = obuf.cpu().numpy()
    assert np.all(o[:, k:] == SENTINEL), "columns past k were written"
    expect, l1 = P.embed_rows_inverse(fmt, n, k, payload, ids, T.bf16_bits_to_f64(sbits))
    assert_within(o[:, :k].astype(np.float64), expect, 1e-3 * l1 + 1e-5, "embed strided")

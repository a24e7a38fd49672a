"""GPU parity of the batch-1 matrix-core GEMV at the edges of the shapes it
takes: the smallest and largest row lengths (k = 1024, 2048 and 6144), a
matrix just above its 2^29-weight threshold, and a row count that leaves the
last 32-row block partly empty.

Each payload repeats a few hundred rows of the six hard kinds of
test_gpu_numerics (all-zero rows at unit and large scales, sparse rows,
single weights on the smallest activations), cyclically, to n rows: row r is
base row r % N0.  Every output is held to the stated bound
    |gpu - oracle| <= 1e-3 * sum_j |w_j x'_j| + 1e-5
against the oracle's projection of the base rows, through the GEMV on a
rotated input, the one-launch decode step and the one-launch output head;
all-zero rows must come out exactly 0.
"""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import head as Hd, projection as P, transform as T
from gpu_util import assert_within, dev, say, signs_dev, x_dev, x_f64
from test_gpu_numerics import activation, hard_rows, row2d

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FMT = "PQ2_0_G128"
N0 = 600
THRESHOLD = 1 << 29

# (k, extra rows past the threshold): each n is above 2^29 / k and not a
# multiple of 32
SHAPES = [(1024, 11), (2048, 19), (6144, 5)]


def shape_rows(k, extra):
    return -(-THRESHOLD // k) + extra


def cyclic_payload(n0, n, k, payload):
    """The payload of n rows whose row r is row r % n0 of the given n0-row
    payload, plane by plane."""
    gs, gb = tq.geometry(FMT, n0, k), tq.geometry(FMT, n, k)
    big = np.zeros(gb["payload_bytes"], np.uint8)
    reps = -(-n // n0)
    for plane in ("base", "high", "scale"):
        nb = gs[plane + "_bytes"]
        if not nb:
            continue
        per_row = nb // n0
        src = payload[gs[plane + "_offset"]:gs[plane + "_offset"] + nb]
        big[gb[plane + "_offset"]:gb[plane + "_offset"] + per_row * n] = np.tile(src, reps)[:per_row * n]
    return big


def check_cyclic(got, expect, bound, zero_rows, what):
    n = got.size
    idx = np.arange(n) % N0
    err = np.abs(got - expect[idx]) / bound[idx]
    worst = int(np.argmax(err))
    assert float(err[worst]) <= 1.0, "%s: row %d |err|/bound %r (got %r, oracle %r)" % (
        what, worst, float(err[worst]), float(got[worst]), float(expect[idx[worst]]))
    z = got[np.isin(idx, zero_rows)]
    assert np.all(z == 0.0), "%s: all-zero rows must give exactly 0" % what
    # the last, partial block and the first block, row by row
    assert_within(got[-N0:], expect[idx[-N0:]], bound[idx[-N0:]], what + " last rows")
    assert_within(got[:N0], expect, bound, what + " first rows")


def test_shapes_are_above_the_threshold_and_ragged():
    for k, extra in SHAPES:
        n = shape_rows(k, extra)
        assert n * k >= THRESHOLD and (n - 1) * k < THRESHOLD + extra * k
        assert n % 32 != 0


@pytest.mark.parametrize("k,extra", SHAPES)
def test_f4_gemv_shapes(k, extra):
    n = shape_rows(k, extra)
    rng = np.random.default_rng(k + extra)
    xrot = activation(rng, k, "mixed" if k >= 2048 else "normal").astype(np.float16)
    xrot64 = xrot.astype(np.float64)
    trits, sb, zero_rows = hard_rows(rng, N0, k, xrot64)
    base = tq.pack_rowsplit(FMT, trits, sb)
    say("f4 gemv n=%d k=%d" % (n, k))
    y = tq.gemv_rowsplit(dev(torch, cyclic_payload(N0, n, k, base)), FMT, n, k, dev(torch, row2d(xrot)))
    torch.cuda.synchronize()
    expect, bound = P.project_payload(FMT, N0, k, base, xrot64[None, :])
    check_cyclic(y.cpu().numpy()[0].astype(np.float64), expect[0], bound[0], zero_rows,
                 "gemv n=%d k=%d" % (n, k))


@pytest.mark.parametrize("k,extra", SHAPES)
def test_f4_rotated_gemv_shapes(k, extra):
    n = shape_rows(k, extra)
    rng = np.random.default_rng(2 * k + extra)
    xb = synth.f32_to_bf16_bits(row2d(activation(rng, k, "small")))
    sbits = synth.sign_bits(rng, k)
    xrot64 = T.forward(x_f64(xb, "bf16"), T.bf16_bits_to_f64(sbits))
    trits, sb, zero_rows = hard_rows(rng, N0, k, xrot64[0])
    base = tq.pack_rowsplit(FMT, trits, sb)
    say("f4 rotated gemv n=%d k=%d" % (n, k))
    y = tq.rotated_gemv_rowsplit(dev(torch, cyclic_payload(N0, n, k, base)), FMT, n, k,
                                 x_dev(torch, xb, "bf16"), signs_dev(torch, sbits))
    torch.cuda.synchronize()
    expect, bound = P.project_payload(FMT, N0, k, base, xrot64)
    check_cyclic(y.cpu().numpy()[0].astype(np.float64), expect[0], bound[0], zero_rows,
                 "rotated n=%d k=%d" % (n, k))


@pytest.mark.parametrize("k,extra", SHAPES)
def test_f4_head_shapes(k, extra):
    n = shape_rows(k, extra)
    rng = np.random.default_rng(3 * k + extra)
    xb = synth.f32_to_bf16_bits(row2d(activation(rng, k, "normal")))
    sbits = synth.sign_bits(rng, k)
    gbits = synth.norm_weight_bits(rng, k)
    eps = 1e-6
    xrot64 = T.forward(Hd.rmsnorm(x_f64(xb, "bf16"), T.bf16_bits_to_f64(gbits), eps),
                       T.bf16_bits_to_f64(sbits))
    trits, sb, zero_rows = hard_rows(rng, N0, k, xrot64[0])
    base = tq.pack_rowsplit(FMT, trits, sb)
    say("f4 head n=%d k=%d" % (n, k))
    work = torch.zeros(2, dtype=torch.int64, device="cuda")
    logits = torch.empty(n, dtype=torch.float32, device="cuda")
    gd = dev(torch, gbits.view(np.int16)).view(torch.bfloat16)
    tok = tq.head_argmax(dev(torch, cyclic_payload(N0, n, k, base)), FMT, n, k, x_dev(torch, xb, "bf16"),
                         gd, eps, signs_dev(torch, sbits), work, logits=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy().astype(np.float64)
    logits_o, bound, _ = Hd.head(FMT, N0, k, base, x_f64(xb, "bf16"), T.bf16_bits_to_f64(gbits), eps,
                                 T.bf16_bits_to_f64(sbits))
    check_cyclic(lg, logits_o[0], bound[0], zero_rows, "head n=%d k=%d" % (n, k))
    # the token is the first row holding the largest logit
    assert int(tok.item()) == int(np.flatnonzero(lg == lg.max())[0])
    assert np.all(work.cpu().numpy() == 0)

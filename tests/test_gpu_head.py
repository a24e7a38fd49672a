"""GPU parity of the one-launch output head (RMSNorm, signed transform, head
GEMV, greedy token), through the C ABI.

The bar: every logit within |gpu - oracle| <= 1e-3 * sum_j |w_j x'_j| + 1e-5
against the float64 oracle.  The token is a decision taken on the kernel's fp32 logits,
so it must be exactly the lowest index of their maximum; it must also be a
valid choice for the oracle (its logit within the bounds of the oracle's
maximum), and the oracle's own choice wherever the oracle's top two logits
are further apart than the bounds.
"""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import codec, head as Hd, projection as P, transform as T
from gpu_util import assert_within, dev, say, signs_dev, x_dev, x_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FMT = "PQ2_0_G128"


def rand_x(rng, k, xdt, scale=3.0):
    x = (rng.standard_normal((1, k)) * scale).astype(np.float32)
    if xdt == "f32":
        return x
    if xdt == "bf16":
        return synth.f32_to_bf16_bits(x)
    return x.astype(np.float16).view(np.uint16)


def bits_dev(bits):
    return dev(torch, np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def run_head(payload_d, n, k, x, xdt, gbits, eps, sbits, want_logits=True):
    work = torch.zeros(2, dtype=torch.int64, device="cuda")
    logits = torch.empty(n, dtype=torch.float32, device="cuda") if want_logits else None
    tok = tq.head_argmax(payload_d, FMT, n, k, x_dev(torch, x, xdt), bits_dev(gbits), eps,
                         signs_dev(torch, sbits), work, logits=logits)
    torch.cuda.synchronize()
    assert not work.any(), "work words must be left zero"
    lg = None if logits is None else logits.cpu().numpy().astype(np.float64)
    return int(tok.item()), lg


def check(payload, n, k, x, xdt, gbits, eps, sbits, tok, lg):
    logits_o, bound, xrot = Hd.head(FMT, n, k, payload, x_f64(x, xdt), T.bf16_bits_to_f64(gbits),
                                    eps, T.bf16_bits_to_f64(sbits))
    lo = logits_o[0]
    b = bound[0]
    assert_within(lg, lo, b, "head logits")
    # the decision on the kernel's own logits: lowest index of their maximum
    assert tok == int(np.flatnonzero(lg == lg.max())[0])
    # a valid choice for the oracle
    io = int(Hd.greedy(lo)[0])
    assert lo[tok] >= lo[io] - (b[tok] + b[io])
    top2 = np.sort(lo)[-2:]
    if n == 1 or top2[1] - top2[0] > 2 * b.max():
        assert tok == io
    return io


@pytest.mark.parametrize("n,k,xdt", [(1000, 5120, "bf16"), (3001, 1024, "f32"), (77, 11264, "f16"),
                                     (1, 2048, "bf16"), (40000, 3072, "bf16")])
def test_head_parity(n, k, xdt):
    rng = np.random.default_rng(n + k)
    trits = synth.trits_uniform(rng, n, k)
    sb = synth.scale_bits_uniform(rng, n, synth.groups_of(k), 0.01, 0.04)
    payload = tq.pack_rowsplit(FMT, trits, sb)
    sbits = synth.sign_bits(rng, k)
    gbits = synth.norm_weight_bits(rng, k)
    x = rand_x(rng, k, xdt)
    say("head n=%d k=%d x=%s" % (n, k, xdt))
    pd = dev(torch, payload)
    tok, lg = run_head(pd, n, k, x, xdt, gbits, 1e-6, sbits)
    check(payload, n, k, x, xdt, gbits, 1e-6, sbits, tok, lg)
    # without the logits buffer: the same token
    tok2, _ = run_head(pd, n, k, x, xdt, gbits, 1e-6, sbits, want_logits=False)
    assert tok2 == tok


def test_head_full_vocabulary():
    """The 248320 x 5120 head at full size with a bf16 hidden row."""
    c = synth.make_config(4)
    n, k = c["n"], c["k"]
    payload = tq.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
    del c["trits"]
    gbits = synth.norm_weight_bits(np.random.default_rng(44), k)
    say("head full n=%d k=%d" % (n, k))
    tok, lg = run_head(dev(torch, payload), n, k, c["x"], "bf16", gbits, 1e-6, c["sign_bits"])
    check(payload, n, k, c["x"], "bf16", gbits, 1e-6, c["sign_bits"], tok, lg)


def single_trit_head(n, k, cols, scale_bits_row):
    trits = np.zeros((n, k), np.int8)
    trits[np.arange(n), cols] = 1
    sb = np.repeat(np.asarray(scale_bits_row, np.uint16)[:, None], k // 128, axis=1)
    return tq.pack_rowsplit(FMT, trits, sb)


@pytest.mark.parametrize("dups", [(5, 17, 4000), (0, 1), (4095, 4094, 2)])
def test_head_ties_take_lowest_index(dups):
    """Rows with equal data give bitwise-equal logits; when they carry the
    maximum, the lowest of them is the token."""
    rng = np.random.default_rng(sum(dups))
    n, k = 4096, 2048
    z = rng.standard_normal((1, k))
    c_star = int(np.argmax(z))
    z[0, c_star] += 1.0                          # a clear maximum of x'
    cols = rng.integers(0, k, n)
    cols[cols == c_star] = (c_star + 1) % k
    cols[list(dups)] = c_star
    payload = single_trit_head(n, k, cols, np.full(n, 0x3C00, np.uint16))
    sbits = synth.sign_bits(rng, k)
    x = T.inverse(z, T.bf16_bits_to_f64(sbits)).astype(np.float32)
    gbits = np.full(k, 0x3F80, np.uint16)        # weight 1.0
    say("head ties %s" % (dups,))
    tok, lg = run_head(dev(torch, payload), n, k, x, "f32", gbits, 0.0, sbits)
    assert tok == min(dups)
    assert len(set(lg[list(dups)])) == 1


def test_head_negative_and_zero_logits():
    rng = np.random.default_rng(8)
    n, k = 999, 1024
    sbits = synth.sign_bits(rng, k)
    gbits = synth.norm_weight_bits(rng, k)
    x = rand_x(rng, k, "bf16")
    # all logits negative: scales negative on single-trit rows (-0.02, in
    # the range of the workloads' scales)
    cols = rng.integers(0, k, n)
    neg = single_trit_head(n, k, cols, np.full(n, 0xA51F, np.uint16))   # -0.02
    say("head negative logits")
    tok, lg = run_head(dev(torch, neg), n, k, x, "bf16", gbits, 1e-6, sbits)
    check(neg, n, k, x, "bf16", gbits, 1e-6, sbits, tok, lg)
    # a zero hidden row (eps > 0): x' = 0, every logit is exactly zero and
    # the token is row 0
    trits = synth.trits_uniform(rng, n, k)
    pos = tq.pack_rowsplit(FMT, trits, synth.scale_bits_uniform(rng, n, k // 128, 0.01, 0.04))
    zx = np.zeros((1, k), np.uint16)
    tok, lg = run_head(dev(torch, pos), n, k, zx, "bf16", gbits, 1e-6, sbits)
    assert tok == 0 and not np.any(lg)


def test_head_repeated_calls_share_work():
    """Two calls in a row on one work buffer (left zero by the first) and a
    third on a different hidden row give each its own token."""
    rng = np.random.default_rng(12)
    n, k = 20000, 5120
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = tq.pack_rowsplit(FMT, trits, sb)
    pd = dev(torch, payload)
    sbits = synth.sign_bits(rng, k)
    gbits = synth.norm_weight_bits(rng, k)
    sd, gd = signs_dev(torch, sbits), bits_dev(gbits)
    work = torch.zeros(2, dtype=torch.int64, device="cuda")
    xs = [rand_x(rng, k, "bf16") for _ in range(3)]
    toks, lgs = [], []
    for x in (xs[0], xs[0], xs[1], xs[2]):
        lg = torch.empty(n, dtype=torch.float32, device="cuda")
        toks.append(tq.head_argmax(pd, FMT, n, k, x_dev(torch, x, "bf16"), gd, 1e-6, sd, work,
                                   logits=lg))
        lgs.append(lg)
    torch.cuda.synchronize()
    assert not work.any()
    got = [int(t.item()) for t in toks]
    assert got[0] == got[1]
    for t, lg in zip(got, lgs):
        l = lg.cpu().numpy()
        assert t == int(np.flatnonzero(l == l.max())[0])
    check(payload, n, k, xs[2], "bf16", gbits, 1e-6, sbits, got[3], lgs[3].cpu().numpy().astype(np.float64))


def test_head_rejects_uncovered_requests():
    n, k = 16, 1024
    g = tq.geometry("PTQ1_0_G128", n, k)
    pd = torch.zeros(g["payload_bytes"], dtype=torch.uint8, device="cuda")
    x = torch.zeros(k, dtype=torch.bfloat16, device="cuda")
    work = torch.zeros(2, dtype=torch.int64, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.head_argmax(pd, "PTQ1_0_G128", n, k, x, x, 1e-6, x, work)
    assert e.value.status == 6


def test_head_nan_logits_are_never_chosen():
    """Rows whose logit is NaN (planted through a NaN group scale, outside the
    formats' finite scales, only to make NaN logits) are never the token, even
    where the row would otherwise hold the maximum; a hidden row with a NaN
    makes every logit NaN, and the token is then -1."""
    rng = np.random.default_rng(31)
    n, k = 3000, 2048
    z = rng.standard_normal((1, k))
    c_star = int(np.argmax(z))
    z[0, c_star] += 1.0
    cols = rng.integers(0, k, n)
    cols[cols == c_star] = (c_star + 1) % k
    winners = [7, 1500]                      # would tie for the maximum
    cols[winners] = c_star
    sb = np.full(n, 0x3C00, np.uint16)
    sb[7] = 0x7E00                           # NaN scale: row 7's logit is NaN
    sb[[0, 2999]] = 0x7E00
    payload = single_trit_head(n, k, cols, sb)
    sbits = synth.sign_bits(rng, k)
    x = T.inverse(z, T.bf16_bits_to_f64(sbits)).astype(np.float32)
    gbits = np.full(k, 0x3F80, np.uint16)
    say("head NaN logits")
    pd = dev(torch, payload)
    tok, lg = run_head(pd, n, k, x, "f32", gbits, 0.0, sbits)
    assert np.isnan(lg[[0, 7, 2999]]).all() and not np.isnan(np.delete(lg, [0, 7, 2999])).any()
    assert tok == 1500
    lo, bound, _ = Hd.head(FMT, n, k, payload, x_f64(x, "f32"), T.bf16_bits_to_f64(gbits), 0.0,
                           T.bf16_bits_to_f64(sbits))
    assert int(Hd.greedy(lo)[0]) == 1500
    ok = ~np.isnan(lo[0])
    assert_within(lg[ok], lo[0][ok], bound[0][ok], "head logits beside NaN rows")
    # a NaN in the hidden row: every logit NaN, no token
    xn = x.copy()
    xn[0, 5] = np.nan
    tok, lg = run_head(pd, n, k, xn, "f32", gbits, 0.0, sbits)
    assert np.isnan(lg).all() and tok == -1

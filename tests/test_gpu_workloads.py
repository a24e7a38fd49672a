"""The five workloads end to end at full size, through the C ABI, in the
launch configuration bench.py times: bf16 (or fp32) activations -> signed
transform (binary16 out) -> GEMV / GEMM, and the embedding gather.

Every output is compared with the float64 oracle where the oracle finishes in
seconds (configs 1-3 and the embedding); the 248320-row head and the
2048-row prefill compare sampled outputs the oracle computes one by one.
Bound per output: 1e-3 * sum_j |w_j x'_j| + 1e-5 with x' the oracle's
float64 transform.
"""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import projection as P, transform as T
from gpu_util import assert_within, dev, say, signs_dev, to_f64, x_dev, x_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def rotate_and_project(c, rows=None):
    fmt, n, k = c["fmt"], c["n"], c["k"]
    payload = tq.pack_rowsplit(fmt, c["trits"], c["scale_bits"])
    x = c["x"] if rows is None else c["x"][:rows]
    xd = x_dev(torch, x, c["x_dtype"])
    sd = signs_dev(torch, c["sign_bits"])
    xr = tq.hadamard_signed(xd, sd, out_dtype=torch.float16)
    pd = dev(torch, payload)
    return payload, pd, xr, x


@pytest.mark.parametrize("cfg", [1, 2])
def test_config_gemv_full(cfg):
    c = synth.make_config(cfg)
    say("config %d: %s n=%d k=%d" % (cfg, c["fmt"], c["n"], c["k"]))
    payload, pd, xr, x = rotate_and_project(c)
    y = tq.gemv_rowsplit(pd, c["fmt"], c["n"], c["k"], xr)
    y2 = tq.gemv_rowsplit(pd, c["fmt"], c["n"], c["k"], xr)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    # the one-launch decode step gives the same bits as the two launches
    xd = x_dev(torch, x, c["x_dtype"])
    yf = tq.rotated_gemv_rowsplit(pd, c["fmt"], c["n"], c["k"], xd, signs_dev(torch, c["sign_bits"]))
    torch.cuda.synchronize()
    assert torch.equal(yf, y)
    xr64 = T.forward(x_f64(x, c["x_dtype"]), T.bf16_bits_to_f64(c["sign_bits"]))
    expect, bound = P.project_payload(c["fmt"], c["n"], c["k"], payload, xr64)
    assert_within(to_f64(torch, y), expect, bound, "config %d" % cfg)


def test_config3_down_projection_batches():
    c = synth.make_config(3)
    payload, pd, xr, x = rotate_and_project(c)
    xr64 = T.forward(x_f64(x, "bf16"), T.bf16_bits_to_f64(c["sign_bits"]))
    expect, bound = P.project_payload(c["fmt"], c["n"], c["k"], payload, xr64)
    for b in (1, 4, 8):
        say("config 3: PTQ1_0 5120x17408 batch %d" % b)
        y = tq.gemv_rowsplit(pd, c["fmt"], c["n"], c["k"], xr[:b].contiguous())
        torch.cuda.synchronize()
        assert_within(to_f64(torch, y), expect[:b], bound[:b], "config 3 batch %d" % b)


def test_config4_head_and_embedding():
    c = synth.make_config(4)
    fmt, n, k = c["fmt"], c["n"], c["k"]
    say("config 4: head %s n=%d k=%d" % (fmt, n, k))
    payload, pd, xr, x = rotate_and_project(c)
    y = tq.gemv_rowsplit(pd, fmt, n, k, xr)
    sd = signs_dev(torch, c["sign_bits"])
    ids = c["ids"]
    emb = tq.embed_rows_inverse(pd, fmt, n, k, dev(torch, ids), sd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.integers(0, n, 3000)]))
    xr64 = T.forward(x_f64(x, "bf16"), T.bf16_bits_to_f64(c["sign_bits"]))
    expect, bound = P.project_payload(fmt, n, k, payload, xr64, rows=rows)
    assert_within(to_f64(torch, y)[:, rows], expect, bound, "config 4 head (sampled)")
    e_exp, e_scale = P.embed_rows_inverse(fmt, n, k, payload, ids, T.bf16_bits_to_f64(c["sign_bits"]))
    assert_within(to_f64(torch, emb), e_exp, 1e-3 * e_scale + 1e-5, "config 4 embedding")


def test_config5_prefill_gemm():
    c = synth.make_config(5)
    fmt, n, k = c["fmt"], c["n"], c["k"]
    say("config 5: prefill %d x %d x %d" % (c["x"].shape[0], n, k))
    payload, pd, xr, x = rotate_and_project(c)
    y = tq.gemm_rowsplit(pd, fmt, n, k, xr)
    torch.cuda.synchronize()
    m = x.shape[0]
    rows = np.array([0, 1, 2, 3, 4, 5, 6, 7, 127, 128, 1000, m - 1])
    xr64 = T.forward(x_f64(x[rows], "bf16"), T.bf16_bits_to_f64(c["sign_bits"]))
    expect, bound = P.project_payload(fmt, n, k, payload, xr64)
    got = to_f64(torch, y[torch.as_tensor(rows, device=y.device)])
    assert_within(got, expect, bound, "config 5 prefill (12 rows x all columns)")
    # the GEMV on the same rotated rows meets the same bound
    yv = tq.gemv_rowsplit(pd, fmt, n, k, xr[:8].contiguous())
    torch.cuda.synchronize()
    assert_within(to_f64(torch, yv), expect[:8], bound[:8], "config 5 rows via GEMV")

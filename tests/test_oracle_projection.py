"""Oracle projection pinned to brute force, closed forms and invariants."""

import numpy as np
import pytest

from oracle import codec, projection as P, transform as T
import synth


def make(fmt, n, k, seed, scale_const=None):
    rng = np.random.default_rng(seed)
    trits = synth.trits_sparse(rng, n, k)
    g = synth.groups_of(k)
    sb = synth.scale_bits_lognormal(rng, n, g)
    if scale_const is not None:
        sb[:] = scale_const
    return trits, sb, codec.pack_rowsplit(fmt, trits, sb)


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
@pytest.mark.parametrize("n,k,b", [(6, 1024, 1), (3, 2048, 2), (4, 1000, 1)])
def test_scalar_loop_equals_dense(fmt, n, k, b):
    trits, sb, payload = make(fmt, n, k, n + k)
    rng = np.random.default_rng(9)
    xrot = rng.standard_normal((b, k))
    y_loop = P.project_scalar(fmt, n, k, payload, xrot)
    y_dense, _ = P.project_payload(fmt, n, k, payload, xrot, chunk=2)
    np.testing.assert_allclose(y_loop, y_dense, rtol=1e-12, atol=1e-14)
    # dequantising the payload equals dequantising the generated trits
    w = P.dequantize(fmt, n, k, payload)[:, :k]
    assert np.array_equal(w, P.dequantize_trits(trits, sb))


def test_integer_brute_force():
    # Tiny integer case computed with Python integers: scale 1.0 (0x3C00),
    # x' integers, so the float64 result is exact.
    rng = np.random.default_rng(11)
    n, k = 5, 256
    trits = synth.trits_uniform(rng, n, k)
    sb = np.full((n, 2), 0x3C00, np.uint16)
    payload = codec.pack_rowsplit("PQ2_0_G128", trits, sb)
    xi = rng.integers(-8, 9, size=k)
    expect = [sum(int(trits[r, j]) * int(xi[j]) for j in range(k)) for r in range(n)]
    y, _ = P.project_payload("PQ2_0_G128", n, k, payload, xi[None, :].astype(float))
    assert y[0].tolist() == [float(e) for e in expect]


def test_closed_form_all_plus_one():
    # All trits +1 and scale 1: y_n = sum_j x'_j = 32 * sum_b d_{1024b} x_{1024b}
    # because the all-ones row of H sums each column to 1024 * e_0.
    n, k = 4, 3072
    trits = np.ones((n, k), np.int8)
    sb = np.full((n, k // 128), 0x3C00, np.uint16)
    payload = codec.pack_rowsplit("PQ2_0_G128", trits, sb)
    rng = np.random.default_rng(5)
    d = rng.integers(0, 2, size=k) * 2.0 - 1.0
    x = rng.standard_normal((1, k))
    y, _ = P.projection("PQ2_0_G128", n, k, payload, x, d)
    expect = 32.0 * sum(d[b] * x[0, b] for b in range(0, k, 1024))
    np.testing.assert_allclose(y[0], np.full(n, expect), rtol=1e-12)


def test_zero_cases():
    n, k = 3, 1024
    payload = codec.pack_rowsplit("PTQ1_0_G128", np.zeros((n, k), np.int8),
                                  np.full((n, 8), 0x3C00, np.uint16))
    y, bnd = P.projection("PTQ1_0_G128", n, k, payload,
                          np.random.default_rng(0).standard_normal((2, k)), np.ones(k))
    assert not y.any() and np.all(bnd == P.ABS)
    _, _, payload = make("PQ2_0_G128", n, k, 1)
    y, _ = P.projection("PQ2_0_G128", n, k, payload, np.zeros((1, k)), np.ones(k))
    assert not y.any()


def test_association_with_dense_rotation():
    # (W . blockdiag(H D)/32) x == W . (H(D x)/32)
    n, k = 5, 2048
    _, _, payload = make("PQ2_0_G128", n, k, 3)
    rng = np.random.default_rng(4)
    d = rng.integers(0, 2, size=k) * 2.0 - 1.0
    x = rng.standard_normal((2, k))
    w = P.dequantize("PQ2_0_G128", n, k, payload)
    h = T.hadamard_1024()
    wr = np.zeros_like(w)
    for b in range(0, k, 1024):
        wr[:, b:b + 1024] = (w[:, b:b + 1024] @ h) * d[b:b + 1024] / 32.0
    y_assoc = x @ wr.T
    y, _ = P.projection("PQ2_0_G128", n, k, payload, x, d)
    np.testing.assert_allclose(y, y_assoc, rtol=1e-11, atol=1e-13)


def test_embedding_inverse_properties():
    n, k = 40, 2048
    trits, sb, payload = make("PQ2_0_G128", n, k, 8)
    rng = np.random.default_rng(8)
    d = rng.integers(0, 2, size=k) * 2.0 - 1.0
    ids = np.array([0, 39, 7, 7, 21])
    out, scale = P.embed_rows_inverse("PQ2_0_G128", n, k, payload, ids, d)
    # the forward transform undoes the inverse: back to the dequantised rows
    w = P.dequantize_trits(trits, sb)[ids]
    np.testing.assert_allclose(T.forward(out, d), w, rtol=0, atol=1e-14)
    assert np.array_equal(out[2], out[3])
    # one +1 trit at a block start with scale s gives s * d_block / 32
    one = np.zeros((1, k), np.int8)
    one[0, 1024] = 1
    s_bits = np.full((1, k // 128), 0x3800, np.uint16)   # 0.5
    p1 = codec.pack_rowsplit("PQ2_0_G128", one, s_bits)
    o1, _ = P.embed_rows_inverse("PQ2_0_G128", 1, k, p1, [0], d)
    assert not o1[0, :1024].any()
    assert np.array_equal(o1[0, 1024:], 0.5 * d[1024:] / 32.0)
    with pytest.raises(IndexError):
        P.embed_rows_inverse("PQ2_0_G128", n, k, payload, [n], d)


def test_bound_shape():
    w = np.array([[1.0, -2.0], [0.0, 0.0]])
    x = np.array([[3.0, 1.0]])
    b = P.bound(w, x)
    np.testing.assert_allclose(b, [[1e-3 * 5.0 + 1e-5, 1e-5]])


def test_synth_value_recipes():
    # The generators draw what the workloads state: sparse trits with
    # P(0) = 0.4, lognormal(-4, 0.5) scales, +-1 bf16 signs, N(0,1) bf16 x.
    c = synth.make_config(2, n=512, k=5120, rows=4)
    t = c["trits"]
    assert abs((t == 0).mean() - 0.4) < 0.01 and abs((t == 1).mean() - 0.3) < 0.01
    s = T.fp16_bits_to_f64(c["scale_bits"])
    assert abs(np.median(s) - np.exp(-4.0)) < 0.002
    assert set(np.unique(c["sign_bits"]).tolist()) == {0x3F80, 0xBF80}
    x = T.bf16_bits_to_f64(c["x"])
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05
    c1 = synth.make_config(1)
    s1 = T.fp16_bits_to_f64(c1["scale_bits"])
    assert s1.min() >= 0.0049 and s1.max() <= 0.0501

"""Oracle transform pinned to textbook/library Hadamard facts and closed forms."""

import numpy as np
import pytest
import scipy.linalg

from oracle import transform as T


def popcount_sign(i, j):
    return -1.0 if bin(i & j).count("1") % 2 else 1.0


def test_sylvester_small_textbook():
    h4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    assert np.array_equal(T.sylvester_hadamard(4), h4)


def test_matches_scipy_and_popcount_closed_form():
    h = T.hadamard_1024()
    assert np.array_equal(h, scipy.linalg.hadamard(1024).astype(np.float64))
    idx = np.arange(1024)
    parity = np.array([bin(v).count("1") & 1 for v in range(1024)])
    closed = 1.0 - 2.0 * parity[idx[:, None] & idx[None, :]]
    assert np.array_equal(h, closed)


def test_orthogonal_and_symmetric():
    h = T.hadamard_1024()
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h, 1024.0 * np.eye(1024))


def rand_signs(rng, k):
    return rng.integers(0, 2, size=k) * 2.0 - 1.0


def test_basis_vectors_forward_and_inverse():
    # forward(e_i)[r] = d_i (-1)^popcount(r&i) / 32 (D then H);
    # inverse(e_i)[r] = d_r (-1)^popcount(r&i) / 32 (H then D).
    rng = np.random.default_rng(0)
    d = rand_signs(rng, 1024)
    for i in [0, 1, 2, 3, 5, 64, 511, 1023]:
        e = np.zeros((1, 1024))
        e[0, i] = 1.0
        f = T.forward(e, d)[0]
        v = T.inverse(e, d)[0]
        for r in [0, 1, 7, 100, 777, 1023]:
            assert f[r] == d[i] * popcount_sign(r, i) / 32.0
            assert v[r] == d[r] * popcount_sign(r, i) / 32.0


def test_e0_constant_one_over_sqrt_block():
    # With D = I both transforms map e_0 to the constant vector 1/32.
    e = np.zeros((1, 1024))
    e[0, 0] = 1.0
    ones = np.ones(1024)
    assert np.array_equal(T.forward(e, ones)[0], np.full(1024, 1 / 32))
    assert np.array_equal(T.inverse(e, ones)[0], np.full(1024, 1 / 32))
    d = -ones
    assert np.array_equal(T.forward(e, d)[0], np.full(1024, -1 / 32))


def test_blocks_independent():
    rng = np.random.default_rng(1)
    d = rand_signs(rng, 3072)
    x = np.zeros((1, 3072))
    x[0, 2048 + 17] = 3.0
    y = T.forward(x, d)
    assert not y[0, :2048].any()
    assert np.allclose(np.abs(y[0, 2048:]), 3.0 / 32.0, rtol=0, atol=0)


def test_round_trip_and_norm():
    rng = np.random.default_rng(2)
    k = 5120
    d = rand_signs(rng, k)
    x = rng.standard_normal((3, k))
    assert np.allclose(T.inverse(T.forward(x, d), d), x, rtol=0, atol=1e-12)
    assert np.allclose(T.forward(T.inverse(x, d), d), x, rtol=0, atol=1e-12)
    y = T.forward(x, d)
    for b in range(0, k, 1024):
        np.testing.assert_allclose(np.linalg.norm(y[:, b:b + 1024], axis=1),
                                   np.linalg.norm(x[:, b:b + 1024], axis=1), rtol=1e-13)


def test_forward_is_not_inverse_under_signs():
    # A plausible mistake, applying D after H in the forward transform, must
    # show: the two orders differ unless D is the identity.
    rng = np.random.default_rng(3)
    d = rand_signs(rng, 1024)
    x = rng.standard_normal((1, 1024))
    assert not np.allclose(T.forward(x, d), T.inverse(x, d))


def test_bit_conversions():
    assert T.bf16_bits_to_f64(np.array([0x3F80, 0xBF80, 0x4049, 0x0000]))[:2].tolist() == [1.0, -1.0]
    assert T.bf16_bits_to_f64(np.array([0x4049]))[0] == 3.140625
    assert T.fp16_bits_to_f64(np.array([0x3C00, 0xBC00, 0x2E66, 0x0001])).tolist() == [
        1.0, -1.0, 0.0999755859375, 2.0 ** -24]


@pytest.mark.parametrize("k", [1000, 1536])
def test_rejects_partial_block(k):
    with pytest.raises(ValueError):
        T.forward(np.zeros((1, k)), np.ones(k))


def test_block_l1_over_32_hand_values():
    # The scale of the transform tolerance: per element, the L1 norm of the
    # 1024-element block holding it, over 32 (sum_j |H_ij d_j x_j| / 32 with
    # |H_ij d_j| = 1).  Hand-computed cases: a block of ones gives 1024/32;
    # a block whose only nonzeros are 3 and -4 gives 7/32 (an L2 norm would
    # give 5/32); blocks and rows stay separate (a per-row sum would mix them).
    x = np.zeros((2, 2048))
    x[0, :1024] = 1.0
    x[0, 1024 + 5] = 3.0
    x[0, 1024 + 900] = -4.0
    x[1, 2047] = -0.5
    got = T.block_l1_over_32(x)
    assert got.shape == x.shape
    assert np.all(got[0, :1024] == 32.0)
    assert np.all(got[0, 1024:] == 7.0 / 32.0)
    assert np.all(got[1, :1024] == 0.0)
    assert np.all(got[1, 1024:] == 0.5 / 32.0)


def test_block_l1_over_32_bounds_the_transform():
    # Every output of the transform is at most the block's L1 norm over 32
    # (|H_ij| = 1), with equality where the signs line up: x = d restricted to
    # a block maps its first element to ||x||_1 / 32 exactly.
    rng = np.random.default_rng(4)
    d = rand_signs(rng, 2048)
    x = rng.standard_normal((3, 2048))
    assert np.all(np.abs(T.forward(x, d)) <= T.block_l1_over_32(x) * (1 + 1e-12))
    v = np.abs(rng.standard_normal((1, 2048))) * d
    f = T.forward(v, d)
    l1 = T.block_l1_over_32(v)
    assert np.isclose(f[0, 0], l1[0, 0], rtol=1e-13)
    assert np.isclose(f[0, 1024], l1[0, 1024], rtol=1e-13)

"""Head oracle pinned to closed forms of RMSNorm, hand-made ties of the greedy
choice and a constructed head whose logits are known without the oracle."""

import numpy as np
import pytest

from oracle import codec, head as Hd, transform as T
import synth


def test_rmsnorm_closed_forms():
    # a constant row c*1 with unit weight and eps = 0 becomes sign(c)*1
    for c in (3.0, -0.25, 1e-3):
        y = Hd.rmsnorm(np.full((1, 8), c), np.ones(8), 0.0)
        assert np.allclose(y, np.sign(c), rtol=0, atol=1e-15)
    # [3, 4]: mean square 12.5, so y = [3, 4] / sqrt(12.5 + eps)
    y = Hd.rmsnorm([[3.0, 4.0]], [1.0, 1.0], 0.5)
    assert np.allclose(y, [[3 / np.sqrt(13.0), 4 / np.sqrt(13.0)]], rtol=1e-15)
    # the weight multiplies element by element
    y = Hd.rmsnorm([[3.0, 4.0]], [2.0, -1.0], 0.5)
    assert np.allclose(y, [[6 / np.sqrt(13.0), -4 / np.sqrt(13.0)]], rtol=1e-15)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 1024))
    g = np.ones(1024)
    y = Hd.rmsnorm(x, g, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)   # unit RMS
    assert np.allclose(Hd.rmsnorm(7.5 * x, g, 0.0), y, rtol=1e-13)         # scale-free
    # eps shrinks the output: rms(y) = rms(x) / sqrt(ms(x) + eps)
    ms = np.mean(x * x, axis=1)
    ye = Hd.rmsnorm(x, g, 0.1)
    assert np.allclose(np.sqrt(np.mean(ye * ye, axis=1)), np.sqrt(ms / (ms + 0.1)), rtol=1e-13)


def test_greedy_lowest_index_on_ties():
    assert list(Hd.greedy([[1.0, 3.0, 3.0, 2.0]])) == [1]
    assert list(Hd.greedy([[-5.0, -5.0, -7.0]])) == [0]
    assert list(Hd.greedy([[0.0, -0.0, 0.0]])) == [0]     # -0 equals +0
    assert list(Hd.greedy([[np.inf, 1.0, np.inf]])) == [0]
    assert list(Hd.greedy([[1.0, 2.0], [9.0, 9.0]])) == [1, 0]


def test_greedy_skips_nan_logits():
    # NaN is never the choice; all-NaN rows have none (-1); -inf still counts
    nan = np.nan
    assert list(Hd.greedy([[nan, 1.0, 3.0, nan, 3.0]])) == [2]
    assert list(Hd.greedy([[nan, -np.inf]])) == [1]
    assert list(Hd.greedy([[nan, nan], [nan, 0.5]])) == [-1, 1]


@pytest.mark.parametrize("fmt", ["PQ2_0_G128", "PTQ1_0_G128"])
def test_constructed_head(fmt):
    """Row i of W has one trit +1 at column c_i with scale s_i; the hidden row
    is x = T^-1(z) with unit norm weight and eps = 0.  The transform is
    orthogonal, so rms(x) = rms(z), rmsnorm(x) = x / rms(z) and
    T(rmsnorm(x)) = z / rms(z): logit i = s_i * z[c_i] / rms(z), known
    without running the oracle's pipeline."""
    rng = np.random.default_rng(2)
    n, k = 300, 2048
    cols = rng.integers(0, k, n)
    trits = np.zeros((n, k), np.int8)
    trits[np.arange(n), cols] = 1
    sb = np.full((n, k // 128), 0x3C00, np.uint16)      # 1.0
    s_row = np.where(np.arange(n) % 3 == 0, 0x4000, 0x3C00).astype(np.uint16)  # 2.0 or 1.0
    sb[np.arange(n), cols // 128] = s_row
    payload = codec.pack_rowsplit(fmt, trits, sb)
    sign_bits = synth.sign_bits(rng, k)
    d = T.bf16_bits_to_f64(sign_bits)
    z = rng.standard_normal((1, k))
    x = T.inverse(z, d)
    logits, bound, xrot = Hd.head(fmt, n, k, payload, x, np.ones(k), 0.0, d)
    rms = np.sqrt(np.mean(z * z))
    scale = np.where(s_row == 0x4000, 2.0, 1.0)
    want = scale * z[0, cols] / rms
    assert np.allclose(xrot, z / rms, rtol=1e-12, atol=1e-13)
    assert np.allclose(logits[0], want, rtol=1e-12, atol=1e-13)
    assert Hd.greedy(logits)[0] == int(np.flatnonzero(want == want.max())[0])
    assert np.all(bound > 0)

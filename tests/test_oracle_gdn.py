"""Grouped-V head order oracle pinned to the page's definition, values and
trap, bijectivity, and one-hot inputs whose transform is known."""

import numpy as np
import pytest

from oracle import gdn, transform as T
from conftest import load_golden
import synth

G = load_golden("gdn_perm48.json")


def test_perm48_page_values():
    assert [gdn.perm48(i) for i in range(12)] == G["perm48_first"]
    for i, v in G["perm48_last"].items():
        assert gdn.perm48(int(i)) == v
    a, b, v = G["trap_pair"]
    assert gdn.perm48(a) == gdn.perm48(b) == v


def test_perm48_tiled_to_grouped():
    # target head g*3 + t comes from source head t*16 + g
    for g in range(16):
        for t in range(3):
            assert gdn.perm48(g * 3 + t) == t * 16 + g
    assert sorted(gdn.perm48(i) for i in range(48)) == list(range(48))


def test_perm_row_bijection_and_trap():
    rows = [gdn.perm_row(i) for i in range(6144)]
    assert sorted(rows) == list(range(6144))
    for i, v in G["perm_row_samples"].items():
        assert gdn.perm_row(int(i)) == v
    # perm48 on the raw row indices is not a bijection
    raw = [gdn.perm48(i) for i in range(6144)]
    assert len(set(raw)) < 6144


def test_gather_moves_whole_heads():
    x = np.arange(6144, dtype=np.float64).reshape(1, -1)
    r = gdn.gather(x)[0]
    for j in range(0, 6144, 128):
        src_head = int(r[j]) // 128
        assert np.array_equal(r[j:j + 128], src_head * 128 + np.arange(128))
        assert src_head == gdn.perm48(j // 128)


@pytest.mark.parametrize("src", [0, 5, 130, 2047, 2048, 4095, 6143])
def test_one_hot_lands_at_target(src):
    # a one-hot input at source position src reaches transform position
    # j with perm_row(j) == src, whose transform is d_j/32 times column
    # j mod 1024 of H over j's block
    rng = np.random.default_rng(src)
    d = T.bf16_bits_to_f64(synth.sign_bits(rng, 6144))
    x = np.zeros((1, 6144))
    x[0, src] = 1.0
    # the target position, from the page's head statement: source head
    # t*16 + g goes to target head g*3 + t
    t, g = divmod(src // 128, 16)
    j = (g * 3 + t) * 128 + src % 128
    y = gdn.forward_grouped(x, d)[0]
    blk = j // 1024
    want = np.zeros(6144)
    want[blk * 1024:(blk + 1) * 1024] = d[j] / 32.0 * T.hadamard_1024()[:, j % 1024]
    assert np.array_equal(y, want)


def test_general_shape():
    # 2 x 8 heads of 64: a bijection that reduces to the identity for 1 tile
    assert sorted(gdn.perm_row(i, 2, 8, 64) for i in range(1024)) == list(range(1024))
    assert [gdn.perm_row(i, 1, 16, 64) for i in range(1024)] == list(range(1024))

"""GGUF block stream <-> row-split planes on the GPU (tq_blocks_to_planes,
tq_planes_to_blocks) against the oracle's slices ([ninfer-skill] §4):
bit-exact, every payload byte written (inter-plane padding zero), exact
inverse, at small ragged shapes and at the config 2 / config 3 weight
sizes."""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import codec, geometry as G
from gpu_util import dev, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SHAPES = [("PQ2_0_G128", 3, 200), ("PTQ1_0_G128", 3, 200), ("PQ2_0_G128", 7, 1024),
          ("PTQ1_0_G128", 1000, 5120), ("PQ2_0_G128", 17408, 5120), ("PTQ1_0_G128", 5120, 17408),
          # odd block counts (PQ2_0 blocks move in pairs, the last one alone)
          ("PQ2_0_G128", 1, 128), ("PQ2_0_G128", 3, 384), ("PQ2_0_G128", 1001, 640),
          ("PTQ1_0_G128", 1, 128),
          # the vocabulary head's stream, as the bench transcodes it
          ("PQ2_0_G128", 248320, 5120)]


@pytest.mark.parametrize("fmt,n,k", SHAPES)
def test_blocks_to_planes_bit_exact(fmt, n, k):
    say("blocks -> planes %s n=%d k=%d" % (fmt, n, k))
    geo = G.row_split_geometry(fmt, n, k)
    rng = np.random.default_rng(n + k)
    # any bytes: the transcoder moves bytes, it does not interpret them
    blocks = rng.integers(0, 256, size=n * geo["groups_per_row"] * codec.BLOCK_BYTES[fmt], dtype=np.uint8)
    expect = codec.blocks_to_planes(fmt, n, k, blocks)
    out = torch.full((geo["payload_bytes"],), 0xAA, dtype=torch.uint8, device="cuda")
    got = tq.blocks_to_planes(dev(torch, blocks), fmt, n, k, out=out)
    back = tq.planes_to_blocks(got, fmt, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), expect)
    assert np.array_equal(back.cpu().numpy(), blocks)


@pytest.mark.parametrize("fmt,n,k", SHAPES[:4])
def test_planes_to_blocks_of_packed_weights(fmt, n, k):
    rng = np.random.default_rng(7 * n + k)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = codec.pack_rowsplit(fmt, trits, sb)
    blocks = tq.planes_to_blocks(dev(torch, payload), fmt, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(blocks.cpu().numpy(), codec.planes_to_blocks(fmt, n, k, payload))


def test_transcode_validation_enqueues_nothing():
    n, k = 4, 256
    geo = G.row_split_geometry("PQ2_0_G128", n, k)
    blocks = torch.zeros(n * 2 * 34, dtype=torch.uint8, device="cuda")
    out = torch.full((geo["payload_bytes"] + 256,), 7, dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.blocks_to_planes(blocks, "PQ2_0_G128", n, k, out=out)  # payload size mismatch
    assert e.value.status == 3
    with pytest.raises(tq.TQError) as e:
        tq.blocks_to_planes(blocks[:-1], "PQ2_0_G128", n, k, out=out[:geo["payload_bytes"]])
    assert e.value.status == 3 and "block stream stores" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7).all())

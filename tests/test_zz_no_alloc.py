"""The allocation-free head entry point (tq_head_argmax_noalloc) against the
head entry point with a caller work buffer (tq_head_argmax), through the C
ABI: two calls in a row, the second on a smaller head, each compared with
the work-buffer call on the same inputs (token equal, logits bitwise equal:
the same kernel runs) and with the float64 oracle at the stated bound."""

import numpy as np
import pytest

import ternary_quantized_amd as tq
import synth
from oracle import head as Hd, transform as T
from gpu_util import assert_within, dev, say, signs_dev, x_dev, x_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FMT = "PQ2_0_G128"


def inputs(n, k, seed):
    rng = np.random.default_rng(seed)
    trits = synth.trits_sparse(rng, n, k)
    sb = synth.scale_bits_lognormal(rng, n, synth.groups_of(k))
    payload = tq.pack_rowsplit(FMT, trits, sb)
    sbits = synth.sign_bits(rng, k)
    gbits = synth.norm_weight_bits(rng, k)
    x = synth.activations_bf16_bits(rng, 1, k)
    return payload, sbits, gbits, x


@pytest.mark.parametrize("shapes", [((60000, 5120), (1000, 2048))])
def test_noalloc_head_matches_work_buffer_head(shapes):
    for (n, k), seed in zip(shapes, (5, 6)):
        payload, sbits, gbits, x = inputs(n, k, seed)
        say("noalloc head n=%d k=%d" % (n, k))
        pd, xd, sd = dev(torch, payload), x_dev(torch, x, "bf16"), signs_dev(torch, sbits)
        gd = dev(torch, gbits.view(np.int16)).view(torch.bfloat16)
        lg_a = torch.empty(n, dtype=torch.float32, device="cuda")
        lg_b = torch.empty(n, dtype=torch.float32, device="cuda")
        tok_a = tq.head_argmax_noalloc(pd, FMT, n, k, xd, gd, 1e-6, sd, logits=lg_a)
        work = torch.zeros(2, dtype=torch.int64, device="cuda")
        tok_b = tq.head_argmax(pd, FMT, n, k, xd, gd, 1e-6, sd, work, logits=lg_b)
        torch.cuda.synchronize()
        assert int(tok_a.item()) == int(tok_b.item())
        assert torch.equal(lg_a, lg_b)
        lo, bound, _ = Hd.head(FMT, n, k, payload, x_f64(x, "bf16"), T.bf16_bits_to_f64(gbits), 1e-6,
                               T.bf16_bits_to_f64(sbits))
        lg = lg_a.cpu().numpy().astype(np.float64)
        assert_within(lg, lo[0], bound[0], "noalloc head logits")
        assert int(tok_a.item()) == int(np.flatnonzero(lg == lg.max())[0])

"""The one-launch head entry point on the CPU: argument validation (only
arguments that fail validation, which returns before any HIP call)."""

import ternary_quantized_amd as tq

DEV = 1 << 20      # a 256-byte aligned stand-in address; never dereferenced


def test_head_validation_without_gpu():
    L = tq.lib()
    f = L.tq_head_argmax
    n, k = 64, 5120
    pb = tq.geometry("PQ2_0_G128", n, k)["payload_bytes"]
    ok = dict(x=DEV, xd=1, g=DEV, eps=1e-6, s=DEV, lg=DEV, w=DEV, t=DEV)

    def call(payload=DEV, nbytes=pb, fmt=142, nn=n, kk=k, **kw):
        a = dict(ok, **kw)
        return f(payload, nbytes, fmt, nn, kk, a["x"], a["xd"], a["g"], a["eps"], a["s"], a["lg"],
                 a["w"], a["t"], None)

    assert call(nbytes=pb + 1) == 3                     # payload size
    assert call(fmt=141) == 2                           # format
    assert call(kk=5120 + 128, nbytes=tq.geometry("PQ2_0_G128", n, 5248)["payload_bytes"]) == 5
    assert call(xd=5) == 1                              # dtype
    assert call(eps=-1.0) == 1 and call(eps=float("nan")) == 1 and call(eps=float("inf")) == 1
    assert call(x=None) == 1 and call(g=None) == 1 and call(w=None) == 1 and call(t=None) == 1
    assert call(s=None) == 1                            # signs
    assert call(x=DEV + 8) == 4 and call(g=DEV + 2) == 4 and call(s=DEV + 4) == 4
    assert call(w=DEV + 8) == 4 and call(t=DEV + 2) == 4 and call(lg=DEV + 2) == 4
    # not covered: PTQ1_0, k beyond the batch-1 kernel
    pt = tq.geometry("PTQ1_0_G128", n, k)["payload_bytes"]
    assert call(fmt=143, nbytes=pt) == 6
    assert b"tq_hadamard_signed then tq_gemv_rowsplit" in L.tq_last_error()
    big = 12 * 1024
    assert call(kk=big, nbytes=tq.geometry("PQ2_0_G128", n, big)["payload_bytes"]) == 6

"""The output head of a decode step: RMSNorm, signed transform, ternary head
projection and greedy choice, in float64 (oracle; test infrastructure only).

[tensorsharp] §4.4 gives the order after the last layer: RMSNorm, then the
signed Hadamard transform, then the low-bit output head, which yields the
logits.  Greedy decoding takes the token with the largest logit; a fused
GEMV that finds the argmax over the vocabulary appears in [gguf-explainer]
§4.5 (its drafter kernel).

Readings (the pages name the steps but not their formulas):
* RMSNorm of a row x with weight g: y_j = x_j / sqrt(mean_j(x_j^2) + eps) * g_j,
  eps an argument (the plain RMSNorm; a model that stores g as an offset from
  one passes 1 + g);
* the transform is the forward signed transform of the projection inputs;
* greedy choice: the lowest index among the largest logits; NaN logits are
  never chosen, and a row of NaN logits gives -1.
"""

import numpy as np

from . import projection, transform


def rmsnorm(x, g, eps):
    """Rows of x normalised by their root mean square, times g (float64)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = np.asarray(g, dtype=np.float64).reshape(1, -1)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def greedy(logits):
    """Index of the largest logit per row; the lowest such index on a tie.
    A NaN logit is not a number to compare, so it is never chosen; a row whose
    logits are all NaN has no choice, reported as -1 (a reading: the pages do
    not say)."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    out = []
    for row in logits:
        ok = ~np.isnan(row)
        if not ok.any():
            out.append(-1)
            continue
        best = row[ok].max()
        out.append(int(np.flatnonzero(ok & (row == best))[0]))
    return np.array(out)


def head(fmt, n, k, payload, x, g, eps, signs):
    """(logits [rows, n], acceptance bound [rows, n], xrot [rows, k]) of the
    head step on hidden rows x: xrot = H(D . rmsnorm(x))/32 per block, then
    logits = W . xrot over the row-split payload."""
    xrot = transform.forward(rmsnorm(x, g, eps), signs)
    logits, bound = projection.project_payload(fmt, n, k, payload, xrot)
    return logits, bound, xrot

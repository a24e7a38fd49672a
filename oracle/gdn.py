"""Grouped-V head order of the GatedDeltaNet output before its transform
(oracle; test infrastructure only).

[ninfer-skill] §5: the 48 value heads are stored tiled as (3, 16) and used
grouped as (16, 3): target head g*3 + t comes from source head t*16 + g,
i.e. perm48(i) = (i % 3) * 16 + i // 3; a row index moves at head
granularity, perm_row(i) = perm48(i // 128) * 128 + i % 128 (128 rows per
head, 6144 rows in all).  perm48 applied to the raw row indices is not a
bijection (perm48(1) == perm48(48) == 16).  [tensorsharp] §4.2: with the
grouped GDN metadata set, the input of the projection that follows the
GatedDeltaNet is reordered into that head order before its signed
transform.

Reading: the reordered row is r[j] = x[perm_row(j)] (element j of the
transform input is taken from source position perm_row(j)), generalised to
`tiles` x `groups` heads of `head_dim` elements:
perm(i) = (i % tiles) * groups + i // tiles.
"""

import numpy as np

from . import transform

TILES, GROUPS, HEAD_DIM = 3, 16, 128   # [ninfer-skill] §5/§6: V_HEADS 48, V_HEAD_DIM 128


def perm_head(i, tiles=TILES, groups=GROUPS):
    return (i % tiles) * groups + i // tiles


def perm48(i):
    return perm_head(i, TILES, GROUPS)


def perm_row(i, tiles=TILES, groups=GROUPS, head_dim=HEAD_DIM):
    head, inner = divmod(i, head_dim)
    return perm_head(head, tiles, groups) * head_dim + inner


def gather(x, tiles=TILES, groups=GROUPS, head_dim=HEAD_DIM):
    """Rows of x [rows, tiles*groups*head_dim] in the grouped head order."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    k = tiles * groups * head_dim
    if x.shape[1] != k:
        raise ValueError("width must be tiles * groups * head_dim")
    src = [perm_row(j, tiles, groups, head_dim) for j in range(k)]
    return x[:, src]


def forward_grouped(x, d, tiles=TILES, groups=GROUPS, head_dim=HEAD_DIM):
    """H(D . gather(x)) / 32 per 1024-element block, in float64."""
    return transform.forward(gather(x, tiles, groups, head_dim), d)

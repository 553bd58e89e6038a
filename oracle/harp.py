"""Dense HARP structured rotation.  Test infrastructure only.

[HARP] 2.1: a mixed-radix schedule b = (b_0 .. b_{m-1}) with prod b_t = d;
stage t applies a block-diagonal orthogonal matrix B_t to coordinate groups
separated by a stride permutation.  [HARP] 2.2: each block is
B_{t,c} = Q_{t,c} G_{b_t}; at Theta = 0, Q = I and the rotation reduces to
the fixed RHT up to a fixed permutation convention.

Readings (the pages give only "stride permutation"):
  * index digits: i = sum_t i_t * stride_t with stride_t = prod_{u<t} b_u,
    so stage t acts on digit t, stages applied t = 0, 1, ... in order;
  * the block of stage t that row i belongs to is
    c = (i mod stride_t) + stride_t * floor(i / (stride_t * b_t)),
    i.e. i with digit t deleted, remaining digits in increasing significance;
  * a block acts as out_sub[k] = sum_j B[k][j] in_sub[j];
  * "random-sign Hadamard preconditioning" is the full-length RHT Hn(S x)
    applied before the first stage.
"""

import numpy as np

from .hadamard import rht


def strides(radices):
    st, acc = [], 1
    for b in radices:
        st.append(acc)
        acc *= b
    return st, acc


def check_schedule(radices, d):
    """prod b_t must equal d ([HARP] 2.1); every radix at least 2."""
    if any(int(b) < 2 for b in radices):
        raise ValueError("every radix must be >= 2")
    if int(np.prod([int(b) for b in radices])) != d:
        raise ValueError("product of radices must equal d")


def block_index(i, t, radices):
    st, _ = strides(radices)
    s, b = st[t], radices[t]
    return (i % s) + s * (i // (s * b))


def stage_matrix(blocks_t, t, radices):
    """Dense d x d matrix of stage t from its blocks [d/b_t, b_t, b_t]."""
    st, d = strides(radices)
    s, b = st[t], radices[t]
    blocks_t = np.asarray(blocks_t, dtype=np.float64)
    if blocks_t.shape != (d // b, b, b):
        raise ValueError("blocks of stage %d must be [%d, %d, %d]" % (t, d // b, b, b))
    m = np.zeros((d, d), dtype=np.float64)
    i = np.arange(d)
    dig = (i // s) % b                   # digit t of every row index
    base = i - dig * s                   # same index with digit t zeroed
    c = block_index(i, t, radices)
    for k in range(b):                   # column j = base + k*s agrees on all other digits
        m[i, base + k * s] = blocks_t[c, dig, k]
    return m


def harp_rotate(x, radices, blocks, s=None, precondition=True):
    """y = Stage_{m-1}( ... Stage_0( P x ) ), P = Hn S if precondition else I.

    blocks: list (one per stage) of arrays [d/b_t, b_t, b_t]; x [tokens, d].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[1]
    check_schedule(radices, d)
    if precondition:
        if s is None:
            s = np.ones(d)
        z = rht(x, s)
    else:
        z = x.copy()
    for t in range(len(radices)):
        z = z @ stage_matrix(blocks[t], t, radices).T
    return z

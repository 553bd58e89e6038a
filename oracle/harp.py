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


# ---------------------------------------------------- block parametrisation
#
# [HARP] 2.2: each learned block is B_{t,c}(theta) = Q_{t,c}(theta) G_{b_t},
# G a fixed base mixer (the normalised Sylvester Hadamard when b_t is a power
# of two, otherwise a fixed orthogonal substitute such as the QR factor of a
# Gaussian matrix), Q orthogonal: a Givens rotation when b_t = 2, a Cayley
# map when b_t > 2; Theta = 0 gives Q = I, so B = G.  [HARP] 2.4: the
# parameters may be stored as int8.
#
# Readings (the pages name the maps only):
#   * Givens: Q = [[cos t, -sin t], [sin t, cos t]], one angle per block;
#   * Cayley: Q = (I - A)(I + A)^-1 with A skew-symmetric, its b(b-1)/2
#     parameters the strict upper triangle row by row (A[i][j] = p, i < j,
#     A[j][i] = -p);
#   * int8: theta = s_t * q with one fp32 scale s_t per stage;
#   * layout: stage-major, stage t as [d / b_t][P_t] parameters.


def params_per_block(b):
    return 1 if b == 2 else b * (b - 1) // 2


def skew_from_params(p, b):
    a = np.zeros((b, b), dtype=np.float64)
    iu = np.triu_indices(b, 1)
    a[iu] = np.asarray(p, dtype=np.float64)
    return a - a.T


def cayley(a):
    """Q = (I - A)(I + A)^-1 (orthogonal, det +1 for skew-symmetric A)."""
    i = np.eye(a.shape[0])
    return (i - a) @ np.linalg.inv(i + a)


def givens(theta):
    c, s = np.cos(theta), np.sin(theta)
    return np.array([[c, -s], [s, c]], dtype=np.float64)


def sylvester_mixer(b):
    from .hadamard import sylvester
    return sylvester(b).astype(np.float64) / np.sqrt(b)


def build_blocks(params, radices, d, mixers=None):
    """Blocks Q(theta) G per stage, fp64: a list of [d / b_t, b_t, b_t].

    params: flat, stage-major ([d / b_t][P_t] per stage), already in radians /
    Cayley units (see dequant_params for int8).  mixers: list of b_t x b_t
    matrices, or None for the Sylvester mixer (every radix a power of two)."""
    check_schedule(radices, d)
    params = np.asarray(params, dtype=np.float64)
    out, o = [], 0
    for t, b in enumerate(radices):
        g = sylvester_mixer(b) if mixers is None else np.asarray(mixers[t], dtype=np.float64)
        p = params_per_block(b)
        nb = d // b
        blk = np.empty((nb, b, b), dtype=np.float64)
        for c in range(nb):
            th = params[o + c * p: o + (c + 1) * p]
            q = givens(th[0]) if b == 2 else cayley(skew_from_params(th, b))
            blk[c] = q @ g
        out.append(blk)
        o += nb * p
    return out


def dequant_params(q, scales, radices, d):
    """theta = s_t * q for int8 codes q, one scale per stage."""
    q = np.asarray(q, dtype=np.float64)
    out, o = np.empty_like(q), 0
    for t, b in enumerate(radices):
        n = (d // b) * params_per_block(b)
        out[o:o + n] = q[o:o + n] * float(scales[t])
        o += n
    return out


# ------------------------------------------------------ two-sided application
#
# [HARP] technical summary, proposal paragraph: HARP is a learnable two-sided
# orthogonal processor replacing the fixed RHT of incoherence processing.
# Reading: for a weight matrix W [d_out x d_in] of a layer y = W x, the input
# side rotates every row of W (the d_in coordinates) with R_in and the output
# side every column (the d_out coordinates) with R_out, so the processed
# weight is W~ = R_out W R_in^T (and the layer's output is R_out y when its
# input is R_in x).  Each side is one harp_rotate with its own schedule,
# blocks, signs and preconditioning.


def rotation_matrix(d, radices, blocks, s=None, precondition=True):
    """The d x d matrix R with harp_rotate(x) = x R^T for row vectors x."""
    return harp_rotate(np.eye(d), radices, blocks, s=s, precondition=precondition).T


def harp_two_sided(w, out_side, in_side):
    """W~ = R_out W R_in^T, fp64.  out_side / in_side: dicts of
    (radices, blocks, s, precondition) for harp_rotate on the d_out and d_in
    coordinates."""
    w = np.asarray(w, dtype=np.float64)
    r_out = rotation_matrix(w.shape[0], **out_side)
    r_in = rotation_matrix(w.shape[1], **in_side)
    return r_out @ w @ r_in.T

"""Dense QWHA adapter forward and backward.  Test infrastructure only.

[QWHA] 2.1: the adapter is Delta W = F H^-1 with a single transform on the
input side; F is sparse, built from a value vector c and an index list E.

Reading: F is [d_out x d_in]; with the orthonormal Hn (its own inverse),
Delta W = F Hn and the adapter output for activation rows x is
y = x Delta W^T = (x Hn) F^T.
"""

import numpy as np

from .hadamard import wht


def csr_to_dense(row_ptr, col_idx, vals, d_out, d_in):
    """Dense fp64 F from CSR (duplicates, if any, are summed)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    vals = np.asarray(vals, dtype=np.float64)
    f = np.zeros((d_out, d_in), dtype=np.float64)
    rows = np.repeat(np.arange(d_out), np.diff(row_ptr))
    np.add.at(f, (rows, col_idx), vals)
    return f


def coo_to_csr(rows, cols, vals, d_out):
    """(c, E) as COO triples -> CSR with columns sorted within each row."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    vals = np.asarray(vals)
    order = np.lexsort((cols, rows))
    counts = np.bincount(rows, minlength=d_out)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return row_ptr, cols[order].astype(np.int32), vals[order]


def qwha_forward(x, row_ptr, col_idx, vals, d_out):
    """y = (x Hn) F^T, fp64, x [tokens, d_in]."""
    x = np.asarray(x, dtype=np.float64)
    f = csr_to_dense(row_ptr, col_idx, vals, d_out, x.shape[1])
    return wht(x) @ f.T


# ---------------------------------------------------------------- backward
#
# The adapter is linear in x and in the values c of F ([QWHA] 2.1:
# y = x Delta W^T with Delta W = F Hn), so the gradients of a loss L(y) with
# upstream dy = dL/dy are the adjoint products written out:
#   dL/dx = dy Delta W = (dy F) Hn              (Hn symmetric, Hn^T = Hn)
#   dL/dc_e = sum_t dy[t, o_e] (x_t Hn)[k_e]    for the entry e at (o_e, k_e)


def qwha_backward_input(dy, row_ptr, col_idx, vals, d_in):
    """dx = (dy F) Hn, fp64; dy [tokens, d_out]."""
    dy = np.asarray(dy, dtype=np.float64)
    f = csr_to_dense(row_ptr, col_idx, vals, dy.shape[1], d_in)
    return wht(dy @ f)


def qwha_grad_values(x, dy, row_ptr, col_idx):
    """dc[e] = sum_t dy[t, row(e)] * (x Hn)[t, col_idx[e]], fp64, in CSR entry order."""
    z = wht(np.asarray(x, dtype=np.float64))
    dy = np.asarray(dy, dtype=np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    cols = np.asarray(col_idx, dtype=np.int64)
    return np.einsum("te,te->e", dy[:, rows], z[:, cols])


def csr_transpose(row_ptr, col_idx, vals, d_in):
    """CSR of F^T (= CSC of F) with rows sorted by column of F, plus perm:
    entry j of the result is entry perm[j] of the input."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    cols = np.asarray(col_idx, dtype=np.int64)
    rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    perm = np.lexsort((rows, cols))
    counts = np.bincount(cols, minlength=d_in)
    t_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return t_ptr, rows[perm].astype(np.int32), np.asarray(vals)[perm], perm

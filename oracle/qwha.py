"""Dense QWHA adapter forward.  Test infrastructure only.

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

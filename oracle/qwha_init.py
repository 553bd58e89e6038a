"""QWHA adapter initialisation: quantisation error in the transform basis,
AdaAlloc parameter allocation and selection, and value refinement.
Test infrastructure only.

[QWHA] 2.2: the adapter is initialised in two stages.  AdaAlloc spreads a
total parameter budget p over the output channels in proportion to each
channel's activation error, with a minimum per channel (so the adapter stays
full rank), and inside each channel keeps the coefficients of largest
magnitude.  Refinement then sets the kept values by least squares on the
selected basis vectors, minimising the layer output error
||Delta W_Q X - F H^-1 X||_F^2 rather than copying the dense solution.

Readings (the pages give the rules, not the formulas):
  * Q is this library's quantiser: RHT + per-group RTN, then dequantisation
    and the inverse RHT (rtn.dequantize_inverse); Delta W_Q = W - Q(W).
  * With Delta W = F Hn (the adapter convention of qwha.py), the dense
    coefficient matrix is F_dense = Delta W_Q Hn (Hn is its own inverse).
  * Rows are the output channels; x [T, d_in] holds calibration tokens as
    rows, so the layer output error of channel o is x Delta W_Q[o]^T and its
    "activation error magnitude" is e_o = ||x Delta W_Q[o]^T||_2.
  * Allocation: real budgets r_o = clip(lam e_o, floor, cap) with lam such
    that sum r_o = p, then floor(r_o) plus one for the p - sum floor(r_o)
    channels of largest fractional part (ties to the lower channel index).
    cap bounds a channel's budget (at most d_in; this library refines with
    at most 128 per channel).
  * Selection: the n_o coefficients of largest |F_dense[o][k]|, ties to the
    lower k; stored in CSR with ascending columns.
  * Refinement: per channel, c_o = argmin_c ||x Delta W_Q[o]^T - (x Hn)[:, E_o] c||_2
    (ordinary least squares; E_o the selected columns).
"""

import numpy as np

from .hadamard import wht
from .rtn import dequantize_inverse


def error_coeffs(w, codes, s16, s, bits, group):
    """F_dense = (W - Q(W)) Hn for stored codes / scales of W; fp64 [d_out, d_in]."""
    w = np.asarray(w, dtype=np.float64)
    n = w.shape[1]
    return wht(w - dequantize_inverse(codes, s16, s, bits, group, n))


def channel_errors(x, f_dense):
    """e_o = ||x Delta W[o]^T||_2 with Delta W = F_dense Hn (x [T, d_in])."""
    x = np.asarray(x, dtype=np.float64)
    dw = wht(np.asarray(f_dense, dtype=np.float64))     # F Hn, rows
    return np.sqrt(((x @ dw.T) ** 2).sum(axis=0))


def _water_level(e, p, floor, cap):
    """lam with sum clip(lam e, floor, cap) = p: the sum is continuous and
    non-decreasing in lam, so bisect it."""
    lo, hi = 0.0, 1.0
    while np.clip(hi * e, floor, cap).sum() < p:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.clip(mid * e, floor, cap).sum() < p:
            lo = mid
        else:
            hi = mid
    return lo    # sum clip(lo e) <= p, so floor(r) leaves a non-negative remainder


def allocate(e, p, floor, cap):
    """Integer budgets n_o, floor <= n_o <= cap, sum n_o = p (see the module readings)."""
    e = np.asarray(e, dtype=np.float64)
    m = e.size
    if floor * m > p or cap * m < p or floor > cap:
        raise ValueError("budget outside [floor * rows, cap * rows]")
    if np.all(e == 0):
        real = np.full(m, p / m)
    else:
        real = np.clip(_water_level(e, p, floor, cap) * e, floor, cap)
    base = np.floor(real).astype(np.int64)
    rem = int(p - base.sum())
    if rem < 0 or rem > int((base < cap).sum()):
        raise AssertionError("allocation remainder out of range")
    frac = real - base
    frac[base >= cap] = -1.0                      # a capped channel takes no extra
    order = np.lexsort((np.arange(m), -frac))     # largest fraction, then lower index
    base[order[:rem]] += 1
    return base


def select(f_dense, budgets):
    """CSR support: per row the budget's largest |F| (ties to the lower column),
    columns ascending.  Returns (row_ptr, col_idx)."""
    f = np.abs(np.asarray(f_dense, dtype=np.float64))
    budgets = np.asarray(budgets, dtype=np.int64)
    rows, n = f.shape
    row_ptr = np.zeros(rows + 1, dtype=np.int64)
    np.cumsum(budgets, out=row_ptr[1:])
    cols = np.empty(row_ptr[-1], dtype=np.int64)
    for o in range(rows):
        order = np.lexsort((np.arange(n), -f[o]))   # by magnitude, then index
        cols[row_ptr[o]:row_ptr[o + 1]] = np.sort(order[:budgets[o]])
    return row_ptr, cols


def calibration_gram(x):
    """G = (x Hn)^T (x Hn), fp64 [d_in, d_in]: the Gram matrix of the rotated
    calibration tokens.  The refinement's least squares has the normal
    equations G[E][E] c = (F_dense G)[o][E], and e_o^2 = F_dense[o] G F_dense[o]^T
    (reading of [QWHA] 2.2: least squares on the selected transform columns)."""
    z = wht(np.asarray(x, dtype=np.float64))
    return z.T @ z


def refine(x, f_dense, row_ptr, col_idx):
    """Least-squares values on the support: c_o = argmin ||x dW[o]^T - Z[:, E_o] c||
    with Z = x Hn and dW = F_dense Hn.  fp64, in CSR order."""
    x = np.asarray(x, dtype=np.float64)
    z = wht(x)
    target = x @ wht(np.asarray(f_dense, dtype=np.float64)).T     # [T, d_out]
    vals = np.empty(len(col_idx), dtype=np.float64)
    for o in range(len(row_ptr) - 1):
        a, b = int(row_ptr[o]), int(row_ptr[o + 1])
        if a == b:
            continue
        cols = np.asarray(col_idx[a:b], dtype=np.int64)
        vals[a:b] = np.linalg.lstsq(z[:, cols], target[:, o], rcond=None)[0]
    return vals


def output_error(x, f_dense, row_ptr, col_idx, vals):
    """||x dW^T - x (F Hn)^T||_F^2 for the sparse F given in CSR."""
    x = np.asarray(x, dtype=np.float64)
    d_out, d_in = np.asarray(f_dense).shape
    f = np.zeros((d_out, d_in))
    rows = np.repeat(np.arange(d_out), np.diff(np.asarray(row_ptr)))
    f[rows, np.asarray(col_idx)] = vals
    return float(((x @ wht(np.asarray(f_dense, dtype=np.float64)).T - x @ wht(f).T) ** 2).sum())

"""Planted mistakes in the oracle (on the CPU only): each plausible slip --
a dropped factor, a wrong sign placement, a transposed operand, a wrong
index convention -- must make at least one pin fail."""
import numpy as np
import pytest

import oracle.hadamard as H
import oracle.rtn as R
import oracle.qwha as Q
import oracle.harp as P
import test_oracle_hadamard as th
import test_oracle_rtn as tr
import test_oracle_qwha_harp as tq


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_mutant_unnormalised(monkeypatch):
    orig = H.wht
    monkeypatch.setattr(H, "wht", lambda x, normalize=True: orig(x, normalize=False))
    _fails(th.test_involution_and_norm, 64)


def test_mutant_sequency_order(monkeypatch):
    orig = H.sylvester

    def seq(n):
        h = orig(n)
        changes = (np.diff(h, axis=1) != 0).sum(axis=1)
        return h[np.argsort(changes, kind="stable")]
    monkeypatch.setattr(H, "sylvester", seq)
    _fails(th.test_matches_scipy_hadamard, 8)
    _fails(th.test_golden_h4)


def test_mutant_signs_after(monkeypatch):
    monkeypatch.setattr(H, "rht", lambda x, s: H.wht(x) * s)
    _fails(th.test_sign_diagonal_orthogonality)


def test_mutant_sign_mask_msb_first(monkeypatch):
    def msb(bits, n):
        bits = np.asarray(bits, dtype=np.uint32)
        j = np.arange(n)
        b = (bits[j >> 5] >> (31 - (j & 31)).astype(np.uint32)) & np.uint32(1)
        return 1.0 - 2.0 * b.astype(np.float64)
    monkeypatch.setattr(H, "signs_from_bits", msb)
    _fails(th.test_sign_mask_golden)


def test_mutant_qmax(monkeypatch):
    monkeypatch.setattr(R, "qmax_of", lambda bits: 1 << (bits - 1))
    _fails(tr.test_rtn_invariants, 4)


def test_mutant_floor_rounding(monkeypatch):
    monkeypatch.setattr(R.np, "rint", np.floor)
    try:
        _fails(tr.test_rtn_bruteforce, 4)
    finally:
        monkeypatch.undo()


def test_mutant_pack_msb_first(monkeypatch):
    def pack(q, bits):
        q = np.asarray(q, dtype=np.int64)
        rows, n = q.shape
        u = q & ((1 << bits) - 1)
        planes = (u[:, :, None] >> np.arange(bits)[::-1]) & 1
        return np.packbits(planes.reshape(rows, n * bits).astype(np.uint8), axis=1,
                           bitorder="little")
    monkeypatch.setattr(R, "pack_codes", pack)
    _fails(tr.test_packing_golden)


def test_mutant_dequant_no_sign_extension(monkeypatch):
    def unpack(codes, bits, n):
        planes = np.unpackbits(np.asarray(codes, np.uint8), axis=1, bitorder="little")
        planes = planes[:, :n * bits].reshape(codes.shape[0], n, bits).astype(np.int64)
        return (planes << np.arange(bits)).sum(axis=2)
    monkeypatch.setattr(R, "unpack_codes", unpack)
    _fails(tr.test_grid_constructed_roundtrip, 4, 128, 1024)


def test_mutant_qwha_untransposed(monkeypatch):
    def fwd(x, row_ptr, col_idx, vals, d_out):
        f = Q.csr_to_dense(row_ptr, col_idx, vals, d_out, x.shape[1])
        return H.wht(x) @ f          # F instead of F^T
    monkeypatch.setattr(Q, "qwha_forward", fwd)
    _fails(tq.test_qwha_single_nonzero)


def test_mutant_harp_block_transposed(monkeypatch):
    orig = P.stage_matrix
    monkeypatch.setattr(P, "stage_matrix",
                        lambda b, t, r: orig(np.transpose(np.asarray(b), (0, 2, 1)), t, r))
    _fails(tq.test_harp_bruteforce, (4, 4))


def test_mutant_harp_digit_order(monkeypatch):
    orig = P.stage_matrix

    def rev(b, t, r):
        m = len(r)
        rr = list(r)[::-1]
        # act on digit m-1-t instead of t
        return orig(b, m - 1 - t, rr) if rr == list(r) else orig(b, t, r)[::-1, ::-1]
    monkeypatch.setattr(P, "stage_matrix", rev)
    _fails(tq.test_harp_bruteforce, (2, 4, 3))
    _fails(tq.test_harp_permutation_blocks_at_real_shape)


def test_mutant_qwha_backward_no_transform(monkeypatch):
    def bwd(dy, row_ptr, col_idx, vals, d_in):
        f = Q.csr_to_dense(row_ptr, col_idx, vals, dy.shape[1], d_in)
        return np.asarray(dy, dtype=np.float64) @ f   # the Hn factor dropped
    monkeypatch.setattr(Q, "qwha_backward_input", bwd)
    _fails(tq.test_qwha_backward_input_is_the_adjoint, 64, 48)


def test_mutant_qwha_grad_values_untransformed_x(monkeypatch):
    def gv(x, dy, row_ptr, col_idx):
        rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
        return np.einsum("te,te->e", np.asarray(dy)[:, rows], np.asarray(x)[:, col_idx])  # x, not x Hn
    monkeypatch.setattr(Q, "qwha_grad_values", gv)
    _fails(tq.test_qwha_grad_values_finite_differences)


def test_mutant_cayley_inverse_order(monkeypatch):
    """(I + A)(I - A)^-1 (the inverse rotation) fails the 2x2 closed form."""
    from oracle import harp
    monkeypatch.setattr(harp, "cayley", lambda a: (np.eye(a.shape[0]) + a) @ np.linalg.inv(np.eye(a.shape[0]) - a))
    with pytest.raises(AssertionError):
        import test_oracle_qwha_harp as T
        T.test_cayley_2x2_closed_form()


def test_mutant_mixer_on_the_left(monkeypatch):
    """G Q instead of Q G fails the single-parameter placement pin."""
    from oracle import harp
    orig = harp.build_blocks

    def mutant(params, radices, d, mixers=None):
        blocks = orig(np.zeros_like(np.asarray(params, dtype=float)), radices, d, mixers)
        out, o = [], 0
        for t, b in enumerate(radices):
            g = harp.sylvester_mixer(b) if mixers is None else np.asarray(mixers[t], dtype=float)
            p = harp.params_per_block(b)
            blk = blocks[t].copy()
            for c in range(d // b):
                th = np.asarray(params, dtype=float)[o + c * p: o + (c + 1) * p]
                q = harp.givens(th[0]) if b == 2 else harp.cayley(harp.skew_from_params(th, b))
                blk[c] = g @ q
            out.append(blk)
            o += (d // b) * p
        return out
    monkeypatch.setattr(harp, "build_blocks", mutant)
    with pytest.raises(AssertionError):
        import test_oracle_qwha_harp as T
        T.test_build_blocks_single_parameter_placement()


def test_mutant_gemv_signs_on_the_code_side(monkeypatch):
    """Applying S to the codes before the transform (Hn S (q s)) instead of after
    it fails the brute-force layer."""
    from oracle import gemv, rtn
    import test_oracle_gemv as tg

    def mutant(x, codes, s16, s, bits, group, n):
        y_hat = rtn.dequantize(codes, s16, bits, group, n) * np.asarray(s)[None, :]
        return np.asarray(x, dtype=float) @ H.wht(y_hat).T
    monkeypatch.setattr(gemv, "rht_gemv", mutant)
    with pytest.raises(AssertionError):
        tg.test_gemv_bruteforce_tiny()


# ---- QWHA initialisation (AdaAlloc, refinement)
import oracle.qwha_init as QI
import test_oracle_qwha_init as ti


def test_mutant_error_coeffs_without_transform(monkeypatch):
    monkeypatch.setattr(QI, "error_coeffs", lambda w, c, s16, s, b, g: np.asarray(w, np.float64)
                        - R.dequantize_inverse(c, s16, s, b, g, np.asarray(w).shape[1]))
    _fails(ti.test_error_coeffs_bruteforce)


def test_mutant_channel_errors_in_coefficient_basis(monkeypatch):
    monkeypatch.setattr(QI, "channel_errors", lambda x, f: np.sqrt(((np.asarray(x) @ np.asarray(f).T) ** 2).sum(0)))
    _fails(ti.test_channel_errors_bruteforce)


def test_mutant_allocation_by_squared_error(monkeypatch):
    orig = QI.allocate
    monkeypatch.setattr(QI, "allocate", lambda e, p, fl, cap: orig(np.asarray(e, np.float64) ** 2, p, fl, cap))
    _fails(ti.test_allocate_hand_worked)


def test_mutant_selection_ties_to_higher_index(monkeypatch):
    def sel(f, budgets):
        f = np.abs(np.asarray(f, np.float64))
        budgets = np.asarray(budgets)
        row_ptr = np.concatenate([[0], np.cumsum(budgets)])
        cols = np.concatenate([np.sort(np.lexsort((-np.arange(f.shape[1]), -f[o]))[:budgets[o]])
                               for o in range(f.shape[0])])
        return row_ptr, cols
    monkeypatch.setattr(QI, "select", sel)
    _fails(ti.test_select_bruteforce)


def test_mutant_refine_without_transform(monkeypatch):
    def ref(x, f, row_ptr, cols):
        x = np.asarray(x, np.float64)
        target = x @ H.wht(np.asarray(f, np.float64)).T
        vals = np.empty(len(cols))
        for o in range(len(row_ptr) - 1):
            a, b = row_ptr[o], row_ptr[o + 1]
            if a < b:
                vals[a:b] = np.linalg.lstsq(x[:, cols[a:b]], target[:, o], rcond=None)[0]
        return vals
    monkeypatch.setattr(QI, "refine", ref)
    _fails(ti.test_refine_normal_equations_and_gain)


def test_mutant_gram_without_transform(monkeypatch):
    monkeypatch.setattr(QI, "calibration_gram", lambda x: np.asarray(x, np.float64).T @ np.asarray(x, np.float64))
    _fails(ti.test_calibration_gram_bruteforce)
    _fails(ti.test_calibration_gram_normal_equations)



# ---- parity rules (oracle/compare.py): each mutant is the module's own
# function with one plausible slip written into its source
import inspect
import oracle.compare as C
import test_oracle_compare as tc


def _mutant_of(fn, old, new):
    src = inspect.getsource(fn)
    assert old in src, old
    ns = dict(vars(C))
    exec(src.replace(old, new), ns)
    return ns[fn.__name__]


def test_mutant_boundary_at_integers(monkeypatch):
    monkeypatch.setattr(C, "near_boundary", _mutant_of(C.near_boundary, "np.floor(v) + 0.5", "np.rint(v)"))
    _fails(tc.test_near_boundary_hand_worked)


def test_mutant_absolute_window(monkeypatch):
    monkeypatch.setattr(C, "near_boundary", _mutant_of(C.near_boundary, "window * np.abs(b)", "window"))
    _fails(tc.test_near_boundary_hand_worked)


def test_mutant_midpoint_without_adjacency(monkeypatch):
    monkeypatch.setattr(C, "_fp16_midpoint_exempt",
                        _mutant_of(C._fp16_midpoint_exempt, "return adjacent & (", "return ("))
    _fails(tc.test_fp16_midpoint_adjacency)


def test_mutant_rederive_with_oracle_scale(monkeypatch):
    monkeypatch.setattr(C, "compare_quant",
                        _mutant_of(C.compare_quant, "sd = float(s_dev[r, c])", "sd = float(s_or[r, c])"))
    _fails(tc.test_compare_quant_scale_exempt_rederives_with_device_scale)


def test_mutant_no_exempt_budget(monkeypatch):
    monkeypatch.setattr(C, "compare_quant",
                        _mutant_of(C.compare_quant, "and rep[\"exempt_frac\"] < EXEMPT_BUDGET", ""))
    _fails(tc.test_compare_quant_code_window_and_budget)


def test_mutant_rms_over_the_matrix(monkeypatch):
    monkeypatch.setattr(C, "float_err",
                        _mutant_of(C.float_err, "np.mean(o * o, axis=1, keepdims=True)", "np.mean(o * o, keepdims=True)"))
    _fails(tc.test_float_err_row_rms_floor)


def test_mutant_no_rms_floor(monkeypatch):
    monkeypatch.setattr(C, "float_err", _mutant_of(C.float_err, "np.maximum(np.abs(o), rms)", "np.abs(o)"))
    _fails(tc.test_float_err_row_rms_floor)


def test_mutant_two_sided_untransposed_input_rotation(monkeypatch):
    """R_out W R_in (R_in not transposed) fails the brute-force loops."""
    from oracle import harp
    import test_oracle_harp_two_sided as t2

    def mutant(w, out_side, in_side):
        w = np.asarray(w, dtype=np.float64)
        return harp.rotation_matrix(w.shape[0], **out_side) @ w @ harp.rotation_matrix(w.shape[1], **in_side)
    monkeypatch.setattr(harp, "harp_two_sided", mutant)
    _fails(t2.test_two_sided_bruteforce, (3, 2), (2, 4))

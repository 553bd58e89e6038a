"""Pins of the QWHA initialisation oracle (AdaAlloc allocation and
selection, least-squares refinement): hand-worked allocations, brute-force
loops on tiny layers, the normal equations, and the special cases where the
refinement has a closed form."""
import numpy as np

from oracle import hadamard as H, qwha_init as QI, rtn


def small_layer(seed, d_out=6, n=64, bits=2, group=16):
    rng = np.random.default_rng(seed)
    w = 0.02 * rng.standard_t(3, size=(d_out, n))
    s = np.where(rng.integers(0, 2, n) == 1, -1.0, 1.0)
    codes, s16, *_ = rtn.rht_quantize(w, s, bits, group)
    return w, s, codes, s16


def test_error_coeffs_bruteforce():
    """F_dense[o][k] = sum_i (W - W_hat)[o][i] H[i][k] / sqrt(n), loops only."""
    w, s, codes, s16 = small_layer(0, d_out=3, n=32, bits=4, group=8)
    w_hat = rtn.dequantize_inverse(codes, s16, s, 4, 8, 32)
    f = QI.error_coeffs(w, codes, s16, s, 4, 8)
    want = np.zeros_like(f)
    for o in range(3):
        for k in range(32):
            acc = 0.0
            for i in range(32):
                h = -1.0 if bin(i & k).count("1") % 2 else 1.0
                acc += (w[o, i] - w_hat[o, i]) * h
            want[o, k] = acc / np.sqrt(32)
    assert np.allclose(f, want, atol=1e-14)


def test_error_coeffs_reconstruct_and_exact_layer():
    """Q(W) + F_dense Hn = W; a layer built as irht(q s) (one +-qmax per group
    keeps the scale) is quantised exactly, so its F_dense is zero."""
    w, s, codes, s16 = small_layer(1)
    f = QI.error_coeffs(w, codes, s16, s, 2, 16)
    assert np.allclose(rtn.dequantize_inverse(codes, s16, s, 2, 16, 64) + H.wht(f), w, atol=1e-15)
    rng = np.random.default_rng(2)
    q = rng.integers(-7, 8, size=(4, 64))
    q[:, ::32] = 7
    s16e = rng.uniform(0.01, 0.1, size=(4, 2)).astype(np.float16)
    we = rtn.dequantize_inverse(rtn.pack_codes(q, 4), s16e, s, 4, 32, 64)
    c2, s2, *_ = rtn.rht_quantize(we, s, 4, 32)
    assert np.array_equal(rtn.unpack_codes(c2, 4, 64), q)
    assert np.abs(QI.error_coeffs(we, c2, s2, s, 4, 32)).max() < 1e-12


def test_channel_errors_bruteforce():
    rng = np.random.default_rng(3)
    f = rng.standard_normal((3, 16))
    x = rng.standard_normal((5, 16))
    dw = f @ H.wht(np.eye(16))                  # rows F Hn
    want = [np.sqrt(sum(sum(x[t, i] * dw[o, i] for i in range(16)) ** 2 for t in range(5)))
            for o in range(3)]
    assert np.allclose(QI.channel_errors(x, f), want, atol=1e-12)


def test_allocate_hand_worked():
    # lam = 2 puts every channel strictly between floor and cap: exact shares
    assert QI.allocate([1, 2, 3, 4], 20, 2, 10).tolist() == [2, 4, 6, 8]
    # the first channel sits at the floor; the other three share 10 as 3.33 each,
    # one extra to the lowest index
    assert QI.allocate([0.1, 1, 1, 1], 12, 2, 10).tolist() == [2, 4, 3, 3]
    # a capped channel hands its excess to the others
    assert QI.allocate([100, 1, 1], 12, 1, 6).tolist() == [6, 3, 3]
    # no error anywhere: an even split
    assert QI.allocate([0, 0, 0, 0], 10, 1, 8).tolist() == [3, 3, 2, 2]


def test_allocate_invariants():
    rng = np.random.default_rng(4)
    for trial in range(20):
        m = int(rng.integers(5, 200))
        e = np.exp(rng.standard_normal(m))
        floor, cap = 3, 40
        p = int(rng.integers(floor * m, min(cap * m, 20 * m) + 1))
        n = QI.allocate(e, p, floor, cap)
        assert n.sum() == p and n.min() >= floor and n.max() <= cap
        lam = QI._water_level(e, p, floor, cap)
        real = np.clip(lam * e, floor, cap)
        assert np.all(np.abs(n - real) < 1.0 + 1e-9)
        # more error never gets fewer parameters
        order = np.argsort(e)
        assert np.all(np.diff(n[order]) >= 0)


def test_select_bruteforce():
    rng = np.random.default_rng(5)
    f = rng.standard_normal((7, 40))
    f[2, [3, 9, 17]] = 5.0             # ties at the top: the lower columns win
    f[2, 30] = -5.0
    budgets = np.array([1, 4, 3, 40, 0, 10, 2])
    row_ptr, cols = QI.select(f, budgets)
    assert row_ptr.tolist() == [0] + np.cumsum(budgets).tolist()
    for o in range(7):
        got = cols[row_ptr[o]:row_ptr[o + 1]].tolist()
        # brute force: repeatedly take the largest remaining magnitude, lowest index on ties
        left = list(range(40))
        picked = []
        for _ in range(budgets[o]):
            best = max(left, key=lambda k: (abs(f[o, k]), -k))
            picked.append(best)
            left.remove(best)
        assert got == sorted(picked)
    assert cols[row_ptr[2]:row_ptr[3]].tolist() == [3, 9, 17]


def test_refine_normal_equations_and_gain():
    """The refined values solve Z_E^T (Z_E c - t) = 0, and refining never does
    worse than copying the dense coefficients onto the support."""
    rng = np.random.default_rng(6)
    n, d_out, t = 32, 5, 48
    f = rng.standard_normal((d_out, n))
    x = rng.standard_normal((t, n))
    budgets = np.array([3, 8, 1, 5, 12])
    row_ptr, cols = QI.select(f, budgets)
    vals = QI.refine(x, f, row_ptr, cols)
    z = H.wht(x)
    target = x @ H.wht(f).T
    for o in range(d_out):
        e = cols[row_ptr[o]:row_ptr[o + 1]]
        c = vals[row_ptr[o]:row_ptr[o + 1]]
        grad = z[:, e].T @ (z[:, e] @ c - target[:, o])
        assert np.abs(grad).max() < 1e-9
    direct = f[np.repeat(np.arange(d_out), budgets), cols]
    assert QI.output_error(x, f, row_ptr, cols, vals) <= QI.output_error(x, f, row_ptr, cols, direct) + 1e-12


def test_refine_closed_forms():
    """Orthonormal calibration (x = Hn, so x Hn = I): refinement equals copying
    the dense coefficients.  The full support with enough tokens recovers the
    error exactly."""
    rng = np.random.default_rng(7)
    n = 16
    f = rng.standard_normal((4, n))
    hn = H.wht(np.eye(n))
    row_ptr, cols = QI.select(f, np.array([2, 5, 16, 7]))
    vals = QI.refine(hn, f, row_ptr, cols)
    assert np.allclose(vals, f[np.repeat(np.arange(4), [2, 5, 16, 7]), cols], atol=1e-12)
    x = rng.standard_normal((40, n))
    row_ptr, cols = QI.select(f, np.full(4, n))
    vals = QI.refine(x, f, row_ptr, cols)
    assert np.allclose(vals, f.reshape(-1), atol=1e-10)
    assert QI.output_error(x, f, row_ptr, cols, vals) < 1e-18


def test_calibration_gram_bruteforce():
    """G[a][b] = sum_t (sum_i x[t][i] H[i][a]) (sum_j x[t][j] H[j][b]) / n, loops only."""
    rng = np.random.default_rng(8)
    n, t = 8, 5
    x = rng.standard_normal((t, n))
    g = QI.calibration_gram(x)
    sgn = lambda i, k: -1.0 if bin(i & k).count("1") % 2 else 1.0
    for a in range(n):
        for b in range(n):
            acc = 0.0
            for r in range(t):
                za = sum(x[r, i] * sgn(i, a) for i in range(n))
                zb = sum(x[r, j] * sgn(j, b) for j in range(n))
                acc += za * zb
            assert abs(g[a, b] - acc / n) < 1e-12


def test_calibration_gram_normal_equations():
    """The quadratic form gives the channel errors; solving the normal
    equations on a support gives the least-squares values refine returns."""
    rng = np.random.default_rng(9)
    n, d_out, t = 32, 6, 64
    f = rng.standard_normal((d_out, n))
    x = rng.standard_normal((t, n))
    x[:, 5] *= 20.0                       # an outlier channel
    g = QI.calibration_gram(x)
    p = f @ g
    assert np.allclose(np.sqrt(np.einsum("oi,oi->o", p, f)), QI.channel_errors(x, f), rtol=1e-12)
    row_ptr, cols = QI.select(f, np.array([1, 4, 9, 16, 3, 32]))
    vals = QI.refine(x, f, row_ptr, cols)
    for o in range(d_out):
        e = cols[row_ptr[o]:row_ptr[o + 1]]
        c = np.linalg.solve(g[np.ix_(e, e)], p[o, e])
        assert np.allclose(c, vals[row_ptr[o]:row_ptr[o + 1]], rtol=1e-9, atol=1e-11)


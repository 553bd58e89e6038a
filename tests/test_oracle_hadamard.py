"""Pins of the oracle's Hadamard / WHT / RHT against what the pages and the
mathematics fix: Kronecker construction, H H^T = n I, involution, norm
preservation, closed forms, hand-worked examples, brute force, and the
textbook Sylvester routine in scipy."""
import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard as H
from golden_io import rows, ints


def kron_sylvester(n):
    """H_{2m} = [[H, H], [H, -H]] from H_1 = [1]: an independent construction."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024, 4096])
def test_popcount_equals_kronecker(n):
    assert np.array_equal(H.sylvester(n).astype(np.int64), kron_sylvester(n))


@pytest.mark.parametrize("n", [2, 8, 128, 2048])
def test_matches_scipy_hadamard(n):
    assert np.array_equal(H.sylvester(n), scipy.linalg.hadamard(n))


def test_golden_h4():
    got = H.sylvester(4)
    want = np.array([ints(r[0]) for r in rows("hadamard4.txt")])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n", [2, 16, 256, 1024])
def test_orthogonality_and_symmetry(n):
    h = H.sylvester(n).astype(np.int64)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))
    assert np.array_equal(h, h.T)
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)


def test_golden_worked_wht():
    for n, x, y in rows("wht_worked.txt"):
        x = np.array(ints(x), dtype=np.float64)
        y = np.array(ints(y), dtype=np.float64)
        assert np.array_equal(H.wht(x, normalize=False), y)
        assert np.allclose(H.wht(x), y / np.sqrt(int(n)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64])
def test_exact_dense_bruteforce_small(n):
    """Double loop over (i, j) with the popcount sign, integer inputs: equal
    bit for bit to the oracle's unnormalised product."""
    rng = np.random.default_rng(n)
    x = rng.integers(-(1 << 16), 1 << 16, size=(5, n))
    want = np.zeros((5, n), dtype=np.int64)
    for r in range(5):
        for i in range(n):
            acc = 0
            for j in range(n):
                acc += x[r, j] if bin(i & j).count("1") % 2 == 0 else -x[r, j]
            want[r, i] = acc
    got = H.wht(x.astype(np.float64), normalize=False)
    assert np.array_equal(got, want.astype(np.float64))


@pytest.mark.parametrize("n", [4, 64, 512, 4096])
def test_involution_and_norm(n):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, n))
    y = H.wht(x)
    rms = np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    assert np.max(np.abs(H.wht(y) - x) / rms) < 1e-12
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


@pytest.mark.parametrize("n", [8, 1024])
def test_closed_forms(n):
    e0 = np.zeros(n); e0[0] = 1.0
    ones = np.ones(n)
    assert np.allclose(H.wht(e0), ones / np.sqrt(n), atol=1e-15)
    assert np.allclose(H.wht(ones), np.sqrt(n) * e0, atol=1e-12)
    k = n // 2 + 3
    ek = np.zeros(n); ek[k] = 1.0
    j = np.arange(n)
    walsh = np.array([(-1) ** bin(k & jj).count("1") for jj in j], dtype=np.float64)
    assert np.array_equal(H.wht(ek, normalize=False), walsh)
    rng = np.random.default_rng(3)
    a, b = rng.standard_normal(n), rng.standard_normal(n)
    assert np.allclose(H.wht(2.5 * a - b), 2.5 * H.wht(a) - H.wht(b), atol=1e-12)


def test_normalisation_power_of_four_exact():
    """For n = 4^k the factor 1/sqrt(n) is a power of two: integer inputs give
    exactly (H x) / 2^k."""
    rng = np.random.default_rng(5)
    for n, k in [(4, 1), (16, 2), (64, 3), (4096, 6)]:
        x = rng.integers(-1000, 1000, size=(3, n)).astype(np.float64)
        assert np.array_equal(H.wht(x), H.wht(x, normalize=False) / 2.0 ** k)


def test_sign_mask_golden():
    for words, n, s in rows("sign_mask.txt"):
        w = np.array([int(v, 16) for v in words.split()], dtype=np.uint32)
        want = np.array(ints(s), dtype=np.float64)
        assert want.size == int(n)
        assert np.array_equal(H.signs_from_bits(w, int(n)), want)


def test_sign_diagonal_orthogonality():
    rng = np.random.default_rng(7)
    n = 256
    s = 1.0 - 2.0 * rng.integers(0, 2, n)
    assert np.array_equal(s * s, np.ones(n))
    m = H.rht(np.eye(n), s)              # rows: (Hn S e_i)^T, i.e. (Hn S)^T
    assert np.allclose(m @ m.T, np.eye(n), atol=1e-13)
    x = rng.standard_normal((4, n))
    assert np.allclose(H.irht(H.rht(x, s), s), x, atol=1e-13)
    # S Hn != Hn S in general: the forward places the signs before the transform
    assert not np.allclose(H.rht(x, s), H.wht(x) * s)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        H.sylvester(12)

"""Pins of the oracle's online-RHT low-bit product: a brute-force element
loop on a tiny layer, the rotated-basis identity y = q s . rht(x), and exact
layers built from chosen codes."""
import numpy as np

from oracle import gemv, hadamard as H, rtn


def brute(x, q, s16, signs, group):
    """y[t][o] = sum_i x[t][i] sum_k s_i Hn[i][k] q[o][k] s16[o][k // g], loops only."""
    t_, n = x.shape
    o_ = q.shape[0]
    y = np.zeros((t_, o_))
    for o in range(o_):
        for i in range(n):
            w = 0.0
            for k in range(n):
                h = -1.0 if bin(i & k).count("1") % 2 else 1.0
                w += h * q[o, k] * float(s16[o, k // group])
            w *= signs[i] / np.sqrt(n)
            for t in range(t_):
                y[t, o] += x[t, i] * w
    return y


def test_gemv_bruteforce_tiny():
    rng = np.random.default_rng(0)
    n, o, g, bits = 64, 3, 16, 4
    q = rng.integers(-7, 8, size=(o, n))
    s16 = rng.uniform(0.01, 0.1, size=(o, n // g)).astype(np.float16)
    signs = np.where(rng.integers(0, 2, n) == 1, -1.0, 1.0)
    x = rng.standard_normal((2, n))
    codes = rtn.pack_codes(q, bits)
    got = gemv.rht_gemv(x, codes, s16, signs, bits, g, n)
    assert np.allclose(got, brute(x, q, s16, signs, g), atol=1e-12)


def test_gemv_rotated_basis_identity():
    """(S Hn y_hat) . x = y_hat . (Hn S x): the product in the code basis with
    the rotated activation, which is what an online-rotation kernel computes."""
    rng = np.random.default_rng(1)
    n, o, g, bits = 1024, 5, 64, 2
    q = rng.integers(-1, 2, size=(o, n))
    s16 = rng.uniform(0.01, 0.1, size=(o, n // g)).astype(np.float16)
    signs = np.where(rng.integers(0, 2, n) == 1, -1.0, 1.0)
    x = rng.standard_normal((3, n))
    y_hat = rtn.dequantize(rtn.pack_codes(q, bits), s16, bits, g, n)
    want = H.rht(x, signs) @ y_hat.T
    assert np.allclose(gemv.rht_gemv(x, rtn.pack_codes(q, bits), s16, signs, bits, g, n), want, atol=1e-10)


def test_gemv_of_an_exact_layer():
    """A weight built as W = irht(q s) is represented exactly by (q, s), so the
    product equals x W^T, and quantising W gives back the same codes."""
    rng = np.random.default_rng(2)
    n, o, g, bits = 256, 4, 32, 4
    q = rng.integers(-7, 8, size=(o, n))
    q[:, ::g] = 7                                   # one +-qmax per group keeps the scale
    s16 = rng.uniform(0.01, 0.1, size=(o, n // g)).astype(np.float16)
    signs = np.where(rng.integers(0, 2, n) == 1, -1.0, 1.0)
    w = H.irht((q.reshape(o, n // g, g) * s16.astype(np.float64)[:, :, None]).reshape(o, n), signs)
    x = rng.standard_normal((2, n))
    got = gemv.rht_gemv(x, rtn.pack_codes(q, bits), s16, signs, bits, g, n)
    assert np.allclose(got, x @ w.T, atol=1e-10)
    q2, s2, _, _ = rtn.quantize_rtn(H.rht(w, signs), bits, g)
    assert np.array_equal(q2, q) and np.array_equal(s2, s16)

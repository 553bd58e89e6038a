"""Pins of the oracle's RTN quantiser, packing and dequant-inverse: brute
force over every level, invariants, hand-derived packed bytes, and a
grid-constructed round trip whose codes are known before quantising."""
import numpy as np
import pytest

from oracle import rtn, hadamard as H
from golden_io import rows, ints


def brute_codes(y, s, qmax):
    """argmin over every level of |y - q s|, ties to the even level."""
    levels = np.arange(-qmax, qmax + 1)
    out = np.empty(y.shape, dtype=np.int64)
    for idx, yy in np.ndenumerate(y):
        err = np.abs(yy - levels * s)
        best = np.flatnonzero(err == err.min())
        if best.size > 1:
            best = best[levels[best] % 2 == 0]
        out[idx] = levels[best[0]]
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rtn_bruteforce(bits):
    rng = np.random.default_rng(bits)
    y = rng.standard_normal((6, 32)) * np.exp(rng.standard_normal((6, 1)))
    g = 8
    q, s16, v, s_pre = rtn.quantize_rtn(y, bits, g)
    qm = (1 << (bits - 1)) - 1
    for r in range(6):
        for c in range(32 // g):
            sl = slice(c * g, c * g + g)
            s = float(s16[r, c])
            assert np.array_equal(q[r, sl], brute_codes(y[r, sl], s, qm))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rtn_invariants(bits):
    rng = np.random.default_rng(10 + bits)
    y = rng.standard_t(3, size=(8, 256))
    g = 64
    q, s16, v, s_pre = rtn.quantize_rtn(y, bits, g)
    qm = (1 << (bits - 1)) - 1
    s = s16.astype(np.float64)
    yg = y.reshape(8, -1, g)
    qg = q.reshape(8, -1, g).astype(np.float64)
    # scale is the fp16 nearest to absmax / qmax
    a = np.abs(yg).max(axis=2)
    assert np.allclose(s_pre, a / qm, rtol=0, atol=0)
    lo = np.nextafter(s16, np.float16(0)).astype(np.float64)
    hi = np.nextafter(s16, np.float16(np.inf)).astype(np.float64)
    assert np.all(np.abs(s - s_pre) <= np.abs(lo - s_pre))
    assert np.all(np.abs(s - s_pre) <= np.abs(hi - s_pre))
    # every element within half a step; absmax element maps to +-qmax
    assert np.all(np.abs(yg - qg * s[:, :, None]) <= s[:, :, None] / 2 * (1 + 1e-12))
    amax = np.abs(yg).argmax(axis=2)
    top = np.take_along_axis(qg, amax[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(top) == qm)
    # codes in range, and re-quantising q*s with s returns q
    assert np.abs(q).max() <= qm
    q2 = np.clip(np.rint((qg * s[:, :, None]) / s[:, :, None]), -qm, qm)
    assert np.array_equal(q2, qg)


def test_zero_group():
    y = np.zeros((1, 16)); y[0, 8:] = np.arange(8) - 3.5
    q, s16, v, s_pre = rtn.quantize_rtn(y, 4, 8)
    assert s16[0, 0] == 0 and np.all(q[0, :8] == 0)
    assert s16[0, 1] > 0


def test_packing_golden():
    for bits, codes, by in rows("packing.txt"):
        bits = int(bits)
        q = np.array([ints(codes)])
        want = np.array([[int(b, 16) for b in by.split()]], dtype=np.uint8)
        assert np.array_equal(rtn.pack_codes(q, bits), want)
        assert np.array_equal(rtn.unpack_codes(want, bits, q.shape[1]), q)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_roundtrip(bits):
    qm = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(bits)
    q = rng.integers(-qm - 1, qm + 1, size=(5, 64))   # includes the unused -2^(b-1)
    packed = rtn.pack_codes(q, bits)
    assert packed.shape == (5, 64 * bits // 8)
    assert np.array_equal(rtn.unpack_codes(packed, bits, 64), q)


@pytest.mark.parametrize("bits,g,n", [(4, 128, 1024), (2, 64, 512), (3, 32, 256)])
def test_grid_constructed_roundtrip(bits, g, n):
    """Codes q (one +-qmax per group) and fp16 scales chosen first; x is the
    inverse RHT of q*s.  Quantising x must give back exactly q and s, and
    dequant-inverse must give back x."""
    rng = np.random.default_rng(100 + bits)
    rows_ = 6
    qm = (1 << (bits - 1)) - 1
    q = rng.integers(-qm, qm + 1, size=(rows_, n // g, g))
    pos = rng.integers(0, g, size=(rows_, n // g))
    sign = rng.choice([-1, 1], size=(rows_, n // g))
    np.put_along_axis(q, pos[:, :, None], (sign * qm)[:, :, None], axis=2)
    s16 = (np.exp(rng.uniform(-5, 0, size=(rows_, n // g)))).astype(np.float16)
    y = (q * s16.astype(np.float64)[:, :, None]).reshape(rows_, n)
    s = 1.0 - 2.0 * rng.integers(0, 2, n)
    x = H.irht(y, s)
    codes, s_out, q_out, v, s_pre, y_back = rtn.rht_quantize(x, s, bits, g)
    assert np.array_equal(q_out, q.reshape(rows_, n))
    assert np.array_equal(s_out.view(np.uint16), s16.view(np.uint16))
    x_hat = rtn.dequantize_inverse(codes, s_out, s, bits, g, n)
    assert np.allclose(x_hat, x, atol=1e-12)


def test_rejects_bad_bits():
    with pytest.raises(ValueError):
        rtn.quantize_rtn(np.zeros((1, 8)), 5, 8)

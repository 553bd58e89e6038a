"""Sylvester Hadamard matrix, orthonormal WHT and the randomized Hadamard
transform, all by explicit dense products in fp64.  Test infrastructure only.

[QWHA] 2.1: the WHT kernel has only +-1 entries.  [HARP] 2.2: the base
mixer for power-of-two radices is the normalised Sylvester Hadamard.
[HARP] 1: the RHT is a fixed random sign diagonal followed by the Hadamard
transform, fast and exactly orthogonal.
"""

import numpy as np

_CHUNK = 1024  # rows per dense product (bounds the fp64 temporary)


def is_pow2(n):
    return n >= 1 and (n & (n - 1)) == 0


def sylvester(n):
    """H[i, j] = (-1)^popcount(i & j), int8, n x n.

    Reading: Sylvester ("natural") ordering, the matrix [HARP] 2.2 names;
    not the sequency-ordered Walsh matrix.
    """
    if not is_pow2(n):
        raise ValueError(f"n={n} is not a power of two")
    i = np.arange(n, dtype=np.int64)
    # np.bitwise_count returns uint8: widen before 1 - 2*parity.
    parity = np.bitwise_count(i[:, None] & i[None, :]).astype(np.int64) & 1
    return (1 - 2 * parity).astype(np.int8)


def wht(x, normalize=True):
    """Row-wise WHT: Y = X H (H symmetric), times n^-1/2 when normalize.

    Reading: the orthonormal H/sqrt(n) throughout, so the transform is its
    own inverse; normalize=False gives the raw +-1 product.
    """
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 1
    x2 = x.reshape(1, -1) if squeeze else x
    n = x2.shape[1]
    h = sylvester(n).astype(np.float64)
    out = np.empty_like(x2)
    for r in range(0, x2.shape[0], _CHUNK):
        out[r:r + _CHUNK] = x2[r:r + _CHUNK] @ h
    if normalize:
        out *= 1.0 / np.sqrt(n)
    return out.reshape(x.shape)


def signs_from_bits(bits, n):
    """Unpack the sign diagonal s in {+1,-1}^n from a uint32 bitmask.

    Reading: bit j (LSB first within 32-bit word j // 32) set means s_j = -1.
    """
    bits = np.asarray(bits, dtype=np.uint32)
    if bits.size * 32 < n:
        raise ValueError("bitmask too short")
    j = np.arange(n)
    b = (bits[j >> 5] >> (j & 31).astype(np.uint32)) & np.uint32(1)
    return 1.0 - 2.0 * b.astype(np.float64)


def rht(x, s):
    """Forward RHT along the last axis: Hn (S x).  [HARP] 1.

    Reading: signs first, then the orthonormal transform; one S per layer,
    shared by every row.
    """
    return wht(np.asarray(x, dtype=np.float64) * s)


def irht(y, s):
    """Inverse RHT: S (Hn y), since Hn and S are both involutions."""
    return wht(y) * s

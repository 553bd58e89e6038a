"""Per-group round-to-nearest quantiser on RHT-rotated rows, bit packing,
and dequantisation followed by the inverse RHT.  Test infrastructure only.

The pages name 2-4 bit weights after incoherence processing ([HARP] 1, 4;
[QWHA] 4) but leave the quantiser to other systems; every step below is a
reading, stated where it is made:

  * symmetric absmax per group of g consecutive transformed coordinates,
    qmax = 2^(b-1) - 1, codes in [-qmax, qmax] (the most negative
    two's-complement code is never produced);
  * scale s_pre = absmax / qmax, stored as IEEE fp16 (round to nearest
    even), and the codes are taken with the *stored* scale so that
    dequantisation reproduces what was quantised;
  * rounding half to even; an all-zero group has scale 0 and codes 0;
  * codes are packed as a little-endian bit stream per row: code i sits in
    bits [b*i, b*i + b) of the row's bytes, least significant bit first,
    in two's complement.
"""

import numpy as np

from .hadamard import rht, irht


def qmax_of(bits):
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    return (1 << (bits - 1)) - 1


def quantize_rtn(y, bits, group):
    """Quantise already-rotated rows y [rows, n] (fp64).

    Returns (q int8 [rows, n], s16 float16 [rows, n/g], v fp64 [rows, n],
    s_pre fp64 [rows, n/g]); v = y / s16 is the pre-rounding value and
    s_pre the pre-rounding scale, both kept for the parity exemption rules.
    """
    y = np.asarray(y, dtype=np.float64)
    rows, n = y.shape
    if n % group:
        raise ValueError("group must divide n")
    qm = qmax_of(bits)
    yg = y.reshape(rows, n // group, group)
    a = np.abs(yg).max(axis=2)
    s_pre = a / qm
    s16 = s_pre.astype(np.float16)          # fp64 -> fp16, nearest even
    s = s16.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s > 0, yg / np.where(s > 0, s, 1.0), 0.0)
    q = np.clip(np.rint(v), -qm, qm).astype(np.int8)
    return q.reshape(rows, n), s16, v.reshape(rows, n), s_pre


def pack_codes(q, bits):
    """Two's-complement codes [rows, n] -> uint8 [rows, n*bits/8]."""
    q = np.asarray(q, dtype=np.int64)
    rows, n = q.shape
    if (n * bits) % 8:
        raise ValueError("row does not fill whole bytes")
    u = q & ((1 << bits) - 1)
    bitplanes = (u[:, :, None] >> np.arange(bits)) & 1   # LSB first
    return np.packbits(bitplanes.reshape(rows, n * bits).astype(np.uint8),
                       axis=1, bitorder="little")


def unpack_codes(codes, bits, n):
    """uint8 [rows, n*bits/8] -> signed codes int64 [rows, n]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    bitplanes = np.unpackbits(codes, axis=1, bitorder="little")[:, :n * bits]
    bitplanes = bitplanes.reshape(rows, n, bits).astype(np.int64)
    u = (bitplanes << np.arange(bits)).sum(axis=2)
    return np.where(u >= (1 << (bits - 1)), u - (1 << bits), u)


def rht_quantize(w, s, bits, group):
    """Full forward path: y = Hn(S w), then quantize_rtn and pack.

    Returns (codes uint8, s16 float16, q, v, s_pre, y).
    """
    y = rht(w, s)
    q, s16, v, s_pre = quantize_rtn(y, bits, group)
    return pack_codes(q, bits), s16, q, v, s_pre, y


def dequantize(codes, s16, bits, group, n):
    """Codes and fp16 scales -> y_hat = q * s (fp64)."""
    q = unpack_codes(codes, bits, n).astype(np.float64)
    rows = q.shape[0]
    sc = np.asarray(s16, dtype=np.float16).astype(np.float64)
    return (q.reshape(rows, n // group, group) * sc[:, :, None]).reshape(rows, n)


def dequantize_inverse(codes, s16, s, bits, group, n):
    """Dequantise then invert the RHT: x_hat = S Hn (q * s)."""
    return irht(dequantize(codes, s16, bits, group, n), s)

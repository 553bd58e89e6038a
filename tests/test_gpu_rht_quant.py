"""GPU parity of rht_quantize_rtn / rht_dequantize_inverse against the
oracle: codes bit-exact up to the boundary exemption, scales bit-exact up to
the fp16-midpoint exemption, dequantised floats within tolerance."""
import numpy as np
import pytest
import torch

from oracle import hadamard as H, rtn, compare
from wht_adapters_amd import synth
from gpu_util import dev, mask_dev, host64, codes_host, scales_host, write_report, merge_reports

pytestmark = pytest.mark.gpu


def W():
    from wht_adapters_amd import whtq
    return whtq


def check_quant(w_dev, mask, bits, g, rows_sel=None):
    """Quantise on the GPU and compare (optionally only rows_sel) with the oracle."""
    n = w_dev.shape[1]
    codes, scales = W().rht_quantize_rtn(w_dev, mask_dev(mask), bits, g)
    torch.cuda.synchronize()
    w64 = host64(w_dev if rows_sel is None else w_dev[rows_sel])
    c = codes_host(codes if rows_sel is None else codes[rows_sel])
    sc = scales_host(scales if rows_sel is None else scales[rows_sel])
    s = H.signs_from_bits(mask, n)
    y = H.rht(w64, s)
    q_or, s16, v, s_pre = rtn.quantize_rtn(y, bits, g)
    q_dev = rtn.unpack_codes(c, bits, n)
    rep = compare.compare_quant(q_dev, sc, y, s16, q_or, v, s_pre, bits, g)
    assert rep["ok"], rep
    return codes, scales, rep


@pytest.mark.parametrize("logn", range(6, 14))
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quant_all_sizes(logn, bits):
    n = 1 << logn
    rng = np.random.default_rng(logn * 10 + bits)
    w = dev(0.02 * rng.standard_t(3, size=(21, n)), torch.bfloat16)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    for g in sorted({8, 32, 64, min(128, n), min(256, n)}):
        check_quant(w, mask, bits, g)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_quant_4096_int4_strided_rows(dt):
    """n = 4096 with 4-bit codes and groups of 64..256 on the matrix-core
    kernel: bf16 and fp16 rows read through a row stride wider than the row,
    and a row count that is not a multiple of anything the launch uses."""
    rng = np.random.default_rng(4096 + (dt == torch.float16))
    base = dev(0.02 * rng.standard_t(3, size=(517, 4096 + 72)), dt)
    w = base[:, 8:4096 + 8]
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, 4096))
    for g in (64, 128, 256):
        check_quant(w, mask, 4, g)


@pytest.mark.parametrize("dt", [torch.float32, torch.float16])
def test_quant_other_input_dtypes(dt):
    rng = np.random.default_rng(5)
    n = 1024
    w = dev(rng.standard_normal((33, n)), dt)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    check_quant(w, mask, 4, 128)
    check_quant(w, mask, 2, 64)


def test_quant_no_signs_and_zero_rows():
    n = 512
    w = torch.zeros((4, n), dtype=torch.bfloat16, device="cuda:0")
    w[1] = torch.linspace(-1, 1, n)
    codes, scales = W().rht_quantize_rtn(w, None, 4, 64)
    torch.cuda.synchronize()
    assert torch.all(codes[0] == 0) and torch.all(scales[0] == 0)
    q_or, s16, v, s_pre = rtn.quantize_rtn(H.wht(host64(w)), 4, 64)
    rep = compare.compare_quant(rtn.unpack_codes(codes_host(codes), 4, n), scales_host(scales),
                                H.wht(host64(w)), s16, q_or, v, s_pre, 4, 64)
    assert rep["ok"], rep


@pytest.mark.parametrize("bits,g,n", [(4, 128, 4096), (2, 64, 8192), (3, 32, 1024), (4, 8, 256)])
def test_grid_constructed_roundtrip(bits, g, n):
    """Codes and scales fixed first; x = irht(q*s) in fp64 rounded to fp32.
    The GPU must return exactly q, s (up to the scale exemption), and its
    dequant-inverse must give back x."""
    rng = np.random.default_rng(100 + bits + n)
    rows = 16
    qm = (1 << (bits - 1)) - 1
    q = rng.integers(-qm, qm + 1, size=(rows, n // g, g))
    pos = rng.integers(0, g, size=(rows, n // g))
    np.put_along_axis(q, pos[:, :, None], (rng.choice([-1, 1], (rows, n // g)) * qm)[:, :, None], 2)
    s16 = np.exp(rng.uniform(-5, 0, size=(rows, n // g))).astype(np.float16)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    sgn = H.signs_from_bits(mask, n)
    x = H.irht((q * s16.astype(np.float64)[:, :, None]).reshape(rows, n), sgn).astype(np.float32)
    codes, scales = W().rht_quantize_rtn(dev(x), mask_dev(mask), bits, g)
    torch.cuda.synchronize()
    q_dev = rtn.unpack_codes(codes_host(codes), bits, n)
    assert np.array_equal(q_dev, q.reshape(rows, n))
    assert np.array_equal(scales_host(scales).view(np.uint16), s16.view(np.uint16))
    back = W().rht_dequantize_inverse(codes, scales, mask_dev(mask), bits, g, n, out_dtype=torch.float32)
    assert compare.float_err(host64(back), x.astype(np.float64))[0] <= 1e-5


@pytest.mark.parametrize("logn", range(6, 14))
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
def test_dequant_inverse_parity(logn, bits, odt):
    n = 1 << logn
    rng = np.random.default_rng(logn + 50 * bits)
    w = dev(0.02 * rng.standard_t(3, size=(11, n)), torch.bfloat16)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    g = min(128, n)
    codes, scales = W().rht_quantize_rtn(w, mask_dev(mask), bits, g)
    out = W().rht_dequantize_inverse(codes, scales, mask_dev(mask), bits, g, n, out_dtype=odt)
    want = rtn.dequantize_inverse(codes_host(codes), scales_host(scales), H.signs_from_bits(mask, n),
                                  bits, g, n)
    tol = 1e-5 if odt == torch.float32 else 2e-2
    assert compare.float_err(host64(out), want)[0] <= tol


@pytest.mark.parametrize("bits,g,logn", [(4, 128, 12), (4, 64, 13), (3, 32, 10), (4, 16, 8)])  # (INT2 cannot overflow)
def test_quant_subnormal_scales_clip(bits, g, logn):
    # rows so small that the fp16 scales are subnormal: rounding can shrink
    # a scale enough that the group maximum maps past qmax + 1/2, where the
    # codes must be clipped to +-qmax
    n = 1 << logn
    rng = np.random.default_rng(90 + bits)
    sig = np.exp(rng.uniform(np.log(2e-8), np.log(2e-6), size=(24, 1)))
    w = dev(sig * rng.standard_normal((24, n)), torch.bfloat16)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    y = H.rht(host64(w), H.signs_from_bits(mask, n))
    _, _, v, _ = rtn.quantize_rtn(y, bits, g)
    assert (np.rint(np.abs(v)) > rtn.qmax_of(bits)).sum() > 0  # the case occurs
    check_quant(w, mask, bits, g)


@pytest.mark.parametrize("bits,g,logn", [(4, 128, 12), (2, 64, 13), (3, 32, 10)])
def test_quant_extreme_magnitudes(bits, g, logn):
    """bf16 rows whose fp16 scales overflow to inf (codes 0), a row whose
    groups straddle that threshold (max |y| near 65520 qmax), a row near
    1e4, a normal row, and rows of 1e-30 and 1e-38 (scales 0, codes 0):
    codes and scales follow the oracle bit for bit like any other row."""
    n = 1 << logn
    rng = np.random.default_rng(7 + bits)
    edge = 65520.0 * rtn.qmax_of(bits) / 3.0  # about 3 sigma of a group at the overflow threshold
    sig = np.array([1e6, 3e5, edge, 1e4, 1.0, 1e-30, 1e-38])[:, None]
    w = dev(sig * rng.standard_normal((7, n)), torch.bfloat16)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    codes, scales, _ = check_quant(w, mask, bits, g)
    sc = scales_host(scales).astype(np.float32)
    assert np.isinf(sc[0]).all() and (np.isinf(sc[2]).any() and np.isfinite(sc[2]).any())
    assert (sc[5:] == 0).all()


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("logn,g", [(6, 64), (10, 32), (12, 64), (12, 128), (13, 64), (13, 256), (11, 8)])
def test_dequant_arbitrary_codes(logn, g, bits):
    # every code value, including -2^(b-1), which the quantiser never emits
    n = 1 << logn
    rng = np.random.default_rng(7 * logn + bits + g)
    rows = 13
    codes = torch.from_numpy(rng.integers(0, 256, size=(rows, n * bits // 8), dtype=np.uint8)).to("cuda:0")
    sc = rng.uniform(1e-3, 2.0, size=(rows, n // g)).astype(np.float16)
    scales = torch.from_numpy(sc).to("cuda:0")
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    out = W().rht_dequantize_inverse(codes, scales, mask_dev(mask), bits, g, n, out_dtype=torch.float32)
    want = rtn.dequantize_inverse(codes_host(codes), sc, H.signs_from_bits(mask, n), bits, g, n)
    assert compare.float_err(host64(out), want)[0] <= 1e-5


def _full_quant_report(w, signs, bits, g, chunk):
    """Quantise the whole matrix on the GPU and compare every row with the
    oracle, chunk by chunk; returns (codes, scales, merged report)."""
    n = w.shape[1]
    codes, scales = W().rht_quantize_rtn(w, mask_dev(signs), bits, g)
    torch.cuda.synchronize()
    s = H.signs_from_bits(signs, n)
    reps = []
    for r0 in range(0, w.shape[0], chunk):
        sl = slice(r0, min(r0 + chunk, w.shape[0]))
        y = H.rht(host64(w[sl]), s)
        q_or, s16, v, s_pre = rtn.quantize_rtn(y, bits, g)
        q_dev = rtn.unpack_codes(codes_host(codes[sl]), bits, n)
        reps.append(compare.compare_quant(q_dev, scales_host(scales[sl]), y, s16, q_or, v, s_pre, bits, g))
        print(f"  rows {sl.start}..{sl.stop}: {reps[-1]}", flush=True)
    return codes, scales, merge_reports(reps)


def _full_inverse_err(codes, scales, signs, bits, g, n, chunk):
    """Max scaled error of the GPU inverse (bf16 out) over every row."""
    out = W().rht_dequantize_inverse(codes, scales, mask_dev(signs), bits, g, n)
    s = H.signs_from_bits(signs, n)
    errs, rowws = [], []
    for r0 in range(0, codes.shape[0], chunk):
        sl = slice(r0, min(r0 + chunk, codes.shape[0]))
        want = rtn.dequantize_inverse(codes_host(codes[sl]), scales_host(scales[sl]), s, bits, g, n)
        e, rw = compare.float_err(host64(out[sl]), want)
        errs.append(e)
        rowws.append(rw)
        print(f"  inverse rows {sl.start}..{sl.stop}: max scaled error {e:.3e}", flush=True)
    return max(errs), max(rowws)


def test_full_config_int4_g128_4096():
    """4096 x 4096 Student-t weights with outlier columns, INT4, g = 128:
    every code and scale, and every row of the inverse."""
    d = synth.rht_int4_g128()
    w = dev(d["w"])
    codes, scales, rep = _full_quant_report(w, d["signs"], 4, 128, 4096)
    err, roww = _full_inverse_err(codes, scales, d["signs"], 4, 128, 4096, 4096)
    rep.update(inverse_max_scaled_err=err, inverse_max_row_rel_err=roww, config="rht_int4_g128_4096x4096")
    write_report("parity_rht_int4_g128_4096x4096", rep)
    assert rep["ok"], rep
    assert err <= 2e-2


def test_full_config_int2_g64_28672x8192():
    """28672 x 8192 INT2 g64 at full size: every code and scale of every row
    against the oracle (in row chunks), and every row of the inverse."""
    d = synth.rht_int2_g64()
    w = dev(d["w"])
    codes, scales, rep = _full_quant_report(w, d["signs"], 2, 64, 7168)
    del w
    err, roww = _full_inverse_err(codes, scales, d["signs"], 2, 64, 8192, 7168)
    rep.update(inverse_max_scaled_err=err, inverse_max_row_rel_err=roww, config="rht_int2_g64_28672x8192")
    write_report("parity_rht_int2_g64_28672x8192", rep)
    assert rep["ok"], rep
    assert err <= 2e-2

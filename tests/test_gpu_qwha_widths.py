"""GPU parity of the three QWHA calls at input widths other than 4096:
zero extension below 4096 and the top-bit split at 8192 (forward y, dx and
the value gradient dc), against the dense fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import compare, hadamard as H, qwha
from wht_adapters_amd import synth
from gpu_util import write_report, dev, host64

pytestmark = pytest.mark.gpu
TOL_BF16 = 2e-2
TOL_F32 = 1e-5


def W():
    from wht_adapters_amd import whtq
    return whtq


def random_csr(rng, d_out, d_in, nnz, empty_rows=(), empty_cols=()):
    rows = rng.integers(0, d_out, nnz)
    cols = rng.integers(0, d_in, nnz)
    keep = ~np.isin(rows, empty_rows) & ~np.isin(cols, empty_cols)
    key = np.unique(rows[keep] * d_in + cols[keep])
    rows, cols = key // d_in, key % d_in
    rp = np.r_[0, np.cumsum(np.bincount(rows, minlength=d_out))].astype(np.int32)
    vals = synth.to_bf16(0.1 * rng.standard_normal(rows.size))
    return rp, cols.astype(np.int32), vals


def dx_gpu(dy, rp, ci, vals, d_in):
    t_rp, t_ci, t_pm = W().qwha_csr_transpose(rp, ci, d_in)
    t_v = W().qwha_permute_values(dev(vals), dev(t_pm))
    return W().qwha_adapter_backward_input(dev(dy), dev(t_rp), dev(t_ci), t_v, d_in)


def dc_err(got, want):
    return compare.float_err(np.asarray(got, np.float64)[None, :], np.asarray(want)[None, :])[0]


CASES = [(64, 37, 100, 900), (256, 9, 4096, 20000), (1024, 130, 700, 30000), (2048, 37, 4096, 60000),
         (2048, 1, 8, 40), (8192, 37, 1000, 50000), (8192, 13, 4096, 120000), (8192, 130, 37, 3000)]


@pytest.mark.parametrize("d_in,tokens,d_out,nnz", CASES)
def test_forward(d_in, tokens, d_out, nnz):
    rng = np.random.default_rng(d_in + tokens)
    x = synth.to_bf16(rng.standard_normal((tokens, d_in)))
    rp, ci, v = random_csr(rng, d_out, d_in, nnz, empty_rows=(0,))
    y = W().qwha_adapter_forward(dev(x), dev(rp), dev(ci), dev(v), d_out)
    want = qwha.qwha_forward(synth.bf16_to_f64(x), rp, ci, synth.bf16_to_f64(v), d_out)
    err, _ = compare.float_err(host64(y), want)
    assert err <= TOL_BF16, err
    assert not host64(y)[:, 0].any()


@pytest.mark.parametrize("d_in,tokens,d_out,nnz", CASES)
def test_backward_input(d_in, tokens, d_out, nnz):
    rng = np.random.default_rng(300 + d_in + tokens)
    dy = synth.to_bf16(rng.standard_normal((tokens, d_out)))
    rp, ci, v = random_csr(rng, d_out, d_in, nnz, empty_cols=(1,))
    dx = dx_gpu(dy, rp, ci, v, d_in)
    assert tuple(dx.shape) == (tokens, d_in)
    want = qwha.qwha_backward_input(synth.bf16_to_f64(dy), rp, ci, synth.bf16_to_f64(v), d_in)
    err, _ = compare.float_err(host64(dx), want)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("d_in,tokens,d_out,nnz", CASES)
def test_grad_values(d_in, tokens, d_out, nnz):
    rng = np.random.default_rng(600 + d_in + tokens)
    x = synth.to_bf16(rng.standard_normal((tokens, d_in)))
    dy = synth.to_bf16(rng.standard_normal((tokens, d_out)))
    rp, ci, _ = random_csr(rng, d_out, d_in, nnz)
    dc = W().qwha_adapter_grad_values(dev(x), dev(dy), dev(rp), dev(ci))
    want = qwha.qwha_grad_values(synth.bf16_to_f64(x), synth.bf16_to_f64(dy), rp, ci)
    err = dc_err(host64(dc), want)
    assert err <= TOL_F32, err


@pytest.mark.parametrize("d_in", [64, 2048, 8192])
def test_single_entry_closed_form(d_in):
    """One entry at (o, k) of F: y[t][o] = F[o][k] (Hn x_t)[k],
    dx[t] = F[o][k] dy[t][o] Hn e_k, dc = sum_t dy[t][o] (Hn x_t)[k], with
    the column k of the Sylvester matrix written out (no transform)."""
    rng = np.random.default_rng(d_in)
    tokens, d_out, o = 21, 10, 6
    k = d_in - 3
    x = synth.to_bf16(rng.standard_normal((tokens, d_in)))
    dy = synth.to_bf16(rng.standard_normal((tokens, d_out)))
    rp = np.r_[np.zeros(o + 1, np.int32), np.ones(d_out - o, np.int32)]
    ci = np.array([k], np.int32)
    v = synth.to_bf16(np.array([0.75]))
    hk = H.sylvester(d_in)[:, k].astype(np.float64) / np.sqrt(d_in)
    z = synth.bf16_to_f64(x) @ hk
    y = host64(W().qwha_adapter_forward(dev(x), dev(rp), dev(ci), dev(v), d_out))
    assert np.abs(y[:, o] - 0.75 * z).max() <= 1e-2 * np.abs(z).max()
    assert not np.delete(y, o, axis=1).any()
    dx = host64(dx_gpu(dy, rp, ci, v, d_in))
    want_dx = 0.75 * synth.bf16_to_f64(dy)[:, o:o + 1] * hk[None, :]
    assert np.abs(dx - want_dx).max() <= 1e-2 * np.abs(want_dx).max()
    dc = host64(W().qwha_adapter_grad_values(dev(x), dev(dy), dev(rp), dev(ci)))
    want = float(synth.bf16_to_f64(dy)[:, o] @ z)
    assert abs(dc[0] - want) <= 1e-5 * abs(want)


def test_wide_2048x8192_nnz524288():
    """2048 tokens at d_in = 8192, d_out = 4096, 524,288 entries (64 per
    input column): every y row in chunks, every dx row, every dc entry."""
    rng = np.random.default_rng(8192)
    tokens, d_in, d_out, nnz = 2048, 8192, 4096, 524288
    x = synth.to_bf16(rng.standard_normal((tokens, d_in)))
    dy = synth.to_bf16(rng.standard_normal((tokens, d_out)))
    rp, ci, v = random_csr(rng, d_out, d_in, nnz + nnz // 8)
    y = host64(W().qwha_adapter_forward(dev(x), dev(rp), dev(ci), dev(v), d_out))
    dx = host64(dx_gpu(dy, rp, ci, v, d_in))
    dc = host64(W().qwha_adapter_grad_values(dev(x), dev(dy), dev(rp), dev(ci)))
    x64, dy64, v64 = synth.bf16_to_f64(x), synth.bf16_to_f64(dy), synth.bf16_to_f64(v)
    f = qwha.csr_to_dense(rp, ci, v64, d_out, d_in)
    z = H.wht(x64)
    err_y = compare.float_err(y, z @ f.T)[0]
    err_dx = compare.float_err(dx, H.wht(dy64 @ f))[0]
    rows_of = np.repeat(np.arange(d_out), np.diff(rp))
    want_dc = np.empty(ci.size)
    for e0 in range(0, ci.size, 16384):
        e = slice(e0, min(e0 + 16384, ci.size))
        want_dc[e] = np.einsum("te,te->e", dy64[:, rows_of[e]], z[:, ci[e]])
    err_dc = dc_err(dc, want_dc)
    write_report("parity_qwha_2048x8192_nnz%d" % ci.size,
                 {"y_max_scaled_err": err_y, "dx_max_scaled_err": err_dx, "dc_max_scaled_err": err_dc,
                  "tol_bf16": TOL_BF16, "tol_f32": TOL_F32, "tokens": tokens, "entries": int(ci.size)})
    assert err_y <= TOL_BF16 and err_dx <= TOL_BF16 and err_dc <= TOL_F32


def off_lead_rows(rng, n):
    """Token rows whose mass avoids elements 8m and 8m + 1 (the first 32-bit
    word of every 16-byte chunk the kernels load), at very different
    magnitudes: the per-token staging scale must come from every element."""
    x = np.zeros((7, n))
    x[0, 2] = 3.0e4
    x[1, 5::8] = 1.0e3
    keep = (np.arange(n) % 8) >= 2
    x[2, keep] = rng.standard_normal(keep.sum()) * 1e20
    x[3, keep] = rng.standard_normal(keep.sum()) * 1e-20
    x[4, 7::8] = rng.standard_normal(n // 8) * 100.0
    x[5, 3] = 1e-30
    x[6] = rng.standard_normal(n)
    return x


@pytest.mark.parametrize("d_in", [64, 1024, 4096, 8192])
def test_token_scale_from_every_element(d_in):
    rng = np.random.default_rng(17 + d_in)
    d_out = 512
    x = synth.to_bf16(off_lead_rows(rng, d_in))
    rp, ci, v = random_csr(rng, d_out, d_in, 20 * d_out)
    y = host64(W().qwha_adapter_forward(dev(x), dev(rp), dev(ci), dev(v), d_out))
    assert np.isfinite(y).all()
    want = qwha.qwha_forward(synth.bf16_to_f64(x), rp, ci, synth.bf16_to_f64(v), d_out)
    err = compare.float_err(y, want)[0]
    assert err <= TOL_BF16, err
    dy = synth.to_bf16(off_lead_rows(rng, d_out))
    dx = host64(dx_gpu(dy, rp, ci, v, d_in))
    assert np.isfinite(dx).all()
    want = qwha.qwha_backward_input(synth.bf16_to_f64(dy), rp, ci, synth.bf16_to_f64(v), d_in)
    err = compare.float_err(dx, want)[0]
    assert err <= TOL_BF16, err

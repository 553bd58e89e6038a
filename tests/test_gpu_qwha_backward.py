"""GPU parity of the QWHA adapter backward (dx = (dy F) Hn and dc on the
support of F) against the dense fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import compare, hadamard as H, qwha
from wht_adapters_amd import synth
from gpu_util import write_report, dev, host64

pytestmark = pytest.mark.gpu
TOL_BF16 = 2e-2   # dx is bf16
TOL_F32 = 1e-5    # dc is fp32


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


def dx_gpu(dy, rp, ci, vals, d_in=4096, out=None):
    t_rp, t_ci, t_pm = W().qwha_csr_transpose(rp, ci, d_in)
    v = dev(vals)
    t_v = W().qwha_permute_values(v, dev(t_pm))
    return W().qwha_adapter_backward_input(dev(dy), dev(t_rp), dev(t_ci), t_v, d_in, out=out)


def dc_gpu(x, dy, rp, ci):
    return W().qwha_adapter_grad_values(dev(x), dev(dy), dev(rp), dev(ci))


def dc_err(got, want):
    """fp32 rule with the whole dc vector as one row (floor: its RMS)."""
    return compare.float_err(np.asarray(got, np.float64)[None, :], np.asarray(want)[None, :])[0]


def test_permute_values_exact():
    rng = np.random.default_rng(8)
    rp, ci, vals = random_csr(rng, 300, 4096, 20000)
    t_rp, t_ci, t_pm = W().qwha_csr_transpose(rp, ci, 4096)
    for v in (vals, vals.to(torch.float32)):
        got = W().qwha_permute_values(dev(v), dev(t_pm)).cpu()
        assert torch.equal(got, v[torch.from_numpy(t_pm.astype(np.int64))])


@pytest.mark.parametrize("tokens,d_out,nnz", [(37, 64, 1000), (8, 4096, 20000), (1, 8, 50), (130, 512, 9000),
                                             (13, 37, 800), (20, 2500, 30000), (9, 2049, 7000)])
def test_backward_input_random(tokens, d_out, nnz):
    rng = np.random.default_rng(100 + tokens + d_out)
    dy = synth.to_bf16(rng.standard_normal((tokens, d_out)))
    rp, ci, v = random_csr(rng, d_out, 4096, nnz, empty_rows=(0, 3), empty_cols=(1, 4095))
    dx = dx_gpu(dy, rp, ci, v)
    want = qwha.qwha_backward_input(synth.bf16_to_f64(dy), rp, ci, synth.bf16_to_f64(v), 4096)
    err, roww = compare.float_err(host64(dx), want)
    assert err <= TOL_BF16, (err, roww)


def test_backward_input_identity_and_single_nonzero():
    rng = np.random.default_rng(11)
    n = 4096
    dy = synth.to_bf16(rng.standard_normal((16, n)))
    # F = I: dx = Hn dy
    dx = dx_gpu(dy, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32), synth.to_bf16(np.ones(n)))
    assert compare.float_err(host64(dx), H.wht(synth.bf16_to_f64(dy)))[0] <= TOL_BF16
    # single nonzero F[o, k] = v: dx = v dy[:, o] * (row k of Hn)
    o, k, val = 77, 1234, -0.375
    rp = np.r_[np.zeros(o + 1, np.int32), np.ones(n - o, np.int32)]
    dx = host64(dx_gpu(dy, rp, np.array([k], np.int32), synth.to_bf16(np.array([val]))))
    hk = H.sylvester(n)[k].astype(np.float64) / 64.0
    want = val * synth.bf16_to_f64(dy)[:, o:o + 1] * hk[None, :]
    assert compare.float_err(dx, want)[0] <= TOL_BF16


def test_backward_input_f32_values_strided_out_deterministic():
    rng = np.random.default_rng(12)
    dy = synth.to_bf16(rng.standard_normal((21, 700)))
    rp, ci, v = random_csr(rng, 700, 4096, 12000)
    vf = v.to(torch.float32)
    big = torch.full((21, 4096 + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = big[:, 8:8 + 4096]
    dx1 = dx_gpu(dy, rp, ci, vf, out=out)
    dx2 = dx_gpu(dy, rp, ci, vf)
    assert torch.equal(dx1, dx2)
    assert torch.isnan(big[:, :8]).all() and torch.isnan(big[:, 8 + 4096:]).all()
    want = qwha.qwha_backward_input(synth.bf16_to_f64(dy), rp, ci, vf.double().numpy(), 4096)
    assert compare.float_err(host64(dx1), want)[0] <= TOL_BF16


def test_backward_input_empty_F():
    rng = np.random.default_rng(13)
    dy = synth.to_bf16(rng.standard_normal((10, 100)))
    dx = dx_gpu(dy, np.zeros(101, np.int32), np.zeros(0, np.int32), synth.to_bf16(np.zeros(0)))
    assert not host64(dx).any()


@pytest.mark.parametrize("tokens,d_out,nnz", [(37, 64, 1000), (5, 4096, 20000), (1, 8, 50), (130, 512, 9000),
                                             (300, 1000, 40000), (64, 4096, 70000), (3, 2049, 16385)])
def test_grad_values_random(tokens, d_out, nnz):
    rng = np.random.default_rng(200 + tokens + d_out)
    x = synth.to_bf16(rng.standard_normal((tokens, 4096)))
    dy = synth.to_bf16(rng.standard_normal((tokens, d_out)))
    rp, ci, _ = random_csr(rng, d_out, 4096, nnz, empty_rows=(0, 2))
    dc = dc_gpu(x, dy, rp, ci)
    want = qwha.qwha_grad_values(synth.bf16_to_f64(x), synth.bf16_to_f64(dy), rp, ci)
    err = dc_err(host64(dc), want)
    assert err <= TOL_F32, err


def test_grad_values_deterministic_and_zero_tokens():
    rng = np.random.default_rng(14)
    x = synth.to_bf16(rng.standard_normal((257, 4096)))
    dy = synth.to_bf16(rng.standard_normal((257, 300)))
    rp, ci, _ = random_csr(rng, 300, 4096, 30000)
    a, b = dc_gpu(x, dy, rp, ci), dc_gpu(x, dy, rp, ci)
    assert torch.equal(a, b)
    z = W().qwha_adapter_grad_values(torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda"),
                                     torch.empty((0, 300), dtype=torch.bfloat16, device="cuda"),
                                     dev(rp), dev(ci), out=torch.full((ci.size,), 7.0, device="cuda"))
    assert not z.cpu().numpy().any()


def test_grad_values_single_entry_closed_form():
    """One entry at (o, k): dc = sum_t dy[t, o] (Hn x_t)[k]."""
    rng = np.random.default_rng(15)
    x = synth.to_bf16(rng.standard_normal((50, 4096)))
    dy = synth.to_bf16(rng.standard_normal((50, 10)))
    o, k = 6, 4000
    rp = np.r_[np.zeros(o + 1, np.int32), np.ones(10 - o, np.int32)]
    dc = host64(dc_gpu(x, dy, rp, np.array([k], np.int32)))
    z = synth.bf16_to_f64(x) @ (H.sylvester(4096)[:, k].astype(np.float64) / 64.0)
    want = float(synth.bf16_to_f64(dy)[:, o] @ z)
    assert abs(dc[0] - want) <= 1e-5 * abs(want)


def test_full_config_backward_2048x4096_nnz262144():
    """Every token row of dx and every one of the 262,144 value gradients."""
    d = synth.qwha_backward()
    x, dy, rp, ci, vals = d["x"], d["dy"], d["row_ptr"], d["col_idx"], d["vals"]
    dx = host64(dx_gpu(dy, rp, ci, vals))
    dc = host64(dc_gpu(x, dy, rp, ci))
    want = qwha.qwha_backward_input(synth.bf16_to_f64(dy), rp, ci, synth.bf16_to_f64(vals), 4096)
    err_dx, roww_dx = compare.float_err(dx, want)
    # dc in chunks of entries (the oracle's gathered operands are tokens x entries)
    x64, dy64 = synth.bf16_to_f64(x), synth.bf16_to_f64(dy)
    rows_of = np.repeat(np.arange(4096), np.diff(rp))
    want_dc = np.empty(ci.size)
    z = H.wht(x64)
    for e0 in range(0, ci.size, 16384):
        e = slice(e0, min(e0 + 16384, ci.size))
        want_dc[e] = np.einsum("te,te->e", dy64[:, rows_of[e]], z[:, ci[e]])
    err_dc = dc_err(dc, want_dc)
    write_report("parity_qwha_backward_2048x4096_nnz262144",
                 {"dx_max_scaled_err": err_dx, "dx_max_row_rel_err": roww_dx, "dx_tol": TOL_BF16,
                  "dc_max_scaled_err": err_dc, "dc_tol": TOL_F32, "tokens": 2048, "entries": int(ci.size)})
    assert err_dx <= TOL_BF16 and err_dc <= TOL_F32
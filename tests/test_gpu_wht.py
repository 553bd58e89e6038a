"""GPU parity of wht_batched against the oracle (same seeded inputs)."""
import numpy as np
import pytest
import torch

from oracle import hadamard as H, compare
from wht_adapters_amd import synth
from gpu_util import dev, mask_dev, host64

pytestmark = pytest.mark.gpu

TOL32, TOL16 = 1e-5, 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from wht_adapters_amd import whtq  # noqa: F401  (fails loudly if the library is missing)


def W():
    from wht_adapters_amd import whtq
    return whtq


@pytest.mark.parametrize("logn", range(1, 14))
def test_exact_unnormalised_integers(logn):
    """Integer inputs: every partial sum is exact in fp32, so the raw
    transform must equal the oracle bit for bit."""
    n = 1 << logn
    rng = np.random.default_rng(logn)
    x = rng.integers(-(1 << 10), 1 << 10, size=(13, n)).astype(np.float32)
    y = W().wht_batched(dev(x), normalize=False)
    assert np.array_equal(host64(y), H.wht(x.astype(np.float64), normalize=False))
    xb = rng.integers(-256, 256, size=(5, n)).astype(np.float32)      # exact in bf16
    yb = W().wht_batched(dev(xb, torch.bfloat16), normalize=False, out_dtype=torch.float32)
    assert np.array_equal(host64(yb), H.wht(xb.astype(np.float64), normalize=False))


@pytest.mark.parametrize("n,k", [(4, 1), (16, 2), (64, 3), (1024, 5), (4096, 6)])
def test_exact_normalised_power_of_four(n, k):
    rng = np.random.default_rng(n)
    x = rng.integers(-1000, 1000, size=(9, n)).astype(np.float32)
    y = W().wht_batched(dev(x))
    assert np.array_equal(host64(y), H.wht(x.astype(np.float64), normalize=False) / 2.0 ** k)


@pytest.mark.parametrize("logn", range(1, 14))
@pytest.mark.parametrize("mode", ["none", "before", "after"])
def test_random_f32_all_sizes(logn, mode):
    n = 1 << logn
    rows = 37
    rng = np.random.default_rng(100 + logn)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    bits = rng.integers(0, 2, n)
    mask = synth.sign_bits_to_mask(bits)
    s = H.signs_from_bits(mask, n)
    want = {"none": H.wht(x), "before": H.rht(x, s), "after": H.irht(x, s)}[mode]
    y = W().wht_batched(dev(x), signs=mask_dev(mask), sign_mode=mode)
    err, _ = compare.float_err(host64(y), want)
    assert err <= TOL32, err


@pytest.mark.parametrize("logn", [3, 6, 7, 9, 12, 13])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_16bit_inputs(logn, dt):
    n = 1 << logn
    rng = np.random.default_rng(logn)
    x = dev(rng.standard_normal((19, n)), dt)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    s = H.signs_from_bits(mask, n)
    want = H.rht(host64(x), s)
    y16 = W().wht_batched(x, signs=mask_dev(mask), sign_mode="before")
    y32 = W().wht_batched(x, signs=mask_dev(mask), sign_mode="before", out_dtype=torch.float32)
    assert y16.dtype == dt
    assert compare.float_err(host64(y16), want)[0] <= TOL16
    assert compare.float_err(host64(y32), want)[0] <= TOL32


@pytest.mark.parametrize("logn", [10, 11, 12, 13])
@pytest.mark.parametrize("mode", ["none", "before", "after"])
@pytest.mark.parametrize("rows", [1, 255, 1023, 1024, 1500])
def test_batch_sizes_both_kernels(logn, mode, rows):
    """Below 1024 rows each row is spread over a block of threads, from 1024
    rows on one wave takes a row: both kernels, every sign mode, checked
    against the oracle on sampled rows (first, last and a spread)."""
    n = 1 << logn
    rng = np.random.default_rng(logn * 7 + rows)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    s = H.signs_from_bits(mask, n)
    y = host64(W().wht_batched(dev(x), signs=mask_dev(mask), sign_mode=mode))
    sel = np.unique(np.r_[0:min(rows, 8), np.linspace(0, rows - 1, 16).astype(int), rows - 1])
    xs = x[sel].astype(np.float64)
    want = {"none": H.wht(xs), "before": H.rht(xs, s), "after": H.irht(xs, s)}[mode]
    err, _ = compare.float_err(y[sel], want)
    assert err <= TOL32, err


@pytest.mark.parametrize("logn", [10, 12, 13])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("rows", [100, 1100])
def test_16bit_both_kernels(logn, dt, rows):
    n = 1 << logn
    rng = np.random.default_rng(logn + rows)
    x = dev(rng.standard_normal((rows, n)), dt)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, n))
    s = H.signs_from_bits(mask, n)
    sel = np.linspace(0, rows - 1, 12).astype(int)
    want = H.rht(host64(x[sel]), s)
    y16 = W().wht_batched(x, signs=mask_dev(mask), sign_mode="before")
    y32 = W().wht_batched(x, signs=mask_dev(mask), sign_mode="before", out_dtype=torch.float32)
    assert compare.float_err(host64(y16[sel]), want)[0] <= TOL16
    assert compare.float_err(host64(y32[sel]), want)[0] <= TOL32


def test_pair_sum_rounding():
    """bf16 pairs whose sum / difference needs rounding in fp32: the fused
    first butterfly must round exactly like an fp32 add."""
    rng = np.random.default_rng(7)
    a = rng.standard_normal(4096) * 2.0 ** rng.integers(-30, 30, 4096)
    b = rng.standard_normal(4096) * 2.0 ** rng.integers(-30, 30, 4096)
    x = torch.from_numpy(np.stack([a, b], axis=1)).to(torch.bfloat16)
    xf = x.to(torch.float32).numpy()
    y = W().wht_batched(x.to("cuda:0"), normalize=False, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(y[:, 0], xf[:, 0] + xf[:, 1])
    assert np.array_equal(y[:, 1], xf[:, 0] - xf[:, 1])


def test_full_config_fwht_f32():
    """256 x 4096 fp32, N(0,1) from seed 0, separate output buffer."""
    x = synth.fwht_f32()["x"]
    y = W().wht_batched(dev(x))
    err, roww = compare.float_err(host64(y), H.wht(x.astype(np.float64)))
    assert err <= TOL32, err


def test_inplace_strided_stream_determinism():
    rng = np.random.default_rng(3)
    n = 2048
    big = dev(rng.standard_normal((50, n + 64)).astype(np.float32))
    view = big[:, 32:32 + n]
    want = H.wht(host64(view))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = W().wht_batched(view)
        y2 = W().wht_batched(view)
    s.synchronize()
    assert torch.equal(y1, y2)
    assert compare.float_err(host64(y1), want)[0] <= TOL32
    before = big.clone()
    W().wht_batched(view, out=view)            # exact alias
    torch.cuda.synchronize()
    assert torch.equal(view, y1)
    assert torch.equal(big[:, :32], before[:, :32]) and torch.equal(big[:, 32 + n:], before[:, 32 + n:])


def test_empty_and_single_row():
    e = torch.empty((0, 256), device="cuda:0")
    assert W().wht_batched(e).shape == (0, 256)
    x = dev(np.arange(256, dtype=np.float32)[None])
    assert compare.float_err(host64(W().wht_batched(x)), H.wht(host64(x)))[0] <= TOL32

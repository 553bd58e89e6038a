"""GPU parity of rht_lowbit_gemv (y = x W_hat^T with W_hat decoded from
rht_quantize_rtn codes, the rotation applied to the activations) against
the fp64 oracle: bf16 outputs within 2e-2 of the oracle, scaled by
max(|y|, rms of the token's outputs)."""
import numpy as np
import pytest
import torch

from oracle import gemv, hadamard as H, compare
from wht_adapters_amd import synth
from gpu_util import dev, mask_dev, host64

pytestmark = pytest.mark.gpu

TOL = 2e-2


def W():
    from wht_adapters_amd import whtq
    return whtq


def layer(cfg, rows, n, bits, group, tokens):
    d = synth.lowbit_layer(cfg, rows, n, bits, group, tokens)
    return d, dev(d["x"]), dev(d["codes"]), dev(torch.from_numpy(d["scales"])), mask_dev(d["signs"])


def oracle_rows(d, sel, tokens=None):
    n = d["x"].shape[1]
    s = H.signs_from_bits(d["signs"], n)
    x = synth.bf16_to_f64(d["x"] if tokens is None else d["x"][:tokens])
    return gemv.rht_gemv(x, d["codes"][sel], d["scales"][sel], s, d["bits"], d["group"], n)


def check(got, want):
    sc, roww = compare.float_err(got, want)
    assert sc <= TOL, (sc, roww)
    return sc


def sample_rows(rows, k, seed):
    rng = np.random.default_rng(seed)
    sel = set(rng.choice(rows, min(k, rows), replace=False).tolist())
    sel.update({0, rows - 1})
    return np.array(sorted(sel))


@pytest.mark.parametrize("n,bits,group", [(4096, 2, 16), (4096, 2, 64), (4096, 2, 256),
                                          (4096, 4, 8), (4096, 4, 32), (4096, 4, 128),
                                          (8192, 2, 16), (8192, 2, 32), (8192, 2, 64),
                                          (8192, 4, 16), (8192, 4, 128), (8192, 4, 256)])
def test_gemv_parity(n, bits, group):
    """Every scale-group split of a chunk (1, 2 or 4 groups per 16 bytes) and
    token counts 1, 2, 3 and 5 (full, masked and multi-pass token passes);
    rows past one per wave, oracle on sampled rows."""
    rows = 2600 if n == 4096 else 2200
    d, x, c, s, m = layer(100 + n // 1024 + 10 * bits + group, rows, n, bits, group, 5)
    sel = sample_rows(rows, 40, n + bits)
    want = oracle_rows(d, sel)
    for t in (1, 2, 3, 5):
        y = W().rht_lowbit_gemv(x[:t], c, s, m, bits, group)
        torch.cuda.synchronize()
        check(host64(y)[:, sel], want[:t])


@pytest.mark.parametrize("n,bits,group,rows", [(4096, 2, 64, 7), (8192, 4, 64, 1), (8192, 2, 64, 77),
                                               (4096, 4, 128, 300)])
def test_gemv_small_all_rows(n, bits, group, rows):
    """Fewer rows than waves (and a single row): every output checked."""
    d, x, c, s, m = layer(200 + rows, rows, n, bits, group, 3)
    want = oracle_rows(d, np.arange(rows))
    y = W().rht_lowbit_gemv(x, c, s, m, bits, group)
    torch.cuda.synchronize()
    check(host64(y), want)


def test_gemv_full_size_int2_28672x8192():
    """The 28672 x 8192 INT2 g=64 decode layer in the launch the bench times,
    one and two tokens, the oracle on sampled rows."""
    d = synth.gemv_int2_g64(tokens=2)
    x, c, s, m = dev(d["x"]), dev(d["codes"]), dev(torch.from_numpy(d["scales"])), mask_dev(d["signs"])
    sel = sample_rows(28672, 60, 7)
    want = oracle_rows(d, sel)
    for t in (1, 2):
        y = W().rht_lowbit_gemv(x[:t], c, s, m, 2, 64)
        torch.cuda.synchronize()
        check(host64(y)[:, sel], want[:t])


def test_gemv_full_size_int4_4096x4096():
    d, x, c, s, m = layer(300, 4096, 4096, 4, 128, 4)
    sel = sample_rows(4096, 60, 8)
    want = oracle_rows(d, sel)
    for t in (1, 4):
        y = W().rht_lowbit_gemv(x[:t], c, s, m, 4, 128)
        torch.cuda.synchronize()
        check(host64(y)[:, sel], want[:t])


def test_gemv_no_signs_strides_and_untouched_padding():
    """sign_bits NULL (the plain WHT), x with a row stride above n and y with
    a row stride above rows: the padding of y keeps its sentinel."""
    n, bits, group, rows = 4096, 4, 64, 333
    d, x, c, s, m = layer(400, rows, n, bits, group, 3)
    xs = torch.zeros((3, n + 64), dtype=torch.bfloat16, device="cuda:0")
    xs[:, :n] = x
    ys = torch.full((3, rows + 29), 7.0, dtype=torch.bfloat16, device="cuda:0")
    W().rht_lowbit_gemv(xs[:, :n], c, s, None, bits, group, out=ys[:, :rows])
    torch.cuda.synchronize()
    want = gemv.rht_gemv(synth.bf16_to_f64(d["x"]), d["codes"], d["scales"], np.ones(n), bits, group, n)
    check(host64(ys[:, :rows]), want)
    assert torch.all(ys[:, rows:] == 7.0)


def test_gemv_token_magnitudes():
    """A zero token gives exact zeros; tokens scaled by 2^-100 and 2^100 give
    the scaled outputs (the per-token power-of-two scale keeps fp16 in range)."""
    n, bits, group, rows = 8192, 2, 64, 500
    d, x, c, s, m = layer(500, rows, n, bits, group, 2)
    xt = torch.stack([torch.zeros_like(x[0]), x[0] * 2.0 ** -100, x[1] * 2.0 ** 100])
    y = W().rht_lowbit_gemv(xt, c, s, m, bits, group)
    torch.cuda.synchronize()
    yh = host64(y)
    assert np.all(yh[0] == 0.0)
    want = oracle_rows(d, np.arange(rows))
    check(yh[1:2] * 2.0 ** 100, want[0:1])
    check(yh[2:3] * 2.0 ** -100, want[1:2])


def test_gemv_empty():
    n, bits, group = 4096, 2, 64
    c = torch.zeros((0, n * bits // 8), dtype=torch.uint8, device="cuda:0")
    s = torch.zeros((0, n // group), dtype=torch.float16, device="cuda:0")
    x = torch.zeros((2, n), dtype=torch.bfloat16, device="cuda:0")
    y = W().rht_lowbit_gemv(x, c, s, None, bits, group)
    assert y.shape == (2, 0)
    c1 = torch.zeros((5, n * bits // 8), dtype=torch.uint8, device="cuda:0")
    s1 = torch.zeros((5, n // group), dtype=torch.float16, device="cuda:0")
    y = W().rht_lowbit_gemv(x[:0], c1, s1, None, bits, group)
    assert y.shape == (0, 5)


def test_gemv_agrees_with_dequantised_product():
    """End to end on the GPU: the product through rht_dequantize_inverse's
    rows (fp32 out, then an fp32 matmul) agrees with the online-RHT product."""
    n, bits, group, rows = 4096, 4, 128, 1024
    rng = np.random.default_rng(11)
    w = dev(0.02 * rng.standard_t(3, size=(rows, n)), torch.bfloat16)
    m = mask_dev(synth.sign_bits_to_mask(rng.integers(0, 2, n)))
    codes, scales = W().rht_quantize_rtn(w, m, bits, group)
    w_hat = W().rht_dequantize_inverse(codes, scales, m, bits, group, n, out_dtype=torch.float32)
    x = dev(rng.standard_normal((4, n)), torch.bfloat16)
    y = W().rht_lowbit_gemv(x, codes, scales, m, bits, group)
    ref = x.float() @ w_hat.t()
    torch.cuda.synchronize()
    check(host64(y), host64(ref))


def test_gemv_spiky_rotated_token():
    """A token whose rotation is one spike plus small noise (x = S H e_j / sqrt(n)
    scaled, plus noise): the fixed-point rotated token keeps the spike at full
    scale and rounds the rest; the product still matches the oracle."""
    n, bits, group, rows = 8192, 2, 64, 600
    d, x, c, s, m = layer(600, rows, n, bits, group, 1)
    sv = H.signs_from_bits(d["signs"], n)
    rng = np.random.default_rng(6)
    e = np.zeros((1, n))
    e[0, 1234] = 40.0
    xs = H.irht(e, sv) + 1e-3 * rng.standard_normal((1, n))   # x = S Hn e + noise
    xb = synth.to_bf16(xs)
    y = W().rht_lowbit_gemv(dev(xb), c, s, m, bits, group)
    torch.cuda.synchronize()
    want = gemv.rht_gemv(synth.bf16_to_f64(xb), d["codes"], d["scales"], sv, bits, group, n)
    check(host64(y), want)

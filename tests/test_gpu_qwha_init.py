"""GPU parity of the QWHA initialisation calls (error coefficients, the
calibration Gram matrix, channel errors, top-magnitude selection,
least-squares refinement) against the fp64 oracle.  Each call is fed
inputs the oracle made (rounded to the call's fp32 input type), so no stage
is checked against its own device output; the whole chain is then compared
end to end, where budgets and supports may legitimately differ by
near-ties and the comparison is on what is unique (sums, output error).

Tolerances (u = 2^-24, fp32 unit roundoff):
  error coefficients  2e-4 of the row's rms (fp32 dequantise + fp32 FWHT;
                      ~log2(n) u rms(W) / rms(W - Q(W)))
  Gram matrix         |dG_ab| <= 5e-5 sqrt(G_aa G_bb) (fp32 sums of T products)
  channel errors      1e-4 relative (quadratic form of fp32 G)
  selection           exact (the same fp32 magnitudes on both sides)
  refinement          ||dc|| <= 8 k u cond(G[E][E]) ||c|| + 1e-6 (Cholesky in fp32
                      on fp32-rounded G and P)
"""
import numpy as np
import pytest
import torch

from oracle import compare, hadamard as H, qwha_init as QI, rtn
from wht_adapters_amd import synth
from gpu_util import dev, mask_dev, host64

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def W():
    from wht_adapters_amd import whtq
    return whtq


def quantized(d):
    n = d["w"].shape[1]
    s = H.signs_from_bits(d["signs"], n)
    w64 = synth.bf16_to_f64(d["w"])
    codes, s16, *_ = rtn.rht_quantize(w64, s, d["bits"], d["group"])
    return w64, s, codes, s16


def scales_dev(s16):
    return dev(torch.from_numpy(np.ascontiguousarray(s16, dtype=np.float16)))


def i32(a):
    return dev(np.asarray(a, dtype=np.int32))


@pytest.mark.parametrize("d_out,n,bits,group", [(130, 256, 2, 16), (64, 1024, 3, 64), (200, 4096, 4, 128),
                                                (40, 8192, 2, 64)])
def test_error_coeffs_parity(d_out, n, bits, group):
    d = synth.qinit_layer(200 + n // 256 + bits, d_out, n, 1, bits, group)
    w64, s, codes, s16 = quantized(d)
    want = QI.error_coeffs(w64, codes, s16, s, bits, group)
    got = W().qwha_init_error_coeffs(dev(d["w"]), dev(codes), scales_dev(s16), mask_dev(d["signs"]), bits, group)
    sc, _ = compare.float_err(host64(got), want)
    assert sc < 2e-4, sc


def test_error_coeffs_dtypes_and_strides():
    """fp32 and fp16 weights read through a row stride, output through a
    row stride, no signs."""
    d_out, n, bits, group = 48, 1024, 4, 32
    d = synth.qinit_layer(210, d_out, n, 1, bits, group)
    s = np.ones(n)
    for dt in (torch.float32, torch.float16):
        wt = d["w"].to(dt)
        w64 = wt.to(torch.float64).numpy()
        codes, s16, *_ = rtn.rht_quantize(w64, s, bits, group)
        want = QI.error_coeffs(w64, codes, s16, s, bits, group)
        wpad = torch.zeros((d_out, n + 64), dtype=dt)
        wpad[:, :n] = wt
        out = torch.full((d_out, n + 32), float("nan"), dtype=torch.float32, device="cuda:0")
        W().qwha_init_error_coeffs(dev(wpad)[:, :n], dev(codes), scales_dev(s16), None, bits, group,
                                   out=out[:, :n])
        sc, _ = compare.float_err(host64(out[:, :n]), want)
        assert sc < 2e-4, (dt, sc)
        assert torch.isnan(out[:, n:]).all()


def gram_err(got, want):
    dn = np.sqrt(np.outer(np.diag(want), np.diag(want)))
    return float((np.abs(got - want) / np.maximum(dn, 1e-300)).max())


@pytest.mark.parametrize("tokens,n", [(1, 256), (37, 1024), (300, 4096), (129, 8192)])
def test_gram_parity(tokens, n):
    """Token counts that are not a multiple of the k-step, one token, all
    widths; the result is exactly symmetric."""
    d = synth.qinit_layer(300 + tokens, 1, n, tokens, 4, 128)
    want = QI.calibration_gram(synth.bf16_to_f64(d["x"]))
    g = host64(W().qwha_init_gram(dev(d["x"])))
    assert gram_err(g, want) < 5e-5
    assert np.array_equal(g, g.T)


def test_gram_accumulate_and_empty():
    n, t1, t2 = 512, 100, 61
    d = synth.qinit_layer(320, 1, n, t1 + t2, 4, 128)
    x = d["x"]
    want = QI.calibration_gram(synth.bf16_to_f64(x))
    xs = torch.zeros((t1 + t2, n + 8), dtype=torch.float32)
    xs[:, :n] = x.to(torch.float32)                 # the same values as fp32 rows with a stride
    xs = dev(xs)
    g = W().qwha_init_gram(xs[:t1, :n])
    W().qwha_init_gram(dev(x)[t1:], g=g, accumulate=True)
    assert gram_err(host64(g), want) < 5e-5
    W().qwha_init_gram(dev(x)[:0], g=g, accumulate=True)         # no tokens: unchanged
    assert gram_err(host64(g), want) < 5e-5
    g.fill_(float("nan"))
    W().qwha_init_gram(dev(x)[:0], g=g)                          # no tokens: G = 0
    assert torch.count_nonzero(g).item() == 0


@pytest.mark.parametrize("d_out,n,tokens", [(300, 1024, 200), (77, 4096, 64)])
def test_channel_errors_parity(d_out, n, tokens):
    d = synth.qinit_layer(330 + d_out, d_out, n, tokens, 2, 64)
    w64, s, codes, s16 = quantized(d)
    f32 = QI.error_coeffs(w64, codes, s16, s, 2, 64).astype(np.float32)
    x64 = synth.bf16_to_f64(d["x"])
    g32 = QI.calibration_gram(x64).astype(np.float32)
    p, err = W().qwha_init_channel_errors(dev(f32), dev(g32))
    f64, g64 = f32.astype(np.float64), g32.astype(np.float64)
    want_e = QI.channel_errors(x64, f64)
    assert np.abs(host64(err) - want_e).max() <= 1e-4 * want_e.max()
    assert np.all(np.abs(host64(err) - want_e) <= 1e-4 * want_e + 1e-30)
    sc, _ = compare.float_err(host64(p), f64 @ g64)
    assert sc < 1e-4


@pytest.mark.parametrize("n", [256, 512, 1024, 2048, 4096, 8192])
def test_select_parity(n):
    """Random budgets including 0, 1, n - 1 and n; rows of exact ties, signed
    zeros, denormals and repeated magnitudes; a row stride."""
    rng = np.random.default_rng(n)
    rows = 40
    f = rng.standard_normal((rows, n)).astype(np.float32)
    f[1, :] = 0.5
    f[2, ::3] = -f[2, 0]
    f[3, :] = 0.0
    f[3, ::2] = -0.0
    f[4, :] = np.float32(1e-40) * rng.integers(1, 4, n)
    f[5, :] = np.round(f[5, :] * 4) / 4              # many repeats
    f[6, :] = np.where(rng.random(n) < 0.5, 1.0, -1.0)
    budgets = rng.integers(0, n + 1, rows)
    budgets[:8] = [n, 1, n // 2, n // 3, 7, n - 1, n // 2 + 1, 0]
    budgets[8:12] = [0, 1, n - 1, n]
    row_ptr, cols = QI.select(f.astype(np.float64), budgets)
    fp = np.zeros((rows, n + 16), dtype=np.float32)
    fp[:, :n] = f
    got = W().qwha_init_select(dev(fp)[:, :n], i32(row_ptr))
    assert np.array_equal(got.cpu().numpy(), cols)


def refine_check(g64, p64, row_ptr, cols, got, want):
    """Per-row bound ||dc|| <= 8 k u cond(G[E][E]) ||c|| + 1e-6 ||c||."""
    worst = 0.0
    for o in range(len(row_ptr) - 1):
        a, b = int(row_ptr[o]), int(row_ptr[o + 1])
        if a == b:
            continue
        e = cols[a:b]
        cond = np.linalg.cond(g64[np.ix_(e, e)])
        tol = (8 * (b - a) * U * cond + 1e-6) * np.linalg.norm(want[a:b])
        err = np.linalg.norm(got[a:b] - want[a:b])
        assert err <= tol, (o, b - a, cond, err, tol)
        worst = max(worst, err / max(tol, 1e-300))
    return worst


@pytest.mark.parametrize("n,d_out,tokens", [(256, 90, 400), (1024, 60, 700)])
def test_refine_parity(n, d_out, tokens):
    """Budgets 1..128 including every padding remainder, empty rows; G and P
    are the oracle's, rounded to fp32."""
    d = synth.qinit_layer(340 + n, d_out, n, tokens, 4, 32)
    w64, s, codes, s16 = quantized(d)
    f = QI.error_coeffs(w64, codes, s16, s, 4, 32)
    x64 = synth.bf16_to_f64(d["x"])
    rng = np.random.default_rng(n + 1)
    budgets = rng.integers(1, 129, d_out)
    budgets[:12] = [1, 2, 3, 4, 5, 6, 7, 8, 127, 128, 0, 64]
    row_ptr, cols = QI.select(f, budgets)
    want = QI.refine(x64, f, row_ptr, cols)
    g64 = QI.calibration_gram(x64)
    p64 = f @ g64
    g32, p32 = g64.astype(np.float32), p64.astype(np.float32)
    got = W().qwha_init_refine(dev(g32), dev(p32), i32(row_ptr), i32(cols))
    refine_check(g32.astype(np.float64), p32.astype(np.float64), row_ptr, cols, host64(got), want)


def test_refine_over_limit_is_nan():
    n, d_out, tokens = 256, 3, 300
    d = synth.qinit_layer(350, d_out, n, tokens, 4, 32)
    w64, s, codes, s16 = quantized(d)
    f = QI.error_coeffs(w64, codes, s16, s, 4, 32)
    g = QI.calibration_gram(synth.bf16_to_f64(d["x"]))
    row_ptr, cols = QI.select(f, np.array([10, 129, 5]))
    got = host64(W().qwha_init_refine(dev(g.astype(np.float32)), dev((f @ g).astype(np.float32)),
                                      i32(row_ptr), i32(cols)))
    assert np.isnan(got[10:139]).all()
    assert np.isfinite(got[:10]).all() and np.isfinite(got[139:]).all()


def end_to_end(d, total, floor, cap, sample=None):
    """Run the device chain and the oracle chain on the same layer; compare
    error magnitudes, budgets, supports and the per-row output error."""
    n = d["w"].shape[1]
    bits, group = d["bits"], d["group"]
    w64, s, codes, s16 = quantized(d)
    x64 = synth.bf16_to_f64(d["x"])
    row_ptr_d, col_d, vals_d, err_d = W().qwha_initialize(
        dev(d["w"]), dev(codes), scales_dev(s16), mask_dev(d["signs"]), bits, group, dev(d["x"]),
        total, floor, cap)
    f = QI.error_coeffs(w64, codes, s16, s, bits, group)
    e = QI.channel_errors(x64, f)
    err_d = host64(err_d)
    assert np.all(np.abs(err_d - e) <= 1e-4 * e + 1e-30)
    budgets = QI.allocate(e, total, floor, cap)
    bd = np.diff(row_ptr_d.cpu().numpy().astype(np.int64))
    assert bd.sum() == total and bd.min() >= floor and bd.max() <= cap
    assert np.abs(bd - budgets).max() <= 1
    assert np.mean(bd == budgets) >= 0.99
    rows = d["w"].shape[0]
    sel = np.arange(rows) if sample is None else sample
    rp_d = row_ptr_d.cpu().numpy().astype(np.int64)
    col_d, vals_d = col_d.cpu().numpy(), host64(vals_d)
    same_support = 0
    z = H.wht(x64)
    targets = x64 @ H.wht(f[sel]).T                   # [T, len(sel)]
    for q, o in enumerate(sel):
        a, b = rp_d[o], rp_d[o + 1]
        cd = col_d[a:b]
        assert np.all(np.diff(cd) > 0) and cd.min() >= 0 and cd.max() < n
        # the device support is the top-|F| set of its own budget on the oracle's F,
        # up to near-ties at the boundary
        rp1, c1 = QI.select(f[o:o + 1], np.array([b - a]))
        same_support += int(np.array_equal(cd, c1))
        # per-row output error of the device values vs the oracle's least
        # squares on the device support
        target = targets[:, q]
        c_or = np.linalg.lstsq(z[:, cd], target, rcond=None)[0]
        r_or = np.linalg.norm(z[:, cd] @ c_or - target)
        r_d = np.linalg.norm(z[:, cd] @ vals_d[a:b] - target)
        assert r_d <= r_or * (1 + 1e-3) + 1e-9 * np.linalg.norm(target), (o, r_d, r_or)
    assert same_support >= 0.98 * len(sel)


def test_initialize_end_to_end():
    d = synth.qinit_layer(360, 384, 1024, 600, 2, 32)
    end_to_end(d, total=40 * 384, floor=8, cap=128)


def test_initialize_end_to_end_widest():
    """n = 8192: every kernel at its largest width (Gram and F G tiles, 32
    values per selection thread, G indices past 2^26)."""
    d = synth.qinit_layer(390, 160, 8192, 400, 2, 64)
    end_to_end(d, total=48 * 160, floor=8, cap=128)


def test_initialize_full_size_sampled():
    """The 4096 x 4096 INT4 g=128 layer with 2048 calibration tokens, budget
    262,144 (floor 16, cap 128): every error magnitude and budget, sampled
    rows' supports and output errors."""
    d = synth.qwha_init_int4_g128()
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([rng.choice(4096, 40, replace=False), [0, 4095]]))
    end_to_end(d, d["total"], d["floor"], d["cap"], sample=sample)


def test_refine_zero_gram_is_nan():
    """A zero Gram matrix (no calibration signal) has zero pivots: every
    value comes out NaN, and rows without a budget are left alone."""
    n = 256
    g = torch.zeros((n, n), dtype=torch.float32, device="cuda:0")
    p = torch.zeros((3, n), dtype=torch.float32, device="cuda:0")
    row_ptr = i32([0, 8, 8, 20])
    cols = i32(list(range(8)) + list(range(100, 112)))
    vals = torch.full((20,), 7.0, dtype=torch.float32, device="cuda:0")
    W().qwha_init_refine(g, p, row_ptr, cols, vals=vals)
    assert torch.isnan(vals).all()


def test_initialize_on_a_side_stream():
    """The chain runs on the caller's current stream; results match the
    default-stream run bit for bit."""
    d = synth.qinit_layer(380, 96, 512, 200, 2, 32)
    w64, s, codes, s16 = quantized(d)
    args = (dev(d["w"]), dev(codes), scales_dev(s16), mask_dev(d["signs"]), 2, 32, dev(d["x"]), 96 * 20, 4, 64)
    ref = W().qwha_initialize(*args)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        got = W().qwha_initialize(*args)
    st.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.cpu(), b.cpu())



def test_select_and_refine_in_a_graph():
    """Both calls captured in a HIP graph with caller-given outputs (the
    bindings read nothing back from the device under capture), replayed
    three times with eager work in between: every replay equals the eager
    result bit for bit."""
    rng = np.random.default_rng(77)
    n, rows, tokens = 256, 24, 300
    f = rng.standard_normal((rows, n)).astype(np.float32)
    budgets = rng.integers(1, 33, rows)
    row_ptr, _ = QI.select(f.astype(np.float64), budgets)
    x = rng.standard_normal((tokens, n))
    g64 = QI.calibration_gram(x)
    g32, p32 = g64.astype(np.float32), (f.astype(np.float64) @ g64).astype(np.float32)
    fd, rp, gd, pd = dev(f), i32(row_ptr), dev(g32), dev(p32)
    col_e = W().qwha_init_select(fd, rp)
    val_e = W().qwha_init_refine(gd, pd, rp, col_e)
    col = torch.empty_like(col_e)
    val = torch.empty_like(val_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # one call outside the capture on this stream
        W().qwha_init_select(fd, rp, col_idx=col)
        W().qwha_init_refine(gd, pd, rp, col, vals=val)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        graph.capture_begin()
        W().qwha_init_select(fd, rp, col_idx=col)
        W().qwha_init_refine(gd, pd, rp, col, vals=val)
        graph.capture_end()
    torch.cuda.synchronize()
    for rep in range(3):
        col.fill_(-1)
        val.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(col, col_e), rep
        assert torch.equal(val, val_e), rep
        W().qwha_init_select(fd, rp)  # eager work between replays

"""Forward plans (qwha_forward_plan + qwha_adapter_forward with a plan): the
planned forward must give bit-identical outputs to the unplanned one (the
plan holds the same segment lists, so every fp32 sum runs in the same
order), and a plan that does not fit the call must be ignored."""
import numpy as np
import pytest
import torch

from oracle import qwha, compare
from wht_adapters_amd import synth
from gpu_util import dev, host64

pytestmark = pytest.mark.gpu
TOL = 2e-2
MAGIC, H_STATUS, H_NREC, H_SPLITS = 0x4c505751, 16, 32, 3


def W():
    from wht_adapters_amd import whtq
    return whtq


def header(plan):
    return plan[:256].cpu().view(torch.int32).numpy()


def check_plan(plan, d_out, nnz):
    """The builder finished every split within the plan's room."""
    h = header(plan)
    assert h[0] == MAGIC and h[1] == d_out and h[2] == nnz
    s = int(h[H_SPLITS])
    assert 1 <= s <= 8
    assert np.all(h[H_STATUS:H_STATUS + s] == 0), h[H_STATUS:H_STATUS + s]
    return s, h[H_NREC:H_NREC + s]


def both(x, rp, ci, v, d_out, plan_tokens=None):
    """(unplanned, planned) outputs; the plan built for plan_tokens tokens."""
    x, rp, ci, v = dev(x), dev(rp), dev(ci), dev(v)
    tokens, d_in = x.shape
    nnz = ci.numel()
    plan = W().qwha_forward_plan(plan_tokens or tokens, d_in, rp, d_out, nnz)
    y0 = W().qwha_adapter_forward(x, rp, ci, v, d_out)
    y1 = W().qwha_adapter_forward(x, rp, ci, v, d_out, plan=plan)
    torch.cuda.synchronize()
    return y0, y1, plan


def long_row_csr(rng, d_out, cap=4097):
    lens = rng.integers(0, 40, d_out)
    lens[::7] = rng.integers(1000, cap, lens[::7].size)
    lens[3:12] = [127, 128, 129, 255, 256, 257, 4096, 1, 0]
    cols = np.concatenate([np.sort(rng.choice(4096, int(l), replace=False)) for l in lens]).astype(np.int32)
    rp = np.r_[0, np.cumsum(lens)].astype(np.int32)
    return rp, cols


def test_full_config_2048x4096_nnz262144_planned():
    d = synth.qwha()
    y0, y1, plan = both(d["x"], d["row_ptr"], d["col_idx"], d["vals"], d["d_out"])
    splits, nrec = check_plan(plan, d["d_out"], int(d["col_idx"].size))
    # two row splits of six chunks each, as the host model of the chunking rule
    # in test_qwha_plan_bound counts them
    assert splits == 2 and list(nrec) == [6, 6]
    assert torch.equal(y0, y1)
    # a plan is reused as is: a second call gives the same bytes
    y2 = W().qwha_adapter_forward(dev(d["x"]), dev(d["row_ptr"]), dev(d["col_idx"]), dev(d["vals"]), d["d_out"],
                                  plan=plan)
    assert torch.equal(y0, y2)


@pytest.mark.parametrize("tokens", [37, 300])
def test_long_rows_planned_against_oracle(tokens):
    """Long rows cut into segments over many chunks: identical to the
    unplanned forward and within tolerance of the oracle."""
    rng = np.random.default_rng(100 + tokens)
    d_out = 700
    rp, cols = long_row_csr(rng, d_out)
    x = synth.to_bf16(rng.standard_normal((tokens, 4096)))
    v = synth.to_bf16(0.05 * rng.standard_normal(cols.size))
    y0, y1, plan = both(x, rp, cols, v, d_out)
    check_plan(plan, d_out, cols.size)
    assert torch.equal(y0, y1)
    want = qwha.qwha_forward(synth.bf16_to_f64(x), rp, cols, synth.bf16_to_f64(v), d_out)
    assert compare.float_err(host64(y1), want)[0] <= TOL


def test_split_rows_fill_many_chunks():
    """Every row just past one segment (130 entries, two segments each), so
    chunks end on the partial slots rather than the row count: the plan's
    room bound must hold (status 0 in every split)."""
    rng = np.random.default_rng(7)
    d_out = 4096
    lens = np.full(d_out, 130)
    lens[::5] = 3
    cols = np.concatenate([np.sort(rng.choice(4096, int(l), replace=False)) for l in lens]).astype(np.int32)
    rp = np.r_[0, np.cumsum(lens)].astype(np.int32)
    x = synth.to_bf16(rng.standard_normal((20, 4096)))
    v = synth.to_bf16(0.05 * rng.standard_normal(cols.size))
    y0, y1, plan = both(x, rp, cols, v, d_out)
    splits, nrec = check_plan(plan, d_out, cols.size)
    assert np.all(nrec >= 7)  # 512 rows a split, 410 of them split: 820 segments over 112 slots a chunk
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("d_in", [64, 1024, 2048])
def test_narrower_inputs_planned(d_in):
    rng = np.random.default_rng(d_in)
    d_out, nnz = 333, 4000
    rows = rng.integers(0, d_out, nnz)
    colsr = rng.integers(0, d_in, nnz)
    key = np.unique(rows * d_in + colsr)
    rows, cols = key // d_in, (key % d_in).astype(np.int32)
    rp = np.r_[0, np.cumsum(np.bincount(rows, minlength=d_out))].astype(np.int32)
    x = synth.to_bf16(rng.standard_normal((45, d_in)))
    v = synth.to_bf16(0.1 * rng.standard_normal(cols.size))
    y0, y1, _ = both(x, rp, cols, v, d_out)
    assert torch.equal(y0, y1)


def test_f32_values_and_empty_support_planned():
    rng = np.random.default_rng(11)
    d_out = 256
    rp, cols = long_row_csr(rng, d_out, cap=1500)
    x = synth.to_bf16(rng.standard_normal((24, 4096)))
    v = torch.from_numpy((0.05 * rng.standard_normal(cols.size)).astype(np.float32))
    y0, y1, _ = both(x, rp, cols, v, d_out)
    assert torch.equal(y0, y1)
    # F = 0: no entries at all
    rp0 = np.zeros(d_out + 1, dtype=np.int32)
    e = np.zeros(0, dtype=np.int32)
    y0, y1, plan = both(x, rp0, e, torch.zeros(0, dtype=torch.bfloat16), d_out)
    check_plan(plan, d_out, 0)
    assert torch.equal(y0, y1) and not torch.any(y1)


def test_mismatched_plans_are_ignored():
    """A plan built for another token count (another split of the rows), a
    plan with a spoiled header and a plan passed with too small a size are
    all ignored: the output is the unplanned one."""
    rng = np.random.default_rng(5)
    d_out = 900
    rp, cols = long_row_csr(rng, d_out, cap=2000)
    x = synth.to_bf16(rng.standard_normal((2048, 4096)))
    v = synth.to_bf16(0.05 * rng.standard_normal(cols.size))
    y0, y1, plan_other = both(x, rp, cols, v, d_out, plan_tokens=37)
    assert header(plan_other)[H_SPLITS] == 8  # 3 token tiles: eight splits; 2048 tokens: two
    assert torch.equal(y0, y1)
    xd, rpd, cd, vd = dev(x), dev(rp), dev(cols), dev(v)
    plan = W().qwha_forward_plan(2048, 4096, rpd, d_out, cols.size)
    spoiled = plan.clone()
    spoiled[:4] = 0
    assert torch.equal(y0, W().qwha_adapter_forward(xd, rpd, cd, vd, d_out, plan=spoiled))
    assert torch.equal(y0, W().qwha_adapter_forward(xd, rpd, cd, vd, d_out, plan=plan[:256]))
    assert torch.equal(y0, W().qwha_adapter_forward(xd, rpd, cd, vd, d_out, plan=plan))


def test_d_in_8192_needs_no_plan():
    rng = np.random.default_rng(8192)
    d_out, nnz = 128, 3000
    rows = np.sort(rng.integers(0, d_out, nnz))
    cols = rng.integers(0, 8192, nnz).astype(np.int32)
    key = np.unique(rows * 8192 + cols)
    rows, cols = key // 8192, (key % 8192).astype(np.int32)
    rp = np.r_[0, np.cumsum(np.bincount(rows, minlength=d_out))].astype(np.int32)
    x = synth.to_bf16(rng.standard_normal((12, 8192)))
    v = synth.to_bf16(0.1 * rng.standard_normal(cols.size))
    assert W().raw().qwha_forward_plan_bytes(12, 8192, d_out, cols.size) == 0
    y0, y1, _ = both(x, rp, cols, v, d_out)
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("tokens,d_out,nnz", [(1, 5, 40), (17, 8, 200), (3, 9, 0)])
def test_small_shapes_planned(tokens, d_out, nnz):
    """One token, outputs narrower than a 16-byte store, one or two row
    splits (at most one per 8 rows) and an empty support: the planned
    forward gives the unplanned bytes."""
    rng = np.random.default_rng(tokens * 100 + d_out)
    rows = np.sort(rng.integers(0, d_out, nnz))
    cols = rng.integers(0, 4096, nnz)
    key = np.unique(rows * 4096 + cols)
    rows, cols = key // 4096, (key % 4096).astype(np.int32)
    rp = np.r_[0, np.cumsum(np.bincount(rows, minlength=d_out))].astype(np.int32)
    x = synth.to_bf16(rng.standard_normal((tokens, 4096)))
    v = synth.to_bf16(0.1 * rng.standard_normal(cols.size))
    y0, y1, plan = both(x, rp, cols, v, d_out)
    splits, _ = check_plan(plan, d_out, cols.size)
    assert splits == (d_out + 7) // 8
    assert torch.equal(y0, y1)

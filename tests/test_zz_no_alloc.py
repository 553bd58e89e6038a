"""The allocation-free value gradient (qwha_adapter_grad_values_noalloc)
against the workspace entry point it shares its kernels with: the same bits,
and the oracle's values within the fp32 rule, on two calls in a row, the
second smaller than the first (so the fixed per-GPU scratch array holds the
first call's data when the second one starts)."""
import numpy as np
import pytest
import torch

from oracle import compare, qwha
from wht_adapters_amd import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu


def W():
    from wht_adapters_amd import whtq
    return whtq


def _case(rng, tokens, d_out, nnz):
    x = synth.to_bf16(rng.standard_normal((tokens, 4096)))
    dy = synth.to_bf16(rng.standard_normal((tokens, d_out)))
    rows = rng.integers(0, d_out, nnz)
    cols = rng.integers(0, 4096, nnz)
    key = np.unique(rows * 4096 + cols)
    rows, cols = key // 4096, key % 4096
    rp = np.r_[0, np.cumsum(np.bincount(rows, minlength=d_out))].astype(np.int32)
    return x, dy, rp, cols.astype(np.int32)


def _err(got, want):
    return compare.float_err(np.asarray(got, np.float64)[None, :], np.asarray(want)[None, :])[0]


def test_noalloc_matches_workspace_entry_two_calls():
    d = synth.qwha_backward()          # 2048 tokens, 262,144 entries: the full workload first
    x, dy, rp, ci = dev(d["x"]), dev(d["dy"]), dev(d["row_ptr"]), dev(d["col_idx"])
    a = W().qwha_adapter_grad_values_noalloc(x, dy, rp, ci)
    b = W().qwha_adapter_grad_values(x, dy, rp, ci)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    toks = np.arange(0, 2048, 97)
    rows = np.arange(0, 4096, 211)
    lens = np.diff(d["row_ptr"])[rows]
    ent = np.concatenate([np.arange(d["row_ptr"][o], d["row_ptr"][o + 1]) for o in rows])
    sub_rp = np.r_[0, np.cumsum(lens)].astype(np.int32)
    want = qwha.qwha_grad_values(synth.bf16_to_f64(d["x"]), synth.bf16_to_f64(d["dy"])[:, rows], sub_rp,
                                 d["col_idx"][ent])
    assert _err(a.cpu().numpy()[ent], want) <= 1e-5
    del toks
    # second call, smaller (fewer tokens, entries and rows), right after the first
    rng = np.random.default_rng(2024)
    xs, dys, rps, cis = _case(rng, 300, 1000, 40000)
    a2 = W().qwha_adapter_grad_values_noalloc(dev(xs), dev(dys), dev(rps), dev(cis))
    b2 = W().qwha_adapter_grad_values(dev(xs), dev(dys), dev(rps), dev(cis))
    torch.cuda.synchronize()
    assert torch.equal(a2, b2)
    want2 = qwha.qwha_grad_values(synth.bf16_to_f64(xs), synth.bf16_to_f64(dys), rps, cis)
    assert _err(a2.cpu().numpy(), want2) <= 1e-5


def test_noalloc_zero_tokens_and_capacity():
    rng = np.random.default_rng(5)
    x, dy, rp, ci = _case(rng, 4, 64, 500)
    z = W().qwha_adapter_grad_values_noalloc(torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda"),
                                             torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                                             dev(rp), dev(ci), out=torch.full((ci.size,), 7.0, device="cuda"))
    assert not z.cpu().numpy().any()
    big = torch.empty((5000, 4096), dtype=torch.bfloat16, device="cuda")   # 5000 x 16 KiB > 64 MiB
    dyb = torch.empty((5000, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(W().WhtqError) as e:
        W().qwha_adapter_grad_values_noalloc(big, dyb, dev(rp), dev(ci))
    assert e.value.status == 5

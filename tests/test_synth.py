"""Seeded generators: determinism and the structure the workloads ask for."""
import numpy as np
import torch

from wht_adapters_amd import synth


def test_determinism_and_dtypes():
    a = synth.rht_weights(2, 64, 256)
    b = synth.rht_weights(2, 64, 256)
    assert a["w"].dtype == torch.bfloat16
    assert torch.equal(a["w"], b["w"]) and np.array_equal(a["signs"], b["signs"])
    assert a["signs"].dtype == np.uint32 and a["signs"].size == 256 // 32
    c = synth.rht_weights(5, 64, 256)
    assert not torch.equal(a["w"], c["w"])


def test_outlier_columns_scaled():
    d = synth.rht_weights(2, 512, 4096)
    w = synth.bf16_to_f64(d["w"])
    col_rms = np.sqrt((w * w).mean(axis=0))
    top = set(np.argsort(col_rms)[-4:])
    assert top == set(d["outlier_cols"].tolist())


def test_fwht_input_is_seed0():
    x = synth.fwht_f32(rows=4, n=16)["x"]
    assert x.dtype == np.float32
    assert np.array_equal(x, np.random.default_rng(0).standard_normal((4, 16)).astype(np.float32))


def test_nnz_allocation():
    r = np.exp(synth.child_rng(3, 1).standard_normal(4096))
    n = synth.allocate_nnz(r, 262144, floor=8, cap=4096)
    assert n.sum() == 262144 and n.min() >= 8 and n.max() <= 4096
    # proportional above the floor: ordering of budgets follows r
    big = n > 8
    assert np.all(np.diff(n[big][np.argsort(r[big])]) >= -1)


def test_sparse_adapter_small():
    rp, ci, v = synth.sparse_adapter(3, 64, 128, 1024)
    assert rp[0] == 0 and rp[-1] == 1024 and np.all(np.diff(rp) >= 8)
    for o in range(64):
        c = ci[rp[o]:rp[o + 1]]
        assert np.all(np.diff(c) > 0) and c.min() >= 0 and c.max() < 128
    assert v.dtype == torch.bfloat16 and v.numel() == 1024


def test_orthogonal_blocks():
    b = synth.orthogonal_blocks(np.random.default_rng(0), 10, 16)
    assert b.dtype == np.float32
    eye = np.einsum("cij,ckj->cik", b.astype(np.float64), b.astype(np.float64))
    assert np.allclose(eye, np.eye(16)[None], atol=1e-6)


def test_sign_mask_packing():
    bits = np.zeros(40, np.uint8); bits[[0, 2, 33]] = 1
    m = synth.sign_bits_to_mask(bits)
    assert m.tolist() == [5, 2]

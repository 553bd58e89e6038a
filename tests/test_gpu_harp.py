"""GPU parity of harp_rotate against the dense-stage oracle."""
import numpy as np
import pytest
import torch

from oracle import hadamard as H, harp, compare
from wht_adapters_amd import synth
from gpu_util import write_report, dev, mask_dev, host64

pytestmark = pytest.mark.gpu
TOL = 2e-2
RAD = [16, 16, 16]


def W():
    from wht_adapters_amd import whtq
    return whtq


def flat(blocks, dtype=torch.float32):
    return torch.from_numpy(np.concatenate([np.asarray(b, np.float32).reshape(-1) for b in blocks])).to(dtype)


def run(x, blocks, mask=None, pre=True, bdt=torch.float32):
    return W().harp_rotate(dev(x), dev(flat(blocks, bdt)), RAD, mask_dev(mask) if mask is not None else None, pre)


def digits(i):
    return [i % 16, (i // 16) % 16, i // 256]


def test_permutation_blocks_exact():
    """Identity blocks except one permutation block per stage, no
    preconditioning: every output is one input value, so the result must be
    the predicted permutation bit for bit (checks the MFMA operand layouts
    and the digit / block-index convention at the real shape)."""
    rng = np.random.default_rng(5)
    x = synth.to_bf16(rng.standard_normal((37, 4096)))
    blocks = []
    for t in range(3):
        bl = np.broadcast_to(np.eye(16, dtype=np.float32), (256, 16, 16)).copy()
        for _ in range(5):
            bl[int(rng.integers(0, 256))] = np.eye(16, dtype=np.float32)[rng.permutation(16)]
        blocks.append(bl)
    y = run(x, blocks, pre=False)
    want = synth.bf16_to_f64(x)
    for t in range(3):
        z = want.copy()
        bl = blocks[t]
        for i in range(4096):
            dg = digits(i)
            rest = [dd for u, dd in enumerate(dg) if u != t]
            c = rest[0] + 16 * rest[1]
            k = int(np.argmax(bl[c][dg[t]]))
            j = list(dg); j[t] = k
            z[:, i] = want[:, j[0] + 16 * j[1] + 256 * j[2]]
        want = z
    assert np.array_equal(host64(y), want)


def test_hadamard_blocks_equal_wht():
    """Theta = 0: blocks H16/4 compose to the Sylvester WHT (H16/4 is exact in bf16)."""
    rng = np.random.default_rng(6)
    x = synth.to_bf16(rng.standard_normal((20, 4096)))
    h = (H.sylvester(16) / 4.0).astype(np.float32)
    blocks = [np.broadcast_to(h, (256, 16, 16)) for _ in range(3)]
    y = run(x, blocks, pre=False)
    err = compare.float_err(host64(y), H.wht(synth.bf16_to_f64(x)))[0]
    print(f"hadamard blocks: max scaled error {err:.3e}")
    assert err <= TOL
    eye = [np.broadcast_to(np.eye(16, dtype=np.float32), (256, 16, 16)) for _ in range(3)]
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, 4096))
    y = run(x, eye, mask=mask, pre=True)
    want = H.rht(synth.bf16_to_f64(x), H.signs_from_bits(mask, 4096))
    err = compare.float_err(host64(y), want)[0]
    print(f"max scaled error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("bdt", [torch.float32, torch.float16])
@pytest.mark.parametrize("tokens", [1, 15, 16, 31, 100])
def test_random_orthogonal(tokens, bdt):
    rng = np.random.default_rng(tokens)
    x = synth.to_bf16(rng.standard_normal((tokens, 4096)))
    blocks = [synth.orthogonal_blocks(rng, 256, 16) for _ in range(3)]
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, 4096))
    y = run(x, blocks, mask=mask, bdt=bdt)
    want = harp.harp_rotate(synth.bf16_to_f64(x), RAD, blocks, s=H.signs_from_bits(mask, 4096))
    err = compare.float_err(host64(y), want)[0]
    print(f"max scaled error {err:.3e}")
    assert err <= TOL


def test_fp16_blocks_match_fp32_blocks():
    """The kernel rounds fp32 blocks to fp16 (nearest even) before its MFMAs,
    so blocks handed over already rounded the same way give the same bits."""
    rng = np.random.default_rng(77)
    x = synth.to_bf16(rng.standard_normal((48, 4096)))
    blocks = [synth.orthogonal_blocks(rng, 256, 16) for _ in range(3)]
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, 4096))
    y32 = run(x, blocks, mask=mask, bdt=torch.float32)
    y16 = run(x, blocks, mask=mask, bdt=torch.float16)
    assert torch.equal(y32.cpu(), y16.cpu())


@pytest.mark.parametrize("bdt", [torch.float16, torch.float32])
def test_full_config_8192x4096(bdt):
    """At the full size, with fp16 blocks as bench.py times them and fp32
    blocks: every one of the 8192 tokens against the oracle."""
    d = synth.harp()
    y = host64(W().harp_rotate(dev(d["x"]), dev(flat(d["blocks"], bdt)), d["radices"], mask_dev(d["signs"]), True))
    want = harp.harp_rotate(synth.bf16_to_f64(d["x"]), RAD, d["blocks"], s=H.signs_from_bits(d["signs"], 4096))
    err, roww = compare.float_err(y, want)
    write_report("parity_harp_8192x4096_" + str(bdt).split(".")[-1] + "_blocks",
                 {"tokens": 8192, "max_scaled_err": err, "max_row_rel_err": roww, "tol": TOL})
    assert err <= TOL


def off_lead_rows(rng, n):
    """Rows whose mass avoids elements 8m and 8m + 1 (the first 32-bit word
    of every 16-byte chunk the kernel loads), at very different magnitudes:
    the per-row power-of-two scale must come from every element."""
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


@pytest.mark.parametrize("pre", [True, False])
def test_row_scale_from_every_element(pre):
    rng = np.random.default_rng(91)
    x = synth.to_bf16(off_lead_rows(rng, 4096))
    blocks = [synth.orthogonal_blocks(rng, 256, 16) for _ in range(3)]
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, 4096))
    y = host64(run(x, blocks, mask=mask if pre else None, pre=pre, bdt=torch.float16))
    assert np.isfinite(y).all()
    want = harp.harp_rotate(synth.bf16_to_f64(x), RAD, blocks, s=H.signs_from_bits(mask, 4096) if pre else None,
                            precondition=pre)
    err = compare.float_err(y, want)[0]
    assert err <= TOL, err

"""GPU parity of harp_build_blocks (B = Q(theta) G: Givens for radix 2,
Cayley above) against the fp64 oracle, and the blocks it builds in use."""
import numpy as np
import pytest
import torch

from oracle import hadamard as H, harp, compare
from wht_adapters_amd import synth
from gpu_util import dev, host64

pytestmark = pytest.mark.gpu


def W():
    from wht_adapters_amd import whtq
    return whtq


def n_params(radices, d):
    return sum((d // b) * harp.params_per_block(b) for b in radices)


def qr_mixers(rng, radices):
    return [synth.orthogonal_blocks(rng, 1, b)[0].astype(np.float64) for b in radices]


def flat(mats):
    return torch.from_numpy(np.concatenate([np.asarray(m, np.float32).reshape(-1) for m in mats]))


def gpu_blocks(radices, d, blocks_flat):
    out, o = [], 0
    for b in radices:
        out.append(blocks_flat[o:o + d * b].reshape(d // b, b, b))
        o += d * b
    return out


@pytest.mark.parametrize("radices,scale", [((2, 4, 8, 16), 0.3), ((8, 8, 8, 5, 2), 0.2), ((3, 7, 5), 0.5),
                                           ((16, 16, 16), 0.1), ((2,) * 6, 1.5), ((11, 13), 0.25)])
def test_build_f32_params(radices, scale):
    d = int(np.prod(radices))
    rng = np.random.default_rng(d)
    p = (scale * rng.standard_normal(n_params(radices, d))).astype(np.float32)
    pow2 = all(b & (b - 1) == 0 for b in radices)
    mix = None if pow2 else qr_mixers(rng, radices)
    out = W().harp_build_blocks(dev(torch.from_numpy(p)), radices, d,
                                mixers=None if mix is None else dev(flat(mix)))
    want = harp.build_blocks(p.astype(np.float64), list(radices), d, mix)
    got = gpu_blocks(radices, d, host64(out))
    for g, w in zip(got, want):
        assert np.abs(g - w).max() <= 2e-6, np.abs(g - w).max()
        # the built blocks are orthogonal to fp32 accuracy
        eye = np.einsum("cij,ckj->cik", g, g)
        assert np.abs(eye - np.eye(g.shape[1])).max() <= 5e-6


def test_build_int8_params_and_fp16_blocks():
    radices, d = (8, 8, 8, 5, 2), 5120
    rng = np.random.default_rng(7)
    q = rng.integers(-127, 128, n_params(radices, d)).astype(np.int8)
    scales = np.array([0.004, 0.003, 0.005, 0.002, 0.01], np.float32)
    mix = qr_mixers(rng, radices)
    out = W().harp_build_blocks(dev(torch.from_numpy(q)), radices, d, scales=dev(torch.from_numpy(scales)),
                                mixers=dev(flat(mix)), out_dtype=torch.float16)
    theta = harp.dequant_params(q, scales.astype(np.float64), list(radices), d)
    want = harp.build_blocks(theta, list(radices), d, mix)
    got = gpu_blocks(radices, d, host64(out))
    for g, w in zip(got, want):
        assert np.abs(g - w).max() <= 1e-3   # one fp16 rounding of values <= 1


def test_theta_zero_gives_the_mixer_and_the_rht():
    """Theta = 0: B = G; with Sylvester mixers and the preconditioning off,
    the rotation built from them is the WHT ([HARP] 2.2)."""
    radices, d = (16, 16, 16), 4096
    out = W().harp_build_blocks(torch.zeros(n_params(radices, d), device="cuda"), radices, d)
    got = gpu_blocks(radices, d, host64(out))
    for b, g in zip(radices, got):
        assert np.abs(g - harp.sylvester_mixer(b)).max() <= 1e-7
    x = synth.to_bf16(np.random.default_rng(1).standard_normal((8, d)))
    y = W().harp_rotate(dev(x), out, radices, None, False)
    assert compare.float_err(host64(y), H.wht(synth.bf16_to_f64(x)))[0] <= 2e-2


def test_built_blocks_through_the_general_rotation():
    radices, d = (8, 8, 8, 5, 2), 5120
    rng = np.random.default_rng(11)
    p = (0.2 * rng.standard_normal(n_params(radices, d))).astype(np.float32)
    mix = qr_mixers(rng, radices)
    blocks = W().harp_build_blocks(dev(torch.from_numpy(p)), radices, d, mixers=dev(flat(mix)))
    x = synth.to_bf16(rng.standard_normal((13, d)))
    y = W().harp_rotate(dev(x), blocks, radices, None, False)
    want = harp.harp_rotate(synth.bf16_to_f64(x), list(radices),
                            harp.build_blocks(p.astype(np.float64), list(radices), d, mix), precondition=False)
    assert compare.float_err(host64(y), want)[0] <= 8e-3

"""GPU parity of harp_rotate on general mixed-radix schedules (radices 2..16,
any product d <= 8192, power-of-two d with the preconditioning) against the
dense-stage oracle."""
import numpy as np
import pytest
import torch

from oracle import hadamard as H, harp, compare
from wht_adapters_amd import synth
from gpu_util import dev, mask_dev, host64

pytestmark = pytest.mark.gpu
TOL = 2e-2   # bf16 output


def W():
    from wht_adapters_amd import whtq
    return whtq


def flat(blocks, dtype=torch.float32):
    return torch.from_numpy(np.concatenate([np.asarray(b, np.float32).reshape(-1) for b in blocks])).to(dtype)


def padded_rows(x):
    """bf16 [tokens, d] in storage whose rows start 16-byte aligned (the ABI rule)."""
    t, d = x.shape
    ld = d if d * 2 < 16 else -(-d // 8) * 8
    buf = torch.zeros((t, ld), dtype=torch.bfloat16, device="cuda")
    buf[:, :d] = dev(x)
    return buf[:, :d]


def run(x, radices, blocks, mask=None, pre=False, bdt=torch.float32):
    xd = padded_rows(x)
    out = padded_rows(torch.zeros_like(x))
    return W().harp_rotate(xd, dev(flat(blocks, bdt)), tuple(radices), mask_dev(mask) if mask is not None else None,
                           pre, out=out)


def rand_blocks(rng, radices):
    d = int(np.prod(radices))
    return [synth.orthogonal_blocks(rng, d // b, b) for b in radices]


SCHED = [
    ((8, 8, 8, 5, 2), 19, False),     # the page's d = 5120 example
    ((5, 3, 2), 40, False),
    ((2, 4, 3), 33, False),
    ((3, 7, 5), 9, False),            # odd d = 105: element loads and stores
    ((16, 8), 70, True),
    ((4, 4, 4, 4, 4, 4), 21, True),   # d = 4096, radix 4
    ((2,) * 13, 7, True),             # d = 8192, radix 2
    ((16, 16, 16, 2), 5, True),       # d = 8192, the largest tile
    ((12, 10, 11, 6), 6, False),      # d = 7920, radices 9..16 split over lanes
    ((13, 9, 14, 2, 2), 4, False),
    ((16, 16, 4), 30, True),
    ((16, 16, 2, 9), 11, False),      # d = 4608: two 512-thread blocks per CU, 4-token tiles
    ((16, 15, 5, 4), 9, False),       # d = 4800: one 1024-thread block per CU
]


@pytest.mark.parametrize("radices,tokens,pre", SCHED)
def test_general_schedules(radices, tokens, pre):
    d = int(np.prod(radices))
    rng = np.random.default_rng(d + tokens)
    x = synth.to_bf16(rng.standard_normal((tokens, d)))
    blocks = rand_blocks(rng, radices)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, d)) if pre else None
    y = run(x, radices, blocks, mask, pre)
    s = H.signs_from_bits(mask, d) if pre else None
    want = harp.harp_rotate(synth.bf16_to_f64(x), list(radices), blocks, s=s, precondition=pre)
    err, roww = compare.float_err(host64(y), want)
    assert err <= TOL, (err, roww)
    # fp32 arithmetic throughout: well inside the bf16 budget
    assert err <= 8e-3, err


@pytest.mark.parametrize("radices", [(4, 4, 4, 4, 4, 4), (2,) * 10, (16, 8, 8), (8, 2, 16, 4)])
def test_hadamard_blocks_give_the_wht(radices):
    """Blocks H_b / sqrt(b) in every stage, no preconditioning: exactly the
    orthonormal Sylvester WHT (the digit convention's Theta = 0 case)."""
    d = int(np.prod(radices))
    rng = np.random.default_rng(d)
    x = synth.to_bf16(rng.standard_normal((12, d)))
    blocks = [np.broadcast_to((H.sylvester(b) / np.sqrt(b)).astype(np.float32), (d // b, b, b)).copy()
              for b in radices]
    y = run(x, radices, blocks)
    err, _ = compare.float_err(host64(y), H.wht(synth.bf16_to_f64(x)))
    assert err <= 8e-3, err


def test_identity_blocks_give_the_rht():
    radices = (8, 8, 8, 2, 2, 2)
    d = 4096
    rng = np.random.default_rng(3)
    x = synth.to_bf16(rng.standard_normal((10, d)))
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, d))
    blocks = [np.broadcast_to(np.eye(b, dtype=np.float32), (d // b, b, b)).copy() for b in radices]
    y = run(x, radices, blocks, mask, pre=True)
    want = H.rht(synth.bf16_to_f64(x), H.signs_from_bits(mask, d))
    assert compare.float_err(host64(y), want)[0] <= 8e-3


def test_permutation_blocks_exact_mixed_radix():
    """Identity blocks except a few permutation blocks: every output is one
    input value, so the result is the predicted permutation bit for bit
    (checks the digit and block-index convention for non-power-of-two radices)."""
    radices = (5, 4, 6)
    d = 120
    rng = np.random.default_rng(9)
    x = synth.to_bf16(rng.standard_normal((11, d)))
    blocks = []
    for b in radices:
        bl = np.broadcast_to(np.eye(b, dtype=np.float32), (d // b, b, b)).copy()
        for _ in range(4):
            bl[int(rng.integers(0, d // b))] = np.eye(b, dtype=np.float32)[rng.permutation(b)]
        blocks.append(bl)
    y = run(x, radices, blocks)
    want = harp.harp_rotate(synth.bf16_to_f64(x), list(radices), blocks, precondition=False)
    assert np.array_equal(host64(y), want)


def test_fp16_blocks_and_ragged_tokens():
    radices = (8, 8, 8, 5, 2)
    d = 5120
    rng = np.random.default_rng(4)
    blocks = rand_blocks(rng, radices)
    b16 = [np.asarray(b, np.float16).astype(np.float32) for b in blocks]
    for tokens in (1, 6, 7, 8, 15):
        x = synth.to_bf16(rng.standard_normal((tokens, d)))
        y = run(x, radices, blocks, bdt=torch.float16)
        want = harp.harp_rotate(synth.bf16_to_f64(x), list(radices), b16, precondition=False)
        assert compare.float_err(host64(y), want)[0] <= 8e-3


def test_orthogonal_inverse_roundtrip():
    """Stages with B^T in reverse order undo the rotation (orthogonal blocks)."""
    radices = (8, 8, 8, 5, 2)
    d = 5120
    rng = np.random.default_rng(6)
    blocks = rand_blocks(rng, radices)
    x = synth.to_bf16(rng.standard_normal((9, d)))
    y = run(x, radices, blocks)
    # inverse: stage t^-1 = blocks transposed, applied last-stage first; as a
    # schedule that is the reversed radices with digits reversed, which the
    # oracle checks through the dense matrices
    m = np.eye(d)
    for t in range(len(radices)):
        m = harp.stage_matrix(blocks[t], t, list(radices)) @ m
    back = host64(y) @ m   # y = x M^T  ->  x = y M
    assert compare.float_err(back, synth.bf16_to_f64(x))[0] <= 2e-2


TOL_F32 = 1e-5   # fp32 output


def padded_rows_f32(x):
    t, d = x.shape
    ld = d if d * 4 < 16 else -(-d // 4) * 4
    buf = torch.zeros((t, ld), dtype=torch.float32, device="cuda")
    buf[:, :d] = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda")
    return buf[:, :d]


@pytest.mark.parametrize("radices,tokens,pre", [((16, 16, 16), 37, True), ((8, 8, 8, 5, 2), 11, False),
                                                ((5, 3, 2), 40, False), ((3, 7, 5), 9, False),
                                                ((2,) * 13, 5, True), ((16, 16, 16, 2), 3, True)])
def test_f32_rows(radices, tokens, pre):
    """fp32 rows (every schedule, the radix-16 one included, on the fp32 tile):
    the fp32 rule against the oracle."""
    rng = np.random.default_rng(sum(radices) + tokens)
    d = int(np.prod(radices))
    x = rng.standard_normal((tokens, d)).astype(np.float32)
    blocks = rand_blocks(rng, radices)
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, d)) if pre else None
    out = padded_rows_f32(np.zeros_like(x))
    y = W().harp_rotate(padded_rows_f32(x), dev(flat(blocks)), tuple(radices),
                        mask_dev(mask) if mask is not None else None, pre, out=out)
    want = harp.harp_rotate(x.astype(np.float64), list(radices), blocks,
                            s=H.signs_from_bits(mask, d) if pre else None, precondition=pre)
    assert compare.float_err(host64(y), want)[0] <= TOL_F32


def _two_sided_gpu(w_dev, out_side, in_side):
    """W~ = R_out W R_in^T as two harp_rotate calls: the rows of W (input
    side), then the rows of the transpose (output side)."""
    def rot(x, sd):
        mask = sd["mask"]
        return W().harp_rotate(x, dev(flat(sd["blocks"])), tuple(sd["radices"]),
                               mask_dev(mask) if mask is not None else None, sd["precondition"])
    t = rot(w_dev, in_side)
    return rot(t.t().contiguous(), out_side).t()


def _side(rng, radices, pre):
    d = int(np.prod(radices))
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, d)) if pre else None
    return {"radices": list(radices), "blocks": rand_blocks(rng, radices), "mask": mask, "precondition": pre}


def _oracle_side(sd):
    d = int(np.prod(sd["radices"]))
    return {"radices": sd["radices"], "blocks": sd["blocks"],
            "s": H.signs_from_bits(sd["mask"], d) if sd["mask"] is not None else None,
            "precondition": sd["precondition"]}


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_two_sided(dt):
    """A 320 x 4096 weight: the input side the radix-16 schedule with the
    RHT preconditioning, the output side 8 * 8 * 5; and a 4096 x 5120 bf16
    weight with the page's 8 * 8 * 8 * 5 * 2 schedule on the input side."""
    rng = np.random.default_rng(7 if dt == torch.float32 else 8)
    cases = [((8, 8, 5), False, (16, 16, 16), True)]
    if dt == torch.bfloat16:
        cases.append(((16, 16, 16), True, (8, 8, 8, 5, 2), False))
    for rout, pout, rin, pin in cases:
        so, si = _side(rng, rout, pout), _side(rng, rin, pin)
        d_out, d_in = int(np.prod(rout)), int(np.prod(rin))
        w = (0.02 * rng.standard_t(3, size=(d_out, d_in))).astype(np.float32)
        w_dev = torch.from_numpy(w).to("cuda").to(dt)
        got = host64(_two_sided_gpu(w_dev, so, si))
        want = harp.harp_two_sided(host64(w_dev), _oracle_side(so), _oracle_side(si))
        err = compare.float_err(got, want)[0]
        assert err <= (TOL_F32 if dt == torch.float32 else TOL), (rout, rin, err)


@pytest.mark.parametrize("radices,pre", [((16, 8, 8), False), ((8, 8, 8, 4), True), ((5, 5, 5, 8, 2), False),
                                         ((2, 8, 2), False), ((8, 8, 8), True)])
def test_small_tiles_matrix_cores(radices, pre):
    """bf16 rows of small d with a mean radix of at least 4 run on the matrix
    cores in 16-token tiles: token counts around the tile, fp16 blocks against
    the oracle, fp32 blocks giving the same bits (rounded to fp16 the same
    way), and rows of very different magnitudes."""
    d = int(np.prod(radices))
    rng = np.random.default_rng(d + len(radices))
    blocks = rand_blocks(rng, radices)
    b16 = [np.asarray(b, np.float16).astype(np.float32) for b in blocks]
    mask = synth.sign_bits_to_mask(rng.integers(0, 2, d)) if pre else None
    s = H.signs_from_bits(mask, d) if pre else None
    for tokens in (1, 15, 16, 17, 40):
        x = synth.to_bf16(rng.standard_normal((tokens, d)))
        y16 = run(x, radices, blocks, mask=mask, pre=pre, bdt=torch.float16)
        y32 = run(x, radices, blocks, mask=mask, pre=pre, bdt=torch.float32)
        assert torch.equal(y16.cpu(), y32.cpu())
        want = harp.harp_rotate(synth.bf16_to_f64(x), list(radices), b16, s=s, precondition=pre)
        err = compare.float_err(host64(y16), want)[0]
        assert err <= 1e-2, (tokens, err)
    x = np.zeros((5, d))
    x[0, 2] = 3.0e4
    keep = (np.arange(d) % 8) >= 2
    x[1, keep] = rng.standard_normal(keep.sum()) * 1e20
    x[2, keep] = rng.standard_normal(keep.sum()) * 1e-20
    x[3, 5::8] = 1e3
    x[4] = rng.standard_normal(d)
    x = synth.to_bf16(x)
    y = host64(run(x, radices, blocks, mask=mask, pre=pre, bdt=torch.float16))
    assert np.isfinite(y).all()
    want = harp.harp_rotate(synth.bf16_to_f64(x), list(radices), b16, s=s, precondition=pre)
    assert compare.float_err(y, want)[0] <= 1e-2

"""Pins of the oracle's QWHA adapter and HARP rotation: special cases that
reduce to the plain WHT / identity, single-nonzero and permutation cases
predicted position by position, brute-force loops on tiny shapes, norm
preservation and exact inversion."""
import numpy as np
import pytest

from oracle import hadamard as H, qwha, harp
from golden_io import rows, ints


def brute_wht(x):
    n = x.shape[-1]
    out = np.zeros_like(x, dtype=np.float64)
    for i in range(n):
        for j in range(n):
            sgn = -1.0 if bin(i & j).count("1") % 2 else 1.0
            out[..., i] += sgn * x[..., j]
    return out / np.sqrt(n)


def dense_to_csr(f):
    r, c = np.nonzero(f)
    return qwha.coo_to_csr(r, c, f[r, c], f.shape[0])


# ------------------------------------------------------------------- QWHA

def test_qwha_identity_and_involution():
    rng = np.random.default_rng(0)
    n = 256
    x = rng.standard_normal((5, n))
    rp, ci, v = dense_to_csr(np.eye(n))
    assert np.allclose(qwha.qwha_forward(x, rp, ci, v, n), H.wht(x), atol=1e-12)
    hn = H.sylvester(n) / np.sqrt(n)
    rp, ci, v = dense_to_csr(hn)
    assert np.allclose(qwha.qwha_forward(x, rp, ci, v, n), x, atol=1e-12)


def test_qwha_single_nonzero():
    rng = np.random.default_rng(1)
    n, o, k, val = 64, 17, 40, -0.375
    x = rng.standard_normal((3, n))
    y = qwha.qwha_forward(x, np.r_[np.zeros(o + 1, int), np.ones(n - o, int)],
                          np.array([k]), np.array([val]), n)
    want = np.zeros((3, n)); want[:, o] = val * H.wht(x)[:, k]
    assert np.allclose(y, want, atol=1e-14)


@pytest.mark.parametrize("d_in,d_out", [(8, 8), (16, 12), (4, 16)])
def test_qwha_bruteforce(d_in, d_out):
    rng = np.random.default_rng(d_in * 100 + d_out)
    x = rng.standard_normal((4, d_in))
    nnz = d_out * 3
    r = rng.integers(0, d_out, nnz)
    c = rng.integers(0, d_in, nnz)
    keep = np.unique(r * d_in + c, return_index=True)[1]
    r, c = r[keep], c[keep]
    v = rng.standard_normal(r.size)
    rp, ci, vv = qwha.coo_to_csr(r, c, v, d_out)
    assert np.all(np.diff(rp) >= 0) and rp[-1] == r.size
    z = brute_wht(x)
    want = np.zeros((4, d_out))
    for o in range(d_out):
        for e in range(rp[o], rp[o + 1]):
            want[:, o] += vv[e] * z[:, ci[e]]
    assert np.allclose(qwha.qwha_forward(x, rp, ci, vv, d_out), want, atol=1e-12)


def random_csr(rng, d_out, d_in, per_row):
    r = np.repeat(np.arange(d_out), per_row)
    c = np.concatenate([rng.choice(d_in, per_row, replace=False) for _ in range(d_out)])
    return qwha.coo_to_csr(r, c, rng.standard_normal(r.size), d_out)


@pytest.mark.parametrize("d_in,d_out", [(64, 48), (256, 256), (16, 40)])
def test_qwha_backward_input_is_the_adjoint(d_in, d_out):
    # <y(x), dy> = <x, dx(dy)> for the linear map x -> y: pins the backward
    # to the forward without restating either
    rng = np.random.default_rng(d_in + d_out)
    rp, ci, v = random_csr(rng, d_out, d_in, min(5, d_in))
    x = rng.standard_normal((7, d_in))
    dy = rng.standard_normal((7, d_out))
    y = qwha.qwha_forward(x, rp, ci, v, d_out)
    dx = qwha.qwha_backward_input(dy, rp, ci, v, d_in)
    assert np.isclose(np.sum(y * dy), np.sum(x * dx), rtol=1e-12, atol=1e-12)


def test_qwha_grad_values_finite_differences():
    # the forward is linear in each value: moving c_e by 1 changes <y, dy> by dc_e
    rng = np.random.default_rng(5)
    d_in, d_out = 32, 24
    rp, ci, v = random_csr(rng, d_out, d_in, 4)
    x = rng.standard_normal((6, d_in))
    dy = rng.standard_normal((6, d_out))
    base = np.sum(qwha.qwha_forward(x, rp, ci, v, d_out) * dy)
    dc = qwha.qwha_grad_values(x, dy, rp, ci)
    for e in range(len(v)):
        v2 = v.copy(); v2[e] += 1.0
        assert np.isclose(np.sum(qwha.qwha_forward(x, rp, ci, v2, d_out) * dy) - base, dc[e], atol=1e-11)


@pytest.mark.parametrize("d_in,d_out", [(8, 8), (16, 12)])
def test_qwha_backward_bruteforce(d_in, d_out):
    rng = np.random.default_rng(d_in * 7 + d_out)
    rp, ci, v = random_csr(rng, d_out, d_in, 3)
    x = rng.standard_normal((3, d_in))
    dy = rng.standard_normal((3, d_out))
    dz = np.zeros((3, d_in))
    dc = np.zeros(len(v))
    z = brute_wht(x)
    for o in range(d_out):
        for e in range(rp[o], rp[o + 1]):
            dz[:, ci[e]] += v[e] * dy[:, o]
            dc[e] = np.dot(dy[:, o], z[:, ci[e]])
    assert np.allclose(qwha.qwha_backward_input(dy, rp, ci, v, d_in), brute_wht(dz), atol=1e-12)
    assert np.allclose(qwha.qwha_grad_values(x, dy, rp, ci), dc, atol=1e-12)


def test_qwha_backward_identity_f():
    rng = np.random.default_rng(9)
    n = 128
    rp, ci, v = dense_to_csr(np.eye(n))
    x = rng.standard_normal((4, n)); dy = rng.standard_normal((4, n))
    assert np.allclose(qwha.qwha_backward_input(dy, rp, ci, v, n), H.wht(dy), atol=1e-12)
    assert np.allclose(qwha.qwha_grad_values(x, dy, rp, ci), np.sum(dy * H.wht(x), axis=0), atol=1e-12)


def test_csr_transpose():
    rng = np.random.default_rng(11)
    d_out, d_in = 20, 12
    rp, ci, v = random_csr(rng, d_out, d_in, 3)
    trp, tci, tv, perm = qwha.csr_transpose(rp, ci, v, d_in)
    assert np.array_equal(qwha.csr_to_dense(trp, tci, tv, d_in, d_out), qwha.csr_to_dense(rp, ci, v, d_out, d_in).T)
    assert np.array_equal(tv, np.asarray(v)[perm])
    for k in range(d_in):  # rows of F^T hold increasing rows of F
        assert np.all(np.diff(tci[trp[k]:trp[k + 1]]) > 0)


# ------------------------------------------------------------------- HARP

def digits(i, radices):
    out = []
    for b in radices:
        out.append(i % b)
        i //= b
    return out


def undigits(dg, radices):
    i, mul = 0, 1
    for dd, b in zip(dg, radices):
        i += dd * mul
        mul *= b
    return i


def brute_stage(z, blocks_t, t, radices):
    """out[i] = sum_k B_{t,c}[i_t, k] z[i with digit t := k], with c the
    remaining digits in increasing significance."""
    d = z.shape[-1]
    out = np.zeros_like(z)
    for i in range(d):
        dg = digits(i, radices)
        rest = [dd for u, dd in enumerate(dg) if u != t]
        rad_rest = [b for u, b in enumerate(radices) if u != t]
        c = undigits(rest, rad_rest)
        for k in range(radices[t]):
            j = list(dg); j[t] = k
            out[..., i] += blocks_t[c, dg[t], k] * z[..., undigits(j, radices)]
    return out


@pytest.mark.parametrize("radices", [(4, 4), (2, 2, 2), (5, 3, 2), (2, 4, 3)])
def test_harp_bruteforce(radices):
    rng = np.random.default_rng(sum(radices))
    d = int(np.prod(radices))
    blocks = [rng.standard_normal((d // b, b, b)) for b in radices]
    x = rng.standard_normal((3, d))
    z = x.copy()
    for t in range(len(radices)):
        z = brute_stage(z, blocks[t], t, radices)
    got = harp.harp_rotate(x, radices, blocks, precondition=False)
    assert np.allclose(got, z, atol=1e-12)


@pytest.mark.parametrize("b,m", [(4, 2), (2, 3), (4, 3), (16, 2), (16, 3)])
def test_harp_hadamard_blocks_equal_wht(b, m):
    """Theta = 0: every block is the normalised Sylvester H_b, and the stages
    compose to exactly the length-d Sylvester WHT under this digit convention."""
    d = b ** m
    hb = H.sylvester(b) / np.sqrt(b)
    blocks = [np.broadcast_to(hb, (d // b, b, b)) for _ in range(m)]
    rng = np.random.default_rng(b * 10 + m)
    x = rng.standard_normal((4, d))
    assert np.allclose(harp.harp_rotate(x, [b] * m, blocks, precondition=False),
                       H.wht(x), atol=1e-12)
    s = 1.0 - 2.0 * rng.integers(0, 2, d)
    eye = [np.broadcast_to(np.eye(b), (d // b, b, b)) for _ in range(m)]
    assert np.allclose(harp.harp_rotate(x, [b] * m, eye, s=s, precondition=True),
                       H.rht(x, s), atol=1e-12)
    assert np.allclose(harp.harp_rotate(x, [b] * m, eye, precondition=False), x)


def test_harp_permutation_blocks_at_real_shape():
    """Identity blocks except one permutation block per stage, d = 4096,
    radix 16: the output is the predicted permutation of rht(x), checked
    position by position."""
    rad = [16, 16, 16]
    d = 4096
    rng = np.random.default_rng(42)
    s = 1.0 - 2.0 * rng.integers(0, 2, d)
    blocks, perms, which = [], [], []
    for t in range(3):
        bl = np.broadcast_to(np.eye(16), (256, 16, 16)).copy()
        c = int(rng.integers(0, 256))
        p = rng.permutation(16)
        bl[c] = np.eye(16)[p]             # out_sub[k] = in_sub[p[k]]
        blocks.append(bl); perms.append(p); which.append(c)
    x = rng.standard_normal((2, d))
    got = harp.harp_rotate(x, rad, blocks, s=s, precondition=True)
    z = H.rht(x, s)
    for t in range(3):
        nz = z.copy()
        for i in range(d):
            dg = digits(i, rad)
            rest = [dd for u, dd in enumerate(dg) if u != t]
            if undigits(rest, [16, 16]) == which[t]:
                j = list(dg); j[t] = perms[t][dg[t]]
                nz[:, i] = z[:, undigits(j, rad)]
        z = nz
    assert np.array_equal(got, z)


def test_harp_orthogonal_norm_and_inverse():
    rad = [8, 8, 8, 5, 2]
    d = 5120
    rng = np.random.default_rng(3)
    blocks = []
    for b in rad:
        q, r = np.linalg.qr(rng.standard_normal((d // b, b, b)))
        blocks.append(q)
    x = rng.standard_normal((3, d))
    y = harp.harp_rotate(x, rad, blocks, precondition=False)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    z = y
    for t in reversed(range(len(rad))):
        z = z @ harp.stage_matrix(np.transpose(blocks[t], (0, 2, 1)), t, rad).T
    assert np.allclose(z, x, atol=1e-12)


def test_harp_schedule_golden():
    for d, rad, ok in rows("harp_schedule.txt"):
        d, rad, ok = int(d), ints(rad), bool(int(ok))
        if ok:
            harp.check_schedule(rad, d)
        else:
            with pytest.raises(ValueError):
                harp.check_schedule(rad, d)


# ------------------------------------------- HARP block parametrisation

@pytest.mark.parametrize("b", [3, 4, 5, 8, 11, 16])
def test_cayley_orthogonal_det_one_and_zero(b):
    rng = np.random.default_rng(b)
    a = harp.skew_from_params(0.3 * rng.standard_normal(b * (b - 1) // 2), b)
    assert np.allclose(a, -a.T)
    q = harp.cayley(a)
    assert np.allclose(q.T @ q, np.eye(b), atol=1e-12)
    assert np.isclose(np.linalg.det(q), 1.0)
    assert np.array_equal(harp.cayley(np.zeros((b, b))), np.eye(b))
    # the Cayley map is its own inverse on orthogonal matrices without -1 eigenvalues
    back = (np.eye(b) - q) @ np.linalg.inv(np.eye(b) + q)
    assert np.allclose(back, a, atol=1e-10)


def test_cayley_2x2_closed_form():
    """A = [[0, a], [-a, 0]]: (I - A)(I + A)^-1 = [[1 - a^2, -2a], [2a, 1 - a^2]] / (1 + a^2),
    the rotation by 2 atan(a); a = 1 is the quarter turn [[0, -1], [1, 0]]."""
    for a in (0.25, -0.7, 1.0, 3.0):
        q = harp.cayley(harp.skew_from_params([a], 2))
        want = np.array([[1 - a * a, -2 * a], [2 * a, 1 - a * a]]) / (1 + a * a)
        assert np.allclose(q, want, atol=1e-14)
        assert np.allclose(q, harp.givens(2 * np.arctan(a)), atol=1e-14)
    assert np.allclose(harp.cayley(harp.skew_from_params([1.0], 2)), [[0, -1], [1, 0]], atol=1e-15)


def test_skew_parameter_order():
    """Parameters fill the strict upper triangle row by row."""
    a = harp.skew_from_params([1, 2, 3, 4, 5, 6], 4)
    assert a[0, 1] == 1 and a[0, 2] == 2 and a[0, 3] == 3 and a[1, 2] == 4 and a[1, 3] == 5 and a[2, 3] == 6
    assert a[3, 2] == -6 and np.all(np.diag(a) == 0)


def test_givens_closed_form():
    assert np.allclose(harp.givens(np.pi / 2), [[0, -1], [1, 0]], atol=1e-15)
    assert np.allclose(harp.givens(0.3) @ harp.givens(0.4), harp.givens(0.7), atol=1e-15)


def test_build_blocks_theta_zero_is_the_mixer():
    """Theta = 0 gives B = G: with Sylvester mixers the rotation is the WHT
    ([HARP] 2.2: the fixed RHT is recovered at initialisation)."""
    radices, d = [4, 2, 8], 64
    n = sum((d // b) * harp.params_per_block(b) for b in radices)
    blocks = harp.build_blocks(np.zeros(n), radices, d)
    for b, blk in zip(radices, blocks):
        assert np.array_equal(blk, np.broadcast_to(harp.sylvester_mixer(b), blk.shape))
    x = np.random.default_rng(0).standard_normal((3, d))
    assert np.allclose(harp.harp_rotate(x, radices, blocks, precondition=False), H.wht(x), atol=1e-12)


def test_build_blocks_single_parameter_placement():
    """One nonzero parameter touches one block of one stage."""
    radices, d = [5, 2, 3], 30
    mix = [np.linalg.qr(np.random.default_rng(b).standard_normal((b, b)))[0] for b in radices]
    sizes = [(d // b) * harp.params_per_block(b) for b in radices]
    p = np.zeros(sum(sizes))
    t, c, k = 0, 4, 7          # stage 0 (b = 5, 10 params per block), block 4, parameter 7 = A[2][3]
    p[c * 10 + k] = 0.5
    blocks = harp.build_blocks(p, radices, d, mix)
    for tt, (b, blk) in enumerate(zip(radices, blocks)):
        for cc in range(d // b):
            same = np.allclose(blk[cc], mix[tt])
            assert same == (not (tt == t and cc == c))
    a = np.zeros((5, 5)); a[2, 3], a[3, 2] = 0.5, -0.5
    assert np.allclose(blocks[0][c], harp.cayley(a) @ mix[0])
    # stage 1 (b = 2): a Givens angle
    p = np.zeros(sum(sizes)); p[sizes[0] + 6] = 0.9
    blocks = harp.build_blocks(p, radices, d, mix)
    assert np.allclose(blocks[1][6], harp.givens(0.9) @ mix[1])


def test_dequant_params():
    radices, d = [2, 4], 8
    q = np.arange(-4, 4 + 6 * 2 - 4, dtype=np.int8)[: 4 * 1 + 2 * 6]
    th = harp.dequant_params(q, [0.5, 0.25], radices, d)
    assert np.allclose(th[:4], 0.5 * q[:4]) and np.allclose(th[4:], 0.25 * q[4:])

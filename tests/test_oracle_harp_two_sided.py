"""Pins of the two-sided HARP oracle W~ = R_out W R_in^T ([HARP] technical
summary: a learnable two-sided orthogonal processor): a brute-force quadruple
loop over stage loops written independently of the oracle's stage matrices,
Theta = 0 giving the two-sided Hadamard / RHT, exact orthogonality and
inversion, and the one-sided special case."""
import numpy as np
import pytest

from oracle import hadamard as H, harp
from test_oracle_qwha_harp import brute_stage


def orth64(rng, nb, b):
    """nb orthogonal b x b blocks in fp64 (QR of Gaussians, column signs fixed)."""
    out = np.empty((nb, b, b))
    for c in range(nb):
        q, r = np.linalg.qr(rng.standard_normal((b, b)))
        out[c] = q * np.sign(np.diag(r))
    return out


def side(rng, radices, precondition=False):
    d = int(np.prod(radices))
    blocks = [orth64(rng, d // b, b) for b in radices]
    s = rng.choice([-1.0, 1.0], d) if precondition else None
    return {"radices": list(radices), "blocks": blocks, "s": s, "precondition": precondition}


def brute_rotate_vec(v, sd):
    z = np.asarray(v, dtype=np.float64)
    for t in range(len(sd["radices"])):
        z = brute_stage(z, sd["blocks"][t], t, sd["radices"])
    return z


@pytest.mark.parametrize("rout,rin", [((3, 2), (2, 4)), ((2, 2, 2), (5, 3)), ((4,), (2, 3, 2))])
def test_two_sided_bruteforce(rout, rin):
    rng = np.random.default_rng(len(rout) * 10 + len(rin))
    so, si = side(rng, rout), side(rng, rin)
    d_out, d_in = int(np.prod(rout)), int(np.prod(rin))
    w = rng.standard_normal((d_out, d_in))
    # R_in on every row, then R_out on every column, each by explicit stage loops
    t = np.array([brute_rotate_vec(w[a], si) for a in range(d_out)])
    want = np.array([brute_rotate_vec(t[:, j], so) for j in range(d_in)]).T
    got = harp.harp_two_sided(w, so, si)
    assert np.allclose(got, want, atol=1e-12)
    # element by element: W~[i][j] = sum_a sum_b R_out[i][a] W[a][b] R_in[j][b]
    ro = np.array([brute_rotate_vec(e, so) for e in np.eye(d_out)]).T
    ri = np.array([brute_rotate_vec(e, si) for e in np.eye(d_in)]).T
    i, j = d_out - 1, d_in // 2
    ref = sum(ro[i, a] * w[a, b] * ri[j, b] for a in range(d_out) for b in range(d_in))
    assert abs(got[i, j] - ref) < 1e-12


def test_two_sided_theta_zero_is_two_sided_hadamard_and_rht():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((16, 64))
    had = lambda rad: {"radices": list(rad), "blocks": [np.tile(H.sylvester(b) / np.sqrt(b), (int(np.prod(rad)) // b, 1, 1))
                                                        for b in rad], "s": None, "precondition": False}
    hn16 = H.sylvester(16) / 4.0
    hn64 = H.sylvester(64) / 8.0
    got = harp.harp_two_sided(w, had((4, 4)), had((4, 4, 4)))
    assert np.allclose(got, hn16 @ w @ hn64, atol=1e-12)
    ident = lambda rad, s: {"radices": list(rad), "blocks": [np.tile(np.eye(b), (int(np.prod(rad)) // b, 1, 1))
                                                             for b in rad], "s": s, "precondition": True}
    so, si = rng.choice([-1.0, 1.0], 16), rng.choice([-1.0, 1.0], 64)
    got = harp.harp_two_sided(w, ident((4, 4), so), ident((8, 8), si))
    assert np.allclose(got, hn16 @ np.diag(so) @ w @ np.diag(si) @ hn64, atol=1e-12)


def test_two_sided_orthogonal_and_inverse():
    rng = np.random.default_rng(4)
    so, si = side(rng, (8, 8, 8, 5, 2)[:3], True), side(rng, (5, 3, 2))
    w = rng.standard_normal((512, 30))
    got = harp.harp_two_sided(w, so, si)
    assert abs(np.linalg.norm(got) - np.linalg.norm(w)) < 1e-10 * np.linalg.norm(w)
    ro = harp.rotation_matrix(512, **so)
    ri = harp.rotation_matrix(30, **si)
    assert np.allclose(ro.T @ got @ ri, w, atol=1e-11)


def test_two_sided_identity_input_side_is_one_sided():
    rng = np.random.default_rng(5)
    so = side(rng, (4, 2), True)
    w = rng.standard_normal((8, 12))
    ident = {"radices": [12], "blocks": [np.eye(12)[None]], "s": None, "precondition": False}
    got = harp.harp_two_sided(w, so, ident)
    want = harp.harp_rotate(w.T, so["radices"], so["blocks"], s=so["s"], precondition=True).T
    assert np.allclose(got, want, atol=1e-12)

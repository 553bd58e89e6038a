"""The host-side budget allocation of the QWHA initialisation
(qwha_init_allocate, a C call on host arrays) against the oracle's
allocation, exactly, on the same fp32 error magnitudes."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import qwha_init as QI

EINVAL, EUNSUP = 1, 2


@pytest.fixture(scope="module")
def lib():
    from wht_adapters_amd import whtq
    return whtq.raw()


def alloc(lib, err, n, total, floor, cap):
    e = np.ascontiguousarray(err, dtype=np.float32)
    rp = np.zeros(e.size + 1, dtype=np.int32)
    st = lib.qwha_init_allocate(e.ctypes.data_as(ctypes.c_void_p), e.size, n, total, floor, cap,
                                rp.ctypes.data_as(ctypes.c_void_p))
    return st, rp


def test_allocate_hand_worked(lib):
    for e, p, fl, cap, want in (([1, 2, 3, 4], 20, 2, 10, [2, 4, 6, 8]),
                                ([0.1, 1, 1, 1], 12, 2, 10, [2, 4, 3, 3]),
                                ([100, 1, 1], 12, 1, 6, [6, 3, 3]),
                                ([0, 0, 0, 0], 10, 1, 8, [3, 3, 2, 2])):
        st, rp = alloc(lib, e, 64, p, fl, cap)
        assert st == 0
        assert np.diff(rp).tolist() == want


@pytest.mark.parametrize("seed", range(12))
def test_allocate_matches_oracle(lib, seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 3000))
    # error magnitudes as the device produces them: fp32, log-normal spread,
    # a few exact repeats and a few zeros
    e = np.exp(1.5 * rng.standard_normal(m)).astype(np.float32)
    if m > 10:
        e[rng.integers(0, m, 5)] = e[0]
        e[rng.integers(0, m, 3)] = 0.0
    floor = int(rng.integers(0, 16))
    cap = int(rng.integers(max(floor, 1), 129))
    p = int(rng.integers(floor * m, cap * m + 1))
    st, rp = alloc(lib, e, 4096, p, floor, cap)
    try:
        want = QI.allocate(e.astype(np.float64), p, floor, cap)
    except (ValueError, AssertionError):
        want = None
    if want is None or not np.isfinite(QI._water_level(e.astype(np.float64), p, floor, cap)):
        assert st == EINVAL
        return
    assert st == 0
    assert rp[0] == 0
    assert np.array_equal(np.diff(rp), want)


def test_allocate_statuses(lib):
    e = np.ones(8, dtype=np.float32)
    assert alloc(lib, e, 64, 8 * 3 - 1, 3, 10)[0] == EINVAL      # below floor * rows
    assert alloc(lib, e, 64, 8 * 10 + 1, 3, 10)[0] == EINVAL     # above cap * rows
    assert alloc(lib, e, 64, 40, 6, 5)[0] == EINVAL              # floor > cap
    assert alloc(lib, e, 8, 40, 3, 9)[0] == EINVAL               # cap > n
    assert alloc(lib, e, 4096, 8 * 129, 3, 129)[0] == EUNSUP     # cap above the refinement's limit
    bad = e.copy()
    bad[3] = np.nan
    assert alloc(lib, bad, 64, 40, 3, 10)[0] == EINVAL
    bad[3] = -1.0
    assert alloc(lib, bad, 64, 40, 3, 10)[0] == EINVAL
    # zero-error channels stay at the floor: 6 * 10 + 2 * 2 < 70 is unreachable
    z = e.copy()
    z[:2] = 0.0
    assert alloc(lib, z, 64, 70, 2, 10)[0] == EINVAL
    assert alloc(lib, z, 64, 64, 2, 10)[0] == 0

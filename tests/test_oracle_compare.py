"""Pins of the parity rules in oracle/compare.py (CPU only).

Every GPU parity test decides pass or fail through these rules, so each one
is pinned here by hand-worked values:

  * the code exemption window |v - b| <= 1e-6 |b| around the nearest
    half-integer b (not the nearest integer, not an absolute window);
  * the scale exemption only at the midpoint of two *adjacent* fp16 values;
  * in a scale-exempt group the codes are re-derived with the device's
    scale, not the oracle's;
  * the exempt-count budget of 1e-4 of all elements;
  * the float error floored at the row RMS of the oracle output, not the
    matrix RMS and not the bare element.
"""
import numpy as np

from oracle import compare as C
from oracle import rtn


def test_near_boundary_hand_worked():
    v = np.array([2.5 + 2e-6,      # |v-b| = 2e-6 <= 2.5e-6: inside
                  2.5 + 3e-6,      # 3e-6 > 2.5e-6: outside
                  -0.5 - 4e-7,     # b = -0.5, window 5e-7: inside
                  -0.5 - 6e-7,     # outside (an absolute 1e-6 window would take it)
                  3.0,             # an integer is half a step from any boundary
                  0.0,
                  1e-7,
                  7.5 * (1 + 9e-7),
                  7.5 * (1 + 1.1e-6),
                  -6.5 * (1 + 5e-7)])
    want = np.array([True, False, True, False, False, False, False, True, False, True])
    assert np.array_equal(C.near_boundary(v), want)


def test_fp16_midpoint_adjacency():
    lo, hi = np.float16(1.0), np.float16(1.0009765625)     # adjacent: ulp 2^-10
    mid = (float(lo) + float(hi)) / 2
    assert C._fp16_midpoint_exempt(mid, lo, hi)
    assert C._fp16_midpoint_exempt(mid * (1 + 9e-7), hi, lo)
    assert not C._fp16_midpoint_exempt(mid * (1 + 2e-6), lo, hi)
    # two ulps apart: 1.0009765625 is their mean, but it is an fp16 value,
    # not a rounding midpoint, so no device may pick either neighbour
    far = np.float16(1.001953125)
    assert not C._fp16_midpoint_exempt(1.0009765625, lo, far)
    # adjacency across a binade boundary: 1 - 2^-11 and 1.0
    below = np.float16(0.99951171875)
    assert C._fp16_midpoint_exempt((0.99951171875 + 1.0) / 2, below, lo)


def _quant_case(y, bits, group):
    q, s16, v, s_pre = rtn.quantize_rtn(y, bits, group)
    return q, s16, v, s_pre


def test_compare_quant_scale_exempt_rederives_with_device_scale():
    # absmax 7 * 1.00048828125 puts s_pre exactly on the midpoint between the
    # adjacent fp16 values 1.0 and 1 + 2^-10; round-half-even gives 1.0
    a = 7 * 1.00048828125
    y = np.array([[a, 2.5005, -1.2, 0, 0, 0, 0, 0.3]])
    q, s16, v, s_pre = _quant_case(y, 4, 8)
    assert float(s16[0, 0]) == 1.0 and s_pre[0, 0] == 1.00048828125
    assert q[0, 1] == 3                      # 2.5005 / 1.0
    s_dev = np.array([[1.0009765625]], dtype=np.float16)
    q_dev = np.clip(np.rint(y / 1.0009765625), -7, 7)   # 2.4980... -> 2
    assert q_dev[0, 1] == 2
    rep = C.compare_quant(q_dev, s_dev, y, s16, q, v, s_pre, 4, 8)
    assert rep["scale_exempt_groups"] == 1 and rep["scale_failures"] == 0
    assert rep["code_mismatch"] == 0 and rep["code_failures"] == 0 and rep["ok"]
    # the device codes taken with the oracle's scale would now be wrong
    rep2 = C.compare_quant(q.copy(), s_dev, y, s16, q, v, s_pre, 4, 8)
    assert rep2["code_failures"] == 1 and not rep2["ok"]
    # a scale two ulps away is a failure, not an exemption
    rep3 = C.compare_quant(q_dev, np.array([[1.001953125]], dtype=np.float16),
                           y, s16, q, v, s_pre, 4, 8)
    assert rep3["scale_failures"] == 1 and rep3["scale_exempt_groups"] == 0 and not rep3["ok"]


def test_compare_quant_code_window_and_budget():
    rows, n = 2048, 8
    y = np.zeros((rows, n))
    y[:, 0] = 7.0                            # s_pre = 1 exactly, s16 = 1.0
    y[5, 1] = 2.5 + 1e-6                     # v within 2.5e-6 of 2.5: exempt
    q, s16, v, s_pre = _quant_case(y, 4, 8)
    assert np.all(s16 == 1.0) and q[5, 1] == 3
    q_dev = q.copy()
    q_dev[5, 1] = 2
    rep = C.compare_quant(q_dev, s16, y, s16, q, v, s_pre, 4, 8)
    assert rep["elements"] == 16384 and rep["exempt_codes"] == 1
    assert rep["code_failures"] == 0 and rep["exempt_frac"] == 1 / 16384 and rep["ok"]
    # a second exemption puts the count at 1.22e-4 of the elements: over budget
    y[9, 3] = -(0.5 + 4e-7)
    q, s16, v, s_pre = _quant_case(y, 4, 8)
    q_dev = q.copy()
    q_dev[5, 1] = 2
    assert q[9, 3] == -1
    q_dev[9, 3] = 0
    rep = C.compare_quant(q_dev, s16, y, s16, q, v, s_pre, 4, 8)
    assert rep["exempt_codes"] == 2 and rep["code_failures"] == 0 and not rep["ok"]
    # outside the window a mismatch is a failure
    y2 = y[:1].copy()
    y2[0, 2] = 2.6
    q, s16, v, s_pre = _quant_case(y2, 4, 8)
    q_dev = q.copy()
    q_dev[0, 2] = 2
    rep = C.compare_quant(q_dev, s16, y2, s16, q, v, s_pre, 4, 8)
    assert rep["code_failures"] == 1 and rep["exempt_codes"] == 0 and not rep["ok"]


def test_float_err_row_rms_floor():
    o = np.array([[3.0, 4.0], [300.0, 400.0]])
    # row 0: rms = sqrt(12.5); an error of rms/10 on the element 3 (below the
    # rms) scales to exactly 0.1 -- not 0.118 (bare element), not 0.0014
    # (matrix rms = 250)
    rms0 = np.sqrt(12.5)
    g = o.copy()
    g[0, 0] += rms0 / 10
    e, roww = C.float_err(g, o)
    assert abs(e - 0.1) < 1e-15
    assert abs(roww - (rms0 / 10) / 5.0) < 1e-15
    # above the rms the element itself is the denominator
    o2 = np.array([[10.0, 1e-4, 1e-4, 1e-4]])
    g2 = o2.copy()
    g2[0, 0] += 1.0
    assert abs(C.float_err(g2, o2)[0] - 0.1) < 1e-12
    # an all-zero row compares absolute differences
    assert C.float_err(np.array([[0.0, 0.5]]), np.zeros((1, 2)))[0] == 0.5

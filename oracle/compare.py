"""Parity rules for comparing a device result with the oracle.
Test infrastructure only.

Codes: bit-exact, except where the oracle's pre-rounding value v lies within
1e-6 relative of a rounding boundary b (the nearest half-integer):
|v - b| <= 1e-6 |b|.  Those are counted as exempt; the exempt count must stay
below 1e-4 of all elements; any other mismatch is a failure.

Scales: bit-exact, except where the oracle's pre-rounding scale s_pre lies
within 1e-6 relative of the fp16 midpoint between the two scales.  In such a
scale-exempt group the oracle codes are re-derived with the device scale and
then checked by the code rule.

Floats: max_i |g_i - o_i| / max(|o_i|, rms(o_row)) <= tol (1e-5 for fp32
outputs, 2e-2 for bf16 outputs).  Reading: a pure elementwise relative
error is unbounded at near-zero outputs of a length-n sum, so the
denominator is floored at the row RMS of the oracle output.
"""

import numpy as np

REL_WINDOW = 1e-6
EXEMPT_BUDGET = 1e-4


def near_boundary(v, window=REL_WINDOW):
    """True where v is within window*|b| of the nearest half-integer b."""
    v = np.asarray(v, dtype=np.float64)
    b = np.floor(v) + 0.5
    return np.abs(v - b) <= window * np.abs(b)


def _fp16_midpoint_exempt(s_pre, s_a, s_b, window=REL_WINDOW):
    a = np.asarray(s_a, dtype=np.float16)
    b = np.asarray(s_b, dtype=np.float16)
    lo = np.minimum(a.astype(np.float64), b.astype(np.float64))
    hi = np.maximum(a.astype(np.float64), b.astype(np.float64))
    adjacent = np.nextafter(lo.astype(np.float16), np.float16(np.inf)).astype(np.float64) == hi
    mid = 0.5 * (lo + hi)
    return adjacent & (np.abs(s_pre - mid) <= window * np.abs(mid))


def compare_quant(q_dev, s_dev, y, s16_or, q_or, v_or, s_pre, bits, group):
    """Compare device codes/scales with the oracle for one matrix.

    q_dev: signed codes from the device [rows, n]; s_dev: device scales as
    float16 [rows, n/g]; y: oracle rotated rows (fp64); the rest from
    rtn.quantize_rtn.  Returns a dict report; report['ok'] is the verdict.
    """
    from .rtn import qmax_of
    rows, n = q_or.shape
    ng = n // group
    s_dev = np.asarray(s_dev, dtype=np.float16)
    s_or = np.asarray(s16_or, dtype=np.float16)
    scale_eq = s_dev.view(np.uint16) == s_or.view(np.uint16)
    scale_ex = (~scale_eq) & _fp16_midpoint_exempt(s_pre, s_dev, s_or)
    scale_fail = (~scale_eq) & (~scale_ex)

    q_ref = q_or.astype(np.int64).copy()
    v_ref = np.asarray(v_or, dtype=np.float64).copy()
    if scale_ex.any():
        qm = qmax_of(bits)
        gr, gc = np.nonzero(scale_ex)
        for r, c in zip(gr, gc):
            sl = slice(c * group, (c + 1) * group)
            sd = float(s_dev[r, c])
            vv = y[r, sl] / sd if sd > 0 else np.zeros(group)
            v_ref[r, sl] = vv
            q_ref[r, sl] = np.clip(np.rint(vv), -qm, qm)

    mism = q_dev.astype(np.int64) != q_ref
    exempt = mism & near_boundary(v_ref)
    fail = mism & ~exempt
    n_el = rows * n
    rep = {
        "elements": int(n_el),
        "groups": int(rows * ng),
        "code_mismatch": int(mism.sum()),
        "exempt_codes": int(exempt.sum()),
        "exempt_frac": float(exempt.sum()) / n_el,
        "code_failures": int(fail.sum()),
        "scale_exempt_groups": int(scale_ex.sum()),
        "scale_failures": int(scale_fail.sum()),
    }
    rep["ok"] = (rep["code_failures"] == 0 and rep["scale_failures"] == 0
                 and rep["exempt_frac"] < EXEMPT_BUDGET)
    return rep


def float_err(g, o):
    """max |g - o| / max(|o|, rms(o_row)) and the max row-wise ||g-o||/||o||."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if g.ndim == 1:
        g, o = g[None], o[None]
    rms = np.sqrt(np.mean(o * o, axis=1, keepdims=True))
    den = np.maximum(np.abs(o), rms)
    den = np.where(den > 0, den, 1.0)
    scaled = np.abs(g - o) / den
    nrm = np.linalg.norm(o, axis=1)
    roww = np.linalg.norm(g - o, axis=1) / np.where(nrm > 0, nrm, 1.0)
    return float(scaled.max()) if scaled.size else 0.0, float(roww.max()) if roww.size else 0.0

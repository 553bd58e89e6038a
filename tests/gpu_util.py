"""Helpers shared by the GPU parity tests (device transfers only)."""
import numpy as np
import torch

DEV = "cuda:0"


def dev(a, dtype=None):
    if isinstance(a, np.ndarray):
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        t = a
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def mask_dev(mask_u32):
    return torch.from_numpy(np.asarray(mask_u32, dtype=np.uint32).view(np.int32).copy()).to(DEV)


def host64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def codes_host(t):
    return t.detach().to("cpu").numpy()


def scales_host(t):
    return t.detach().to("cpu").numpy().astype(np.float16)


def write_report(name, rep):
    """Record a parity report as JSON under $WHTQ_REPORT_DIR (when set), so a
    GPU run can keep the exemption counts the tests measured."""
    import json
    import os
    d = os.environ.get("WHTQ_REPORT_DIR")
    print(f"{name}: {rep}", flush=True)
    if not d:
        return
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, name + ".json"), "w") as f:
        json.dump(rep, f, indent=1, sort_keys=True)


def merge_reports(reps):
    """Sum the counts of compare_quant reports over row chunks."""
    from oracle import compare
    out = {}
    for k in ("elements", "groups", "code_mismatch", "exempt_codes", "code_failures",
              "scale_exempt_groups", "scale_failures"):
        out[k] = int(sum(r[k] for r in reps))
    out["exempt_frac"] = out["exempt_codes"] / max(out["elements"], 1)
    out["ok"] = (out["code_failures"] == 0 and out["scale_failures"] == 0
                 and out["exempt_frac"] < compare.EXEMPT_BUDGET)
    return out

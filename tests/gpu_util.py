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

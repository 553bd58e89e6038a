"""Seeded synthetic inputs for the hot path.

This module only draws random numbers and stores them in the formats the
library takes (fp32 / bf16 rows, a uint32 sign bitmask, CSR, fp32 blocks).
It holds none of the transform or quantiser arithmetic; the HIP library and
the CPU oracle both consume what it produces.

The pages measure on real model weights and benchmark suites that are not
available here; these inputs keep the model shapes (hidden 4096 of the 7B/8B
models, a 28672 x 8192 MLP projection of a 70B model) and the value
structure the pages describe: heavy-tailed weights with outlier columns
(HARP page, section 1), activation outlier channels, and a per-row sparse
budget proportional to an error magnitude with a floor (QWHA page, 2.2).

Seeding: every tensor of workload `cfg` uses
np.random.default_rng(np.random.SeedSequence(0, spawn_key=(cfg, k))) with a
fixed k per tensor; the 256 x 4096 fp32 WHT workload uses default_rng(0).
Draws are fp64 and rounded once to the storage type (bf16 round-to-nearest-
even through torch on the CPU).
"""

import hashlib

import numpy as np
import torch


def child_rng(cfg, k):
    return np.random.default_rng(np.random.SeedSequence(0, spawn_key=(cfg, k)))


def to_bf16(a):
    """fp64/fp32 numpy -> torch.bfloat16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f64(t):
    return t.to(torch.float64).numpy()


def sign_bits_to_mask(bits01):
    """0/1 array (1 means s_j = -1) -> uint32 words, LSB first."""
    bits01 = np.asarray(bits01, dtype=np.uint8)
    n = bits01.size
    pad = (-n) % 32
    b = np.concatenate([bits01, np.zeros(pad, np.uint8)])
    return np.packbits(b, bitorder="little").view("<u4").astype(np.uint32)


def sha256(a):
    if isinstance(a, torch.Tensor):
        a = a.contiguous().view(torch.uint8).numpy() if a.dtype != torch.uint8 else a.numpy()
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


# ---------------------------------------------------------------- primitives

def gaussian_rows(rng, rows, n, chunk=4096):
    out = np.empty((rows, n), dtype=np.float32)
    for r in range(0, rows, chunk):
        out[r:r + chunk] = rng.standard_normal((min(chunk, rows - r), n))
    return out


def student_t_rows(rng, rows, n, scale, chunk=2048):
    out = np.empty((rows, n), dtype=np.float32)
    for r in range(0, rows, chunk):
        out[r:r + chunk] = scale * rng.standard_t(3, (min(chunk, rows - r), n))
    return out


def heavy_weights(cfg, rows, n, n_outlier_cols, factor=20.0):
    """0.02 * Student-t(3) with n_outlier_cols columns scaled by factor -> bf16."""
    w = student_t_rows(child_rng(cfg, 0), rows, n, 0.02)
    cols = child_rng(cfg, 1).choice(n, n_outlier_cols, replace=False)
    w[:, cols] *= factor
    return to_bf16(w), cols


def rademacher_mask(cfg, k, n):
    bits = child_rng(cfg, k).integers(0, 2, n)
    return sign_bits_to_mask(bits)


def allocate_nnz(r, total, floor=8, cap=None):
    """Integer per-row budgets n_o ~ max(floor, lam * r_o) summing to total.

    lam by bisection on the real-valued sum, then floor + largest remainder
    (ties to the lower row index).
    """
    r = np.asarray(r, dtype=np.float64)
    m = r.size
    if floor * m > total:
        raise ValueError("floor * rows exceeds the total budget")
    lo, hi = 0.0, total / r.min() + 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.maximum(floor, mid * r).sum() > total:
            hi = mid
        else:
            lo = mid
    real = np.maximum(floor, lo * r)
    base = np.floor(real).astype(np.int64)
    rem = int(total - base.sum())
    frac = real - base
    order = np.argsort(-frac, kind="stable")
    base[order[:rem]] += 1
    if cap is not None and base.max() > cap:
        raise ValueError("row budget exceeds the cap")
    return base


def sparse_adapter(cfg, d_out, d_in, nnz_total, floor=8, val_std=0.1):
    """CSR F [d_out x d_in]: per-row nnz proportional to a log-normal(0,1)
    error norm with a floor, columns uniform without replacement (sorted),
    values N(0, var 0.01) -> bf16."""
    r = np.exp(child_rng(cfg, 1).standard_normal(d_out))
    counts = allocate_nnz(r, nnz_total, floor=floor, cap=d_in)
    rng_c = child_rng(cfg, 2)
    cols = np.empty(nnz_total, dtype=np.int32)
    row_ptr = np.zeros(d_out + 1, dtype=np.int32)
    np.cumsum(counts, out=row_ptr[1:])
    for o in range(d_out):
        c = rng_c.choice(d_in, counts[o], replace=False)
        c.sort()
        cols[row_ptr[o]:row_ptr[o + 1]] = c
    vals = to_bf16(val_std * child_rng(cfg, 3).standard_normal(nnz_total))
    return row_ptr, cols, vals


def orthogonal_blocks(rng, count, b):
    """count random b x b orthogonal matrices: QR of a Gaussian, Q's columns
    sign-fixed by diag(R) -> fp32 [count, b, b]."""
    g = rng.standard_normal((count, b, b))
    q, r = np.linalg.qr(g)
    d = np.sign(np.diagonal(r, axis1=1, axis2=2))
    d[d == 0] = 1.0
    return (q * d[:, None, :]).astype(np.float32)


# ------------------------------------------------------------ named workloads

WORKLOADS = {
    "fwht_f32_256x4096": "orthonormal FWHT only, fp32, 256 rows x 4096, N(0,1) from seed 0",
    "rht_int4_g128_4096x4096": "RHT + INT4 RTN g=128, bf16 4096 x 4096 Student-t weights",
    "qwha_2048x4096_nnz262144": "QWHA forward, 2048 tokens x 4096, F 4096 x 4096 with 262,144 nnz",
    "qwha_bwd_2048x4096_nnz262144": "QWHA backward (dx and dc), same sizes, upstream dy ~ N(0,1)",
    "harp_8192x4096_r16x3": "HARP: RHT + three radix-16 stages, 8192 tokens x 4096",
    "harp_8192x5120_r88852": "HARP general schedule 8*8*8*5*2, 8192 tokens x 5120 (no preconditioning)",
    "rht_int2_g64_28672x8192": "RHT + INT2 RTN g=64, bf16 28672 x 8192 Student-t weights",
    "gemv_int2_g64_28672x8192_t1": "online-RHT INT2 g=64 product, 28672 x 8192 codes, one decode token",
    "qwha_init_4096x4096_int4_g128_t2048": "QWHA initialisation of a 4096 x 4096 INT4 g=128 layer from "
                                           "2048 calibration tokens, budget 262,144, floor 16, cap 128",
}


def fwht_f32(rows=256, n=4096):
    x = np.random.default_rng(0).standard_normal((rows, n)).astype(np.float32)
    return {"x": x}


def rht_weights(cfg, rows, n, outlier_frac=0.001):
    k = int(round(outlier_frac * n))
    w, cols = heavy_weights(cfg, rows, n, k)
    return {"w": w, "signs": rademacher_mask(cfg, 2, n), "outlier_cols": cols}


def rht_int4_g128(rows=4096, n=4096):
    d = rht_weights(2, rows, n)
    d.update(bits=4, group=128)
    return d


def rht_int2_g64(rows=28672, n=8192):
    d = rht_weights(5, rows, n)
    d.update(bits=2, group=64)
    return d


def qwha(tokens=2048, d_in=4096, d_out=4096, nnz=262144):
    x = to_bf16(gaussian_rows(child_rng(3, 0), tokens, d_in))
    row_ptr, cols, vals = sparse_adapter(3, d_out, d_in, nnz)
    return {"x": x, "row_ptr": row_ptr, "col_idx": cols, "vals": vals, "d_out": d_out}


def qwha_backward(tokens=2048, d_in=4096, d_out=4096, nnz=262144):
    """The QWHA workload plus an upstream gradient dy [tokens, d_out] ~ N(0,1)
    -> bf16 (child stream 4 of the same workload)."""
    d = qwha(tokens, d_in, d_out, nnz)
    d["dy"] = to_bf16(gaussian_rows(child_rng(3, 4), tokens, d_out))
    return d


def harp_general(tokens=8192, radices=(8, 8, 8, 5, 2), outlier_frac=0.005, factor=30.0):
    """The HARP recipe on the page's mixed-radix example d = 5120 = 8*8*8*5*2
    (workload 6): N(0,1) activations with 0.5% channels x30 -> bf16, blocks =
    QR of Gaussians per stage (no sign vector: 5120 is not a power of two,
    so there is no Sylvester preconditioning)."""
    d = int(np.prod(radices))
    x = gaussian_rows(child_rng(6, 0), tokens, d)
    ch = child_rng(6, 1).choice(d, int(round(outlier_frac * d)), replace=False)
    x[:, ch] *= factor
    rng_b = child_rng(6, 3)
    blocks = [orthogonal_blocks(rng_b, d // b, b) for b in radices]
    return {"x": to_bf16(x), "radices": list(radices), "blocks": blocks, "outlier_channels": ch}


def harp(tokens=8192, d=4096, radices=(16, 16, 16), outlier_frac=0.005, factor=30.0):
    x = gaussian_rows(child_rng(4, 0), tokens, d)
    k = int(round(outlier_frac * d))
    ch = child_rng(4, 1).choice(d, k, replace=False)
    x[:, ch] *= factor
    rng_b = child_rng(4, 3)
    blocks = [orthogonal_blocks(rng_b, d // b, b) for b in radices]
    return {"x": to_bf16(x), "signs": rademacher_mask(4, 2, d),
            "radices": list(radices), "blocks": blocks, "outlier_channels": ch}


def lowbit_layer(cfg, rows, n, bits, group, tokens, scale_lo=0.002, scale_hi=0.05,
                 outlier_frac=0.005, factor=30.0):
    """A stored low-bit layer and decode activations for the online-RHT
    product: codes are uniform random bytes (every b-bit field value occurs,
    including the most negative one, which the quantiser never writes), fp16
    scales log-uniform in [scale_lo, scale_hi], activations N(0,1) with a
    fraction of channels x factor (the HARP activation recipe) -> bf16, and a
    Rademacher sign vector.  Streams (cfg, 0..3)."""
    codes = child_rng(cfg, 0).integers(0, 256, size=(rows, n * bits // 8), dtype=np.uint8)
    lg = child_rng(cfg, 1).uniform(np.log(scale_lo), np.log(scale_hi), size=(rows, n // group))
    scales = np.exp(lg).astype(np.float16)
    x = gaussian_rows(child_rng(cfg, 2), tokens, n)
    ch = child_rng(cfg, 3).choice(n, int(round(outlier_frac * n)), replace=False)
    x[:, ch] *= factor
    return {"x": to_bf16(x), "codes": codes, "scales": scales, "signs": rademacher_mask(cfg, 4, n),
            "bits": bits, "group": group}


def gemv_int2_g64(rows=28672, n=8192, tokens=1):
    """Workload 7: decode through the 28672 x 8192 INT2 g=64 layer of workload 5."""
    return lowbit_layer(7, rows, n, 2, 64, tokens)


def qinit_layer(cfg, d_out, n, tokens, bits, group, w_outlier_frac=0.001, x_outlier_frac=0.005, factor=30.0):
    """A layer to initialise an adapter for: bf16 Student-t weights with
    outlier columns (streams (cfg, 0..1)), calibration tokens N(0,1) with a
    fraction of channels x factor -> bf16 (streams (cfg, 2..3)), and a
    Rademacher sign vector (stream (cfg, 4))."""
    w, _ = heavy_weights(cfg, d_out, n, max(1, int(round(w_outlier_frac * n))))
    x = gaussian_rows(child_rng(cfg, 2), tokens, n)
    ch = child_rng(cfg, 3).choice(n, max(1, int(round(x_outlier_frac * n))), replace=False)
    x[:, ch] *= factor
    return {"w": w, "x": to_bf16(x), "signs": rademacher_mask(cfg, 4, n), "bits": bits, "group": group}


def qwha_init_int4_g128(d_out=4096, n=4096, tokens=2048):
    """Workload 8: adapter initialisation of a 4096 x 4096 INT4 g=128 layer
    (budget 64 per channel on average, the QWHA forward workload's 262,144)."""
    d = qinit_layer(8, d_out, n, tokens, 4, 128)
    d.update(total=64 * d_out, floor=16, cap=128)
    return d


#!/usr/bin/env python3
"""Throughput of the MI355X Walsh-Hadamard hot path on one GPU.

Main workload (the one `value` is quoted on): RHT + INT4 round-to-nearest
quantisation, bf16 weight matrix 4096 x 4096, group 128 along d_in, fp16
scales, signed int4 codes -- one `rht_quantize_rtn` launch per step.  The
other workloads (orthonormal FWHT 256 x 4096 fp32, the inverse of the INT4
path, QWHA adapter forward and backward, HARP rotation with the radix-16
schedule and with the mixed-radix 8*8*8*5*2 schedule at d = 5120, 28672 x
8192 RHT + INT2) are timed the same way and reported under "workloads".

Timing: each step processes a different copy of the input, rotating over
copies totalling >= 1 GiB so that inputs come from HBM rather than the
256 MB last-level cache; the K launches are captured once in a HIP graph
(no host launch overhead) and replayed inside a HIP-event pair on the
launch stream.  Data are synthetic (seeded generators in
wht_adapters_amd.synth, whose docstrings give each recipe) with the shapes
and value structure of the workloads.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
GIB = 1 << 30

# algorithmic HBM bytes per launch: inputs read once + outputs written once
ALGO_BYTES = {
    "fwht_f32_256x4096": 2 * 256 * 4096 * 4,
    "rht_int4_g128_4096x4096": 4096 * 4096 * 2 + 512 + 4096 * 2048 + 4096 * 32 * 2,
    "rht_int4_g128_4096x4096_inverse": 4096 * 4096 * 2 + 512 + 4096 * 2048 + 4096 * 32 * 2,
    "qwha_2048x4096_nnz262144": 2 * 2048 * 4096 * 2 + 4097 * 4 + 262144 * 4 + 262144 * 2,
    "harp_8192x4096_r16x3": 2 * 8192 * 4096 * 2 + 3 * 256 * 16 * 16 * 2 + 512,  # fp16 blocks
    # backward to the input: dy in, dx out, the CSR of F^T (row_ptr, col_idx, bf16 values)
    "qwha_bwd_dx_2048x4096_nnz262144": 2 * 2048 * 4096 * 2 + 4097 * 4 + 262144 * 4 + 262144 * 2,
    # gradient of the values: x and dy in, F's row_ptr and col_idx, fp32 dc out
    "qwha_bwd_dc_2048x4096_nnz262144": 2 * 2048 * 4096 * 2 + 4097 * 4 + 262144 * 4 + 262144 * 4,
    "harp_8192x5120_r88852": 2 * 8192 * 5120 * 2 + 5120 * (8 + 8 + 8 + 5 + 2) * 2,  # fp16 blocks
    "rht_int2_g64_28672x8192": 28672 * 8192 * 2 + 1024 + 28672 * 2048 + 28672 * 128 * 2,
    "rht_int2_g64_28672x8192_inverse": 28672 * 8192 * 2 + 1024 + 28672 * 2048 + 28672 * 128 * 2,
    # decode through the INT2 layer: codes + fp16 scales + sign vector + one bf16 token in, bf16 y out
    "gemv_int2_g64_28672x8192_t1": 28672 * 2048 + 28672 * 128 * 2 + 1024 + 8192 * 2 + 28672 * 2,
}
ROWS = {
    "fwht_f32_256x4096": 256, "rht_int4_g128_4096x4096": 4096,
    "rht_int4_g128_4096x4096_inverse": 4096, "qwha_2048x4096_nnz262144": 2048,
    "harp_8192x4096_r16x3": 8192, "rht_int2_g64_28672x8192": 28672,
    "qwha_bwd_dx_2048x4096_nnz262144": 2048, "qwha_bwd_dc_2048x4096_nnz262144": 2048,
    "harp_8192x5120_r88852": 8192,
    "rht_int2_g64_28672x8192_inverse": 28672,
    "gemv_int2_g64_28672x8192_t1": 28672,
}
MAIN = "rht_int4_g128_4096x4096"
KERNEL_SOURCES = {  # sources a workload's kernel is built from (traffic counters go stale with them)
    MAIN: ["rht_quant.hpp", "rq_fwd_b4.hip", "engine.hpp", "io.hpp", "common.hpp", "launch.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "wht_adapters_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(name, launches_bytes):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if name not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    with open(path) as fh:
        tr = json.load(fh).get(name)
    if not tr or tr.get("src_sha") != src_hash(KERNEL_SOURCES[name]):
        return None
    return tr["bytes_per_launch"]


class Timed:
    """K launches of `launch(i)` captured in one HIP graph, replayed between
    two HIP events on the capture stream."""

    def __init__(self, torch, launch, steps, warmup):
        self.torch = torch
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        self.stream = torch.cuda.Stream()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            launch(0)                      # first call on this stream outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph, stream=self.stream):
            for i in range(steps):
                launch(i)
        torch.cuda.synchronize()
        self.steps = steps

    def run(self):
        torch = self.torch
        with torch.cuda.stream(self.stream):
            self.graph.replay()            # untimed replay: pages in the graph
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            # a ~2 ms device-side spin ahead of the start event: the host has queued
            # the whole graph before the GPU reaches e0, so submission latency stays
            # outside the timed region and the per-launch average is kernel time
            torch.cuda._sleep(5_000_000)
            e0.record(self.stream)
            self.graph.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3   # seconds for self.steps launches


def copies(torch, t, total_bytes=GIB, cap=64):
    k = max(2, min(cap, math.ceil(total_bytes / max(1, t.numel() * t.element_size()))))
    return [t.clone() for _ in range(k)]


def result(name, secs, steps):
    per = secs / steps
    gbs = ALGO_BYTES[name] / per / 1e9
    return {"ms_per_launch": per * 1e3, "rows_per_s": ROWS[name] / per, "GBps": gbs,
            "frac_hbm_peak": gbs / PEAK_HBM_GBS, "algo_bytes": ALGO_BYTES[name]}


def bench_quant(torch, W, mask_dev, cfg, name, bits, g, steps, warmup):
    w0 = cfg["w"].to("cuda:0")
    rows, n = w0.shape
    ws = copies(torch, w0)
    sg = mask_dev(cfg["signs"])
    cs = [torch.empty((rows, n * bits // 8), dtype=torch.uint8, device="cuda:0") for _ in ws]
    ss = [torch.empty((rows, n // g), dtype=torch.float16, device="cuda:0") for _ in ws]
    del w0
    fwd = Timed(torch, lambda i: W.rht_quantize_rtn(ws[i % len(ws)], sg, bits, g, cs[i % len(ws)],
                                                    ss[i % len(ws)]), steps, warmup)
    outs = [torch.empty((rows, n), dtype=torch.bfloat16, device="cuda:0") for _ in ws]
    inv = Timed(torch, lambda i: W.rht_dequantize_inverse(cs[i % len(ws)], ss[i % len(ws)], sg, bits, g, n,
                                                          out=outs[i % len(ws)]), steps, warmup)
    r = {name: result(name, fwd.run(), steps)}
    r[name + "_inverse"] = result(name + "_inverse", inv.run(), steps)
    del ws, cs, ss, outs
    torch.cuda.empty_cache()
    return r


def cpu_baseline(cfg, budget_s=12.0):
    """The oracle as it stands, timed on this host on a bounded row sample of
    the main workload."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import hadamard as H, rtn
    from wht_adapters_amd import synth
    w = synth.bf16_to_f64(cfg["w"])
    s = H.signs_from_bits(cfg["signs"], w.shape[1])
    rows_done, t0 = 0, time.perf_counter()
    chunk = 256
    while rows_done < w.shape[0] and time.perf_counter() - t0 < budget_s:
        rtn.rht_quantize(w[rows_done:rows_done + chunk], s, 4, 128)
        rows_done += chunk
    secs = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": rows_done / secs, "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows_done} of 4096 rows of the 4096x4096 INT4 g128 workload "
                      f"(dense fp64 Sylvester product + naive RTN), {secs:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads", default="all",
                    help="all | main | comma list of fwht, qwha, qwha_bwd, harp, harp_gen, int2, gemv, qinit "
                         "(the main workload always runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (PMC calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards rows "
              f"with no communication, so N GPUs would each run this same kernel on rows/N.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from wht_adapters_amd import synth, whtq as W

    def mask_dev(m):
        return torch.from_numpy(np.asarray(m, dtype=np.uint32).view(np.int32).copy()).to("cuda:0")

    torch.cuda.init()
    K, Wm = args.steps, args.warmup
    log(f"[bench] device {torch.cuda.get_device_name(0)}, steps {K}, warmup {Wm}")

    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("[bench] copy probe: 3 x 256 MiB device copy done")

    sel = {"all": {"main", "fwht", "qwha", "qwha_bwd", "harp", "harp_gen", "int2", "gemv", "qinit"},
           "main": {"main"}}.get(
        args.workloads, set(args.workloads.split(",")))
    sel.add("main")  # `value` is always quoted on the main workload
    cfg_main = synth.rht_int4_g128()
    res = bench_quant(torch, W, mask_dev, cfg_main, MAIN, 4, 128, K, Wm)
    log(f"[bench] {MAIN}: {res[MAIN]}")
    if "fwht" in sel:
        x = torch.from_numpy(synth.fwht_f32()["x"]).to("cuda:0")
        xs = copies(torch, x, cap=256)
        ys = [torch.empty_like(x) for _ in xs]
        t = Timed(torch, lambda i: W.wht_batched(xs[i % len(xs)], out=ys[i % len(xs)]), K, Wm)
        res["fwht_f32_256x4096"] = result("fwht_f32_256x4096", t.run(), K)
        log(f"[bench] fwht_f32_256x4096: {res['fwht_f32_256x4096']}")
        del xs, ys
    for fn, nm in (("qwha", "qwha_2048x4096_nnz262144"), ("harp", "harp_8192x4096_r16x3"),
                   ("harp_gen", "harp_8192x5120_r88852")):
        if fn in sel:
            res[nm] = bench_other(torch, W, mask_dev, synth, fn, nm, K, Wm)
            log(f"[bench] {nm}: {res[nm]}")
    if "qwha_bwd" in sel:
        res.update(bench_qwha_bwd(torch, W, synth, K, Wm))
        for nm in ("qwha_bwd_dx_2048x4096_nnz262144", "qwha_bwd_dc_2048x4096_nnz262144"):
            log(f"[bench] {nm}: {res[nm]}")
    if "int2" in sel:
        cfg5 = synth.rht_int2_g64()
        res.update(bench_quant(torch, W, mask_dev, cfg5, "rht_int2_g64_28672x8192", 2, 64, K, Wm))
        log(f"[bench] rht_int2_g64_28672x8192: {res['rht_int2_g64_28672x8192']}")
    if "gemv" in sel:
        nm = "gemv_int2_g64_28672x8192_t1"
        res[nm] = bench_gemv(torch, W, mask_dev, synth, nm, K, Wm)
        log(f"[bench] {nm}: {res[nm]}")
    if "qinit" in sel:
        res[QINIT] = bench_qinit(torch, W, mask_dev, synth, K, Wm)
        log(f"[bench] {QINIT}: {res[QINIT]}")

    main_r = res[MAIN]
    per_launch = main_r["ms_per_launch"] / 1e3
    traffic = traffic_for(MAIN, ALGO_BYTES[MAIN])
    line = {
        "metric": "rows/s and HBM GB/s (% of peak) for RHT+quant at d=4096/8192",
        "value": main_r["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": main_r["ms_per_launch"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "rht_int4_g128_4096x4096", "rows": 4096, "d": 4096, "bits": 4,
                   "group": 128, "input": "bf16 Student-t(3)*0.02, 0.1% outlier columns x20",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": main_r["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": main_r["GBps"] / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "k_rht_quant<12,bf16,4,7>", "algo_bytes_per_launch": ALGO_BYTES[MAIN],
                     "avg_launch_us": per_launch * 1e6},
        "workloads": res,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(cfg_main)
    print(json.dumps(line), flush=True)


def bench_qwha_bwd(torch, W, synth, K, Wm):
    """The adapter's backward at the QWHA workload: dx = (dy F) Hn (value
    permutation into F^T's order + the transposed gather and transform) and
    dc on F's support, timed separately."""
    d = synth.qwha_backward()
    rp = torch.from_numpy(d["row_ptr"]).to("cuda:0")
    ci = torch.from_numpy(d["col_idx"]).to("cuda:0")
    t_rp, t_ci, t_pm = W.qwha_csr_transpose(d["row_ptr"], d["col_idx"], 4096)
    t_rp, t_ci, t_pm = (torch.from_numpy(a).to("cuda:0") for a in (t_rp, t_ci, t_pm))
    v = d["vals"].to("cuda:0")
    t_v = torch.empty_like(v)
    dys = copies(torch, d["dy"].to("cuda:0"))
    xs = copies(torch, d["x"].to("cuda:0"))
    dxs = [torch.empty_like(x) for x in xs]
    dcs = [torch.empty(ci.numel(), dtype=torch.float32, device="cuda:0") for _ in xs]
    ws = torch.empty(W.qwha_grad_values_workspace_bytes(2048, 4096, ci.numel()), dtype=torch.uint8,
                     device="cuda:0")

    def dx_step(i):
        W.qwha_permute_values(v, t_pm, out=t_v)
        W.qwha_adapter_backward_input(dys[i % len(dys)], t_rp, t_ci, t_v, 4096, out=dxs[i % len(dxs)])

    def dc_step(i):
        W.qwha_adapter_grad_values(xs[i % len(xs)], dys[i % len(dys)], rp, ci, out=dcs[i % len(dcs)],
                                   workspace=ws)

    r = {}
    for nm, fn in (("qwha_bwd_dx_2048x4096_nnz262144", dx_step), ("qwha_bwd_dc_2048x4096_nnz262144", dc_step)):
        r[nm] = result(nm, Timed(torch, fn, K, Wm).run(), K)
    del dys, xs, dxs, dcs, ws
    torch.cuda.empty_cache()
    return r


def bench_gemv(torch, W, mask_dev, synth, name, K, Wm):
    """One decode token through the 28672 x 8192 INT2 g=64 layer: the
    online-RHT low-bit product, codes and scales rotating over >= 1 GiB of
    copies so that each launch reads them from HBM."""
    d = synth.gemv_int2_g64()
    c0 = torch.from_numpy(d["codes"]).to("cuda:0")
    s0 = torch.from_numpy(d["scales"]).to("cuda:0")
    x = d["x"].to("cuda:0")
    sg = mask_dev(d["signs"])
    k = max(2, math.ceil(GIB / (c0.numel() + 2 * s0.numel())))
    cs = [c0.clone() for _ in range(k)]
    ss = [s0.clone() for _ in range(k)]
    ys = [torch.empty((1, c0.shape[0]), dtype=torch.bfloat16, device="cuda:0") for _ in range(k)]
    del c0, s0
    t = Timed(torch, lambda i: W.rht_lowbit_gemv(x, cs[i % k], ss[i % k], sg, 2, 64, out=ys[i % k]), K, Wm)
    r = result(name, t.run(), K)
    r["tokens_per_s"] = 1e3 / r["ms_per_launch"]
    del cs, ss, ys
    torch.cuda.empty_cache()
    return r


QINIT = "qwha_init_4096x4096_int4_g128_t2048"


def bench_qinit(torch, W, mask_dev, synth, K, Wm):
    """QWHA initialisation of the 4096 x 4096 INT4 g=128 layer from 2048
    calibration tokens (budget 262,144, floor 16, cap 128): each device stage
    timed alone (a HIP graph of K calls, same buffers), the host allocation on
    the host clock, and the whole chain (device stages + the error copy to the
    host, the allocation and the row pointer copy back) on the host clock."""
    d = synth.qwha_init_int4_g128()
    rows, n = d["w"].shape
    T = d["x"].shape[0]
    total, floor, cap = d["total"], d["floor"], d["cap"]
    dv = "cuda:0"
    w, x, sg = d["w"].to(dv), d["x"].to(dv), mask_dev(d["signs"])
    codes, scales = W.rht_quantize_rtn(w, sg, 4, 128)
    f = torch.empty((rows, n), dtype=torch.float32, device=dv)
    z = torch.empty((T, n), dtype=torch.float32, device=dv)
    g = torch.empty((n, n), dtype=torch.float32, device=dv)
    p = torch.empty((rows, n), dtype=torch.float32, device=dv)
    err = torch.empty(rows, dtype=torch.float32, device=dv)
    col = torch.empty(total, dtype=torch.int32, device=dv)
    vals = torch.empty(total, dtype=torch.float32, device=dv)
    stage = {}
    stage["error_coeffs"] = Timed(torch, lambda i: W.qwha_init_error_coeffs(w, codes, scales, sg, 4, 128, out=f),
                                  K, Wm).run() / K
    stage["gram"] = Timed(torch, lambda i: W.qwha_init_gram(x, g=g, z=z), K, Wm).run() / K
    stage["channel_errors"] = Timed(torch, lambda i: W.qwha_init_channel_errors(f, g, p=p, err=err), K, Wm).run() / K
    reps = max(3, K // 4)
    t0 = time.perf_counter()
    for _ in range(reps):
        rp_host = W.qwha_init_allocate(err, n, total, floor, cap)
    stage["allocate_host"] = (time.perf_counter() - t0) / reps
    row_ptr = rp_host.to(dv)
    stage["select"] = Timed(torch, lambda i: W.qwha_init_select(f, row_ptr, col_idx=col), K, Wm).run() / K
    stage["refine"] = Timed(torch, lambda i: W.qwha_init_refine(g, p, row_ptr, col, vals=vals), K, Wm).run() / K
    for _ in range(Wm):
        W.qwha_initialize(w, codes, scales, sg, 4, 128, x, total, floor, cap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        W.qwha_initialize(w, codes, scales, sg, 4, 128, x, total, floor, cap)
    torch.cuda.synchronize()
    step = (time.perf_counter() - t0) / K
    gram_flop = n * (n + 1) * T        # unique entries of Z^T Z, 2 flops per product
    fg_flop = 2 * rows * n * n
    r = {"ms_per_step": step * 1e3, "layers_per_s": 1.0 / step,
         "stage_ms": {k: v * 1e3 for k, v in stage.items()},
         "gram_TFLOPs": gram_flop / stage["gram"] / 1e12,
         "channel_errors_TFLOPs": fg_flop / stage["channel_errors"] / 1e12,
         "frac_fp32_mfma_peak_channel_errors": fg_flop / stage["channel_errors"] / 157.3e12,
         "select_GBps": rows * n * 4 / stage["select"] / 1e9}
    del f, z, g, p, col, vals
    torch.cuda.empty_cache()
    return r


def bench_other(torch, W, mask_dev, synth, fn, name, K, Wm):
    if fn == "qwha":
        d = synth.qwha()
        x0 = d["x"].to("cuda:0")
        rp = torch.from_numpy(d["row_ptr"]).to("cuda:0")
        ci = torch.from_numpy(d["col_idx"]).to("cuda:0")
        v = d["vals"].to("cuda:0")
        xs = copies(torch, x0)
        ys = [torch.empty((x0.shape[0], d["d_out"]), dtype=torch.bfloat16, device="cuda:0") for _ in xs]
        t = Timed(torch, lambda i: W.qwha_adapter_forward(xs[i % len(xs)], rp, ci, v, d["d_out"],
                                                          out=ys[i % len(xs)]), K, Wm)
    elif fn == "harp_gen":
        d = synth.harp_general()
        x0 = d["x"].to("cuda:0")
        blocks = torch.from_numpy(np.concatenate([b.reshape(-1) for b in d["blocks"]])).to("cuda:0").half()
        xs = copies(torch, x0)
        ys = [torch.empty_like(x0) for _ in xs]
        t = Timed(torch, lambda i: W.harp_rotate(xs[i % len(xs)], blocks, d["radices"], None, False,
                                                 out=ys[i % len(xs)]), K, Wm)
    else:
        d = synth.harp()
        x0 = d["x"].to("cuda:0")
        # the blocks are parameters: handed over in fp16, the precision the stages multiply in
        blocks = torch.from_numpy(np.concatenate([b.reshape(-1) for b in d["blocks"]])).to("cuda:0").half()
        sg = mask_dev(d["signs"])
        xs = copies(torch, x0)
        ys = [torch.empty_like(x0) for _ in xs]
        t = Timed(torch, lambda i: W.harp_rotate(xs[i % len(xs)], blocks, d["radices"], sg, True,
                                                 out=ys[i % len(xs)]), K, Wm)
    r = result(name, t.run(), K)
    torch.cuda.empty_cache()
    return r


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the MI355X Walsh-Hadamard hot path on one GPU.

Main workload (the one `value` is quoted on): RHT + INT4 round-to-nearest
quantisation, bf16 weight matrix 4096 x 4096, group 128 along d_in, fp16
scales, signed int4 codes -- one `rht_quantize_rtn` launch per step.  The
other workloads (orthonormal FWHT 256 x 4096 fp32 and its row sweep, the
inverse of the INT4 path, QWHA adapter forward and backward, HARP rotation
with the radix-16 schedule, with the mixed-radix 8*8*8*5*2 schedule at
d = 5120 and with 16*8*8 at d = 1024 (the matrix-core path of the general
schedules), 28672 x 8192 RHT + INT2 and its inverse, the online-RHT INT2
product, the QWHA initialisation) are timed the same way and reported under
"workloads".

Timing: every launch processes a different copy of the input, rotating over
copies totalling >= 1 GiB, and at least one launch per copy is timed, so the
inputs come from HBM rather than the 256 MB last-level cache.  The launches
are captured once in a HIP graph and replayed between two HIP events on the
launch stream, REPS times; each replay gives one per-launch time, and the
line reports their median, p10, p90 and min (`value` uses the median).  For
the bandwidth-bound workloads a plain 16-byte streaming kernel moving the
same bytes (whtq_stream_probe) is timed the same way: "% achievable".

Data are synthetic (seeded generators in wht_adapters_amd.synth, whose
docstrings give each recipe) with the shapes and value structure of the
workloads.  `python bench.py --summarize-pmc DIR...` turns rocprofv3 counter
CSVs into profiles/counters.json (read back here, per kernel source hash).
"""
import argparse
import csv
import glob
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
PEAK_F16_MFMA_TFLOPS = 2500.0     # dense fp16/bf16 matrix peak
VALU_LANE_OPS = 256 * 64 * 2.4e9  # non-packed fp32 lane-ops/s: 256 CUs x 4 SIMD16 x 2.4 GHz
GIB = 1 << 30
REPS = 9

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
    "harp_8192x1024_r1688": 2 * 8192 * 1024 * 2 + 1024 * (16 + 8 + 8) * 2,  # fp16 blocks
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
    "harp_8192x5120_r88852": 8192, "harp_8192x1024_r1688": 8192,
    "rht_int2_g64_28672x8192_inverse": 28672,
    "gemv_int2_g64_28672x8192_t1": 28672,
}
# k_harp: per 16-token tile, six radix-16 passes of 256 16x16x16 products plus
# the chained learned stage along digit 0 (256 more): 7 x 256 MFMAs of 8192 flop
HARP_MFMA_FLOP = 8192 // 16 * 7 * 256 * 2 * 16 * 16 * 16
MAIN = "rht_int4_g128_4096x4096"
KERNELS = {  # kernel (as rocprofv3 names it) and the sources it is built from, per workload
    MAIN: ("k_rht_quant_mx<12, 1, 4, 7>",
           ["rht_quant_mx.hpp", "rht_quant.hpp", "rq_fwd_b4.hip", "engine.hpp", "io.hpp", "common.hpp",
            "launch.hpp"]),
    "rht_int2_g64_28672x8192": ("k_rht_quant_mx<13, 1, 2, 6>",
                                ["rht_quant_mx.hpp", "rht_quant.hpp", "rq_fwd_b2.hip", "engine.hpp", "io.hpp",
                                 "common.hpp", "launch.hpp"]),
    "rht_int4_g128_4096x4096_inverse": ("k_rht_dequant<12, 4, 7, 1>",
                                        ["rht_quant.hpp", "rq_inv_b4.hip", "engine.hpp", "io.hpp", "common.hpp",
                                         "launch.hpp"]),
    "rht_int2_g64_28672x8192_inverse": ("k_rht_dequant<13, 2, 6, 1>",
                                        ["rht_quant.hpp", "rq_inv_b2.hip", "engine.hpp", "io.hpp", "common.hpp",
                                         "launch.hpp"]),
    "harp_8192x4096_r16x3": ("k_harp<true>", ["harp.hip", "common.hpp", "launch.hpp"]),
    "qwha_2048x4096_nnz262144": ("k_qwha_fwd<1, false>", ["qwha_fwd.hip", "io.hpp", "engine.hpp", "common.hpp"]),
    "harp_8192x1024_r1688": ("k_harp_mx<2, 16>", ["harp_gen.hip", "io.hpp", "common.hpp", "launch.hpp"]),
}
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "wht_adapters_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counters_for(name):
    """Per-launch rocprofv3 counters committed under profiles/counters.json,
    if they were taken on the current kernel sources; else None."""
    if name not in KERNELS or not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as fh:
        c = json.load(fh).get(name)
    if not c or c.get("src_sha") != src_hash(KERNELS[name][1]):
        return None
    return c


class Timed:
    """n launches of `launch(i)` captured in one HIP graph, replayed between
    two HIP events on the capture stream."""

    def __init__(self, torch, launch, n, warmup):
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
            for i in range(n):
                launch(i)
        torch.cuda.synchronize()
        self.n = n

    def run(self, reps=REPS):
        """Per-launch seconds, one value per replay."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            self.graph.replay()            # untimed replay: pages in the graph
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
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
            out.append(e0.elapsed_time(e1) / 1e3 / self.n)
        return out


def n_launch(K, ncopies):
    """Launches per graph: K, and at least one per copy of the input."""
    return max(K, ncopies)


def copies(torch, t, total_bytes=GIB, cap=256):
    k = max(2, min(cap, math.ceil(total_bytes / max(1, t.numel() * t.element_size()))))
    return [t.clone() for _ in range(k)]


def stats(per):
    a = np.sort(np.asarray(per, dtype=np.float64))
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "min": float(a[0]), "reps": int(a.size)}


def result(name, per, rows=None, algo=None):
    st = stats(per)
    med = st["median"]
    algo = ALGO_BYTES[name] if algo is None else algo
    rows = ROWS[name] if rows is None else rows
    gbs = algo / med / 1e9
    return {"ms_per_launch": med * 1e3, "us_p10": st["p10"] * 1e6, "us_p90": st["p90"] * 1e6,
            "us_min": st["min"] * 1e6, "reps": st["reps"], "rows_per_s": rows / med, "GBps": gbs,
            "frac_hbm_peak": gbs / PEAK_HBM_GBS, "algo_bytes": algo}


def achievable(torch, W, r, in_bytes, out_bytes, K, Wm):
    """Time whtq_stream_probe moving the same bytes (rotated the same way) and
    add it to the result r as the achievable reference."""
    ib, ob = in_bytes // 16 * 16, out_bytes // 16 * 16
    k = max(2, math.ceil(GIB / max(1, ib)))
    srcs = [torch.empty(ib, dtype=torch.uint8, device="cuda:0") for _ in range(k)]
    dsts = [torch.empty(max(ob, 16), dtype=torch.uint8, device="cuda:0")[:ob] for _ in range(k)]
    for s in srcs:
        s.fill_(1)
    t = Timed(torch, lambda i: W.stream_probe(srcs[i % k], dsts[i % k]), n_launch(K, k), Wm)
    med = stats(t.run())["median"]
    r["stream_probe_us"] = med * 1e6
    r["stream_probe_frac_hbm_peak"] = (ib + ob) / med / 1e9 / PEAK_HBM_GBS
    r["frac_achievable"] = med / (r["ms_per_launch"] / 1e3)
    del srcs, dsts
    torch.cuda.empty_cache()


def bench_quant(torch, W, mask_dev, cfg, name, bits, g, K, Wm):
    w0 = cfg["w"].to("cuda:0")
    rows, n = w0.shape
    ws = copies(torch, w0)
    sg = mask_dev(cfg["signs"])
    cs = [torch.empty((rows, n * bits // 8), dtype=torch.uint8, device="cuda:0") for _ in ws]
    ss = [torch.empty((rows, n // g), dtype=torch.float16, device="cuda:0") for _ in ws]
    del w0
    nl = n_launch(K, len(ws))
    fwd = Timed(torch, lambda i: W.rht_quantize_rtn(ws[i % len(ws)], sg, bits, g, cs[i % len(ws)],
                                                    ss[i % len(ws)]), nl, Wm)
    outs = [torch.empty((rows, n), dtype=torch.bfloat16, device="cuda:0") for _ in ws]
    inv = Timed(torch, lambda i: W.rht_dequantize_inverse(cs[i % len(ws)], ss[i % len(ws)], sg, bits, g, n,
                                                          out=outs[i % len(ws)]), nl, Wm)
    r = {name: result(name, fwd.run())}
    r[name + "_inverse"] = result(name + "_inverse", inv.run())
    W.rht_quantize_rtn(ws[0], sg, bits, g, cs[0], ss[0])
    torch.cuda.synchronize()
    first = (cs[0].cpu().numpy(), ss[0].cpu().numpy())   # kept for the parity report
    del ws, cs, ss, outs
    torch.cuda.empty_cache()
    code_b = rows * n * bits // 8 + rows * (n // g) * 2
    achievable(torch, W, r[name], rows * n * 2, code_b, K, Wm)
    achievable(torch, W, r[name + "_inverse"], code_b, rows * n * 2, K, Wm)
    return r, first


def bench_fwht(torch, W, synth, K, Wm):
    """The 256 x 4096 fp32 FWHT, then a labelled row sweep (256 .. 65,536 rows)
    that shows where the launch stops being latency-bound."""
    nm = "fwht_f32_256x4096"
    x = torch.from_numpy(synth.fwht_f32()["x"]).to("cuda:0")
    xs = copies(torch, x)
    ys = [torch.empty_like(x) for _ in xs]
    t = Timed(torch, lambda i: W.wht_batched(xs[i % len(xs)], out=ys[i % len(xs)]), n_launch(K, len(xs)), Wm)
    r = {nm: result(nm, t.run())}
    del xs, ys
    achievable(torch, W, r[nm], 256 * 4096 * 4, 256 * 4096 * 4, K, Wm)
    sweep = {}
    for rows in (256, 1024, 4096, 16384, 65536):
        x = torch.randn((rows, 4096), device="cuda:0")
        xs = copies(torch, x)
        ys = [torch.empty_like(x) for _ in xs]
        t = Timed(torch, lambda i: W.wht_batched(xs[i % len(xs)], out=ys[i % len(xs)]), n_launch(K, len(xs)), Wm)
        s = result(nm, t.run(), rows=rows, algo=2 * rows * 4096 * 4)
        sweep[str(rows)] = {k: s[k] for k in ("ms_per_launch", "us_p10", "us_p90", "rows_per_s", "GBps",
                                              "frac_hbm_peak")}
        del x, xs, ys
        torch.cuda.empty_cache()
    r["fwht_f32_rows_x4096_sweep"] = sweep
    return r


def cpu_baselines(first_main, budget_s=4.0):
    """The oracle as it stands, timed on this host: all 4096 rows of the main
    workload (also compared with the GPU's codes for the parity report), and
    bounded samples of the other workloads."""
    from threadpoolctl import threadpool_info
    from oracle import compare, hadamard as H, harp, qwha, rtn
    from wht_adapters_amd import synth
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    host = len(os.sched_getaffinity(0))
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        res = fn()
        return res, time.perf_counter() - t0

    # main workload, whole matrix
    cfg = synth.rht_int4_g128()
    w = synth.bf16_to_f64(cfg["w"])
    s = H.signs_from_bits(cfg["signs"], 4096)
    (codes, s16, q, v, s_pre, y), secs = timed(lambda: rtn.rht_quantize(w, s, 4, 128))
    main = {"value": 4096 / secs, "unit": "rows/s", "cores": int(threads), "host_cores": host,
            "kind": "oracle",
            "sample": f"all 4096 rows of the 4096x4096 INT4 g128 workload (dense fp64 Sylvester product + "
                      f"naive RTN), {secs:.2f} s"}
    q_dev = rtn.unpack_codes(first_main[0], 4, 4096)
    rep = compare.compare_quant(q_dev, first_main[1].astype(np.float16), y, s16, q, v, s_pre, 4, 128)
    parity = dict(rep, config=MAIN, rows=4096)
    del w, y, v, q

    def sample(name, unit, rows_total, fn, rows_done, what):
        _, secs = timed(fn)
        out[name] = {"value": rows_done / secs, "unit": unit, "cores": int(threads), "host_cores": host,
                     "kind": "oracle", "sample": f"{rows_done} of {rows_total} {what}, {secs:.2f} s"}

    x1 = synth.fwht_f32()["x"].astype(np.float64)
    sample("fwht_f32_256x4096", "rows/s", 256, lambda: H.wht(x1), 256, "rows (dense Sylvester product)")
    c5 = synth.rht_int2_g64(rows=512)
    w5 = synth.bf16_to_f64(c5["w"])
    sample("rht_int2_g64_28672x8192", "rows/s", 28672,
           lambda: rtn.rht_quantize(w5, H.signs_from_bits(c5["signs"], 8192), 2, 64), 512,
           "rows (512 rows drawn by the same recipe; dense fp64 Sylvester product + naive RTN)")
    d3 = synth.qwha(tokens=256)
    sample("qwha_2048x4096_nnz262144", "tokens/s", 2048,
           lambda: qwha.qwha_forward(synth.bf16_to_f64(d3["x"]), d3["row_ptr"], d3["col_idx"],
                                     synth.bf16_to_f64(d3["vals"]), d3["d_out"]), 256,
           "tokens (dense F, dense Sylvester product)")
    d4 = synth.harp(tokens=128)
    sample("harp_8192x4096_r16x3", "tokens/s", 8192,
           lambda: harp.harp_rotate(synth.bf16_to_f64(d4["x"]), d4["radices"], d4["blocks"],
                                    s=H.signs_from_bits(d4["signs"], 4096)), 128,
           "tokens (dense stage matrices built and applied)")
    return main, out, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads", default="all",
                    help="all | main | comma list of fwht, qwha, qwha_bwd, harp, harp_gen, harp_mx, int2, gemv, qinit "
                         "(the main workload always runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (PMC calibration)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="write profiles/counters.json from rocprofv3 counter CSVs under DIRs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
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
    log(f"[bench] device {torch.cuda.get_device_name(0)}, steps {K}, warmup {Wm}, reps {REPS}")

    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("[bench] copy probe: 3 x 256 MiB device copy done")

    sel = {"all": {"main", "fwht", "qwha", "qwha_bwd", "harp", "harp_gen", "harp_mx", "int2", "gemv", "qinit"},
           "main": {"main"}}.get(
        args.workloads, set(args.workloads.split(",")))
    sel.add("main")  # `value` is always quoted on the main workload
    cfg_main = synth.rht_int4_g128()
    res, first_main = bench_quant(torch, W, mask_dev, cfg_main, MAIN, 4, 128, K, Wm)
    log(f"[bench] {MAIN}: {res[MAIN]}")
    if "fwht" in sel:
        res.update(bench_fwht(torch, W, synth, K, Wm))
        log(f"[bench] fwht_f32_256x4096: {res['fwht_f32_256x4096']}")
    for fn, nm in (("qwha", "qwha_2048x4096_nnz262144"), ("harp", "harp_8192x4096_r16x3"),
                   ("harp_gen", "harp_8192x5120_r88852"), ("harp_mx", "harp_8192x1024_r1688")):
        if fn in sel:
            res[nm] = bench_other(torch, W, mask_dev, synth, fn, nm, K, Wm)
            log(f"[bench] {nm}: {res[nm]}")
    if "qwha_bwd" in sel:
        res.update(bench_qwha_bwd(torch, W, synth, K, Wm))
        for nm in ("qwha_bwd_dx_2048x4096_nnz262144", "qwha_bwd_dc_2048x4096_nnz262144"):
            log(f"[bench] {nm}: {res[nm]}")
    if "int2" in sel:
        cfg5 = synth.rht_int2_g64()
        r5, _ = bench_quant(torch, W, mask_dev, cfg5, "rht_int2_g64_28672x8192", 2, 64, K, Wm)
        res.update(r5)
        del cfg5
        log(f"[bench] rht_int2_g64_28672x8192: {res['rht_int2_g64_28672x8192']}")
    if "gemv" in sel:
        nm = "gemv_int2_g64_28672x8192_t1"
        res[nm] = bench_gemv(torch, W, mask_dev, synth, nm, K, Wm)
        log(f"[bench] {nm}: {res[nm]}")
    if "qinit" in sel:
        res[QINIT] = bench_qinit(torch, W, mask_dev, synth, K, Wm)
        log(f"[bench] {QINIT}: {res[QINIT]}")

    # what the committed rocprofv3 counters say about each kernel (per launch)
    for nm in KERNELS:
        c = counters_for(nm)
        if nm in res and c:
            res[nm]["counters"] = {k: c[k] for k in ("hbm_bytes", "traffic_ratio", "valu_insts", "valu_busy_pct",
                                                     "mfma_busy_pct", "from") if k in c}
    if "harp_8192x4096_r16x3" in res:
        hr = res["harp_8192x4096_r16x3"]
        hr["mfma_TFLOPs"] = HARP_MFMA_FLOP / (hr["ms_per_launch"] / 1e3) / 1e12
        hr["frac_f16_mfma_peak"] = hr["mfma_TFLOPs"] / PEAK_F16_MFMA_TFLOPS

    main_r = res[MAIN]
    per_launch = main_r["ms_per_launch"] / 1e3
    cm = counters_for(MAIN)
    valu = None
    if cm and "valu_insts" in cm:
        valu = {"valu_insts_per_launch": cm["valu_insts"],
                "valu_floor_us": cm["valu_insts"] * 64 / VALU_LANE_OPS * 1e6,
                "frac_of_valu_floor": cm["valu_insts"] * 64 / VALU_LANE_OPS / per_launch}
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
                     "frac": main_r["GBps"] / PEAK_HBM_GBS,
                     "traffic": cm["hbm_bytes"] if cm and "hbm_bytes" in cm else None,
                     "kernel": KERNELS[MAIN][0], "algo_bytes_per_launch": ALGO_BYTES[MAIN],
                     "avg_launch_us": per_launch * 1e6,
                     "achievable_us": main_r["stream_probe_us"], "frac_achievable": main_r["frac_achievable"],
                     "valu": valu},
        "timing": {"launches_per_replay": n_launch(K, 32), "replays": REPS,
                   "statistic": "median over replays of the per-launch time (p10/p90/min beside it)",
                   "inputs": "rotate over copies totalling >= 1 GiB, each copy at least once per replay"},
        "workloads": res,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        line["cpu_baseline"], line["cpu_baseline_other"], line["parity"] = cpu_baselines(first_main)
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
        r[nm] = result(nm, Timed(torch, fn, n_launch(K, len(xs)), Wm).run())
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
    t = Timed(torch, lambda i: W.rht_lowbit_gemv(x, cs[i % k], ss[i % k], sg, 2, 64, out=ys[i % k]),
              n_launch(K, k), Wm)
    r = result(name, t.run())
    r["tokens_per_s"] = 1e3 / r["ms_per_launch"]
    del cs, ss, ys
    torch.cuda.empty_cache()
    achievable(torch, W, r, ALGO_BYTES[name] - 28672 * 2, 28672 * 2, K, Wm)
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
    med = lambda t: stats(t.run(3))["median"]
    stage["error_coeffs"] = med(Timed(torch, lambda i: W.qwha_init_error_coeffs(w, codes, scales, sg, 4, 128, out=f),
                                      K, Wm))
    stage["gram"] = med(Timed(torch, lambda i: W.qwha_init_gram(x, g=g, z=z), K, Wm))
    stage["channel_errors"] = med(Timed(torch, lambda i: W.qwha_init_channel_errors(f, g, p=p, err=err), K, Wm))
    reps = max(3, K // 4)
    t0 = time.perf_counter()
    for _ in range(reps):
        rp_host = W.qwha_init_allocate(err, n, total, floor, cap)
    stage["allocate_host"] = (time.perf_counter() - t0) / reps
    row_ptr = rp_host.to(dv)
    stage["select"] = med(Timed(torch, lambda i: W.qwha_init_select(f, row_ptr, col_idx=col), K, Wm))
    stage["refine"] = med(Timed(torch, lambda i: W.qwha_init_refine(g, p, row_ptr, col, vals=vals), K, Wm))
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
        # the support is fixed during training: its forward plan is built once, outside the timed region
        # (its own time and the unplanned forward's are reported beside)
        toks, nnz = x0.shape[0], ci.numel()
        plan = W.qwha_forward_plan(toks, 4096, rp, d["d_out"], nnz)
        t = Timed(torch, lambda i: W.qwha_adapter_forward(xs[i % len(xs)], rp, ci, v, d["d_out"],
                                                          out=ys[i % len(xs)], plan=plan), n_launch(K, len(xs)), Wm)
        t_np = Timed(torch, lambda i: W.qwha_adapter_forward(xs[i % len(xs)], rp, ci, v, d["d_out"],
                                                             out=ys[i % len(xs)]), n_launch(K, len(xs)), Wm)
        plans = [torch.empty_like(plan) for _ in range(4)]
        t_pl = Timed(torch, lambda i: W.qwha_forward_plan(toks, 4096, rp, d["d_out"], nnz, out=plans[i % 4]), K, Wm)
    elif fn in ("harp_gen", "harp_mx"):
        d = synth.harp_general() if fn == "harp_gen" else synth.harp_general(radices=(16, 8, 8))
        x0 = d["x"].to("cuda:0")
        blocks = torch.from_numpy(np.concatenate([b.reshape(-1) for b in d["blocks"]])).to("cuda:0").half()
        xs = copies(torch, x0)
        ys = [torch.empty_like(x0) for _ in xs]
        t = Timed(torch, lambda i: W.harp_rotate(xs[i % len(xs)], blocks, d["radices"], None, False,
                                                 out=ys[i % len(xs)]), n_launch(K, len(xs)), Wm)
    else:
        d = synth.harp()
        x0 = d["x"].to("cuda:0")
        # the blocks are parameters: handed over in fp16, the precision the stages multiply in
        blocks = torch.from_numpy(np.concatenate([b.reshape(-1) for b in d["blocks"]])).to("cuda:0").half()
        sg = mask_dev(d["signs"])
        xs = copies(torch, x0)
        ys = [torch.empty_like(x0) for _ in xs]
        t = Timed(torch, lambda i: W.harp_rotate(xs[i % len(xs)], blocks, d["radices"], sg, True,
                                                 out=ys[i % len(xs)]), n_launch(K, len(xs)), Wm)
    r = result(name, t.run())
    if fn == "qwha":
        r["unplanned_us"] = result(name, t_np.run())["ms_per_launch"] * 1e3
        r["plan_build_us"] = result(name, t_pl.run())["ms_per_launch"] * 1e3
        r["plan_bytes"] = plan.numel()
        del plans, plan
    nb = x0.numel() * x0.element_size()
    del xs, ys
    torch.cuda.empty_cache()
    if fn != "qwha":
        achievable(torch, W, r, nb, nb, K, Wm)
    return r


# ---------------------------------------------------------------- counters

def summarize_pmc(dirs):
    """profiles/counters.json from rocprofv3 --pmc CSVs (one counter set per
    run) of the bench command: per kernel of KERNELS, the per-dispatch average
    of each counter.  HBM bytes = 2 x FETCH_SIZE + WRITE_SIZE (KiB), the
    factors a plain 256 MiB device copy gives these counters on MI355X
    (FETCH_SIZE reads 131,087 KiB for 262,144 KiB moved, WRITE_SIZE
    262,144 KiB)."""
    per = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], {}).setdefault(
                        r["Dispatch_Id"], 0.0)
                    per[r["Kernel_Name"]][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    out = json.load(open(COUNTERS)) if os.path.exists(COUNTERS) else {}
    for nm, (kern, srcs) in KERNELS.items():
        hits = [k for k in per if kern in k]
        if not hits:
            continue
        c = per[hits[0]]
        avg = {cn: sum(v.values()) / len(v) for cn, v in c.items()}
        e = {"src_sha": src_hash(srcs), "kernel": kern, "from": "profiles/ (rocprofv3 --pmc, bench.py command)"}
        if "FETCH_SIZE" in avg and "WRITE_SIZE" in avg:
            e["hbm_bytes"] = int((2.0 * avg["FETCH_SIZE"] + avg["WRITE_SIZE"]) * 1024)
            e["traffic_ratio"] = e["hbm_bytes"] / ALGO_BYTES[nm]
        if "SQ_INSTS_VALU" in avg:
            e["valu_insts"] = avg["SQ_INSTS_VALU"]
        if "VALUBusy" in avg:
            e["valu_busy_pct"] = avg["VALUBusy"]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
            # MFMA busy cycles summed over the 1024 SIMDs; GRBM_GUI_ACTIVE summed over the 8 XCDs
            e["mfma_busy_pct"] = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (avg["GRBM_GUI_ACTIVE"] / 8)
        e["counters"] = avg
        out[nm] = e
    with open(COUNTERS, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    print(f"wrote {COUNTERS}: {sorted(out)}")


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the GQA / GQE hot path on one MI355X.

One step runs the whole path once on resident synthetic inputs:
  * GQA causal prefill, bf16 in / fp32 accumulate: B=4, h=32, g=8, T=2048,
    d=128 (the headline workload: ``value`` is its TFLOP/s);
  * GQA decode over a bf16 KV cache: B=64, h=32, g=8, d=128, cache lengths
    uniform in [1024, 8192] (KV GB/s);
  * GQE routed causal prefill, bf16: B=2, T=4096, h=32, g=8, d=128, top-k 1
    and 2 (TFLOP/s of the kept rows).
Every kernel call is bracketed by HIP events recorded on the stream the
library launches on (torch's current stream). Before every timed call a
1 GiB buffer is read (outside the events) so the 256 MB Infinity Cache and
the L2s hold none of the call's inputs; a read is used rather than a write so
that no dirty lines are written back during the timed call. Work is counted
algorithmically: causal prefill flops are 4*d per visible (query, key) pair,
GQE flops only for kept rows, decode bytes only for cached positions below
lens[b] (plus q and out).

After the timed steps, the KV-group sweep (decode, B=32, T=16384, g in
{1, 4, 8, 32}) is timed the same way, with the HBM bytes the counters measured
per g (profiles/traffic_counters.json) beside the cache-size law and, as the
size-matched ceiling, the HBM read microbenchmark streaming the same cache
bytes (one launch, flushed, same events), and the
float64 CPU oracle is timed on the whole prefill workload (cpu_baseline); its
output is compared with the GPU's, element by element.

Prints ONE JSON line. Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA prefill TFLOP/s + decode KV GB/s (fraction of MI355X peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = {
    "prefill": "gqa_routed_query_amd/csrc/attn_bf16.hip",
    "decode": "gqa_routed_query_amd/csrc/decode.hip",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the peak microbenchmarks (HBM read stream, MFMA-only loop)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the sweeps outside the step (KV-group decode, GQE vs GQA over T)")
    ap.add_argument("--only", choices=["prefill", "decode", "gqe", "sweep", "copy", "peaks"], default=None,
                    help="profile helper: run only one kernel family (sweep = the KV-group decode "
                         "sweep, two calls per g; copy = calibration copy; peaks = the peak "
                         "microbenchmarks)")
    return ap.parse_args()


def source_hash(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(name, field="bytes_per_launch"):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[name]
    except (OSError, KeyError, ValueError):
        return None
    src = rec.get("source", KERNEL_SOURCES.get(name))
    if not src or rec.get("source_sha256_16") != source_hash(src):
        return None
    return rec.get(field)


class Timer:
    """Per-call HIP event pairs on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.s = self.torch.cuda.Event(enable_timing=True)
        self.e = self.torch.cuda.Event(enable_timing=True)
        self.s.record()
        return self

    def __exit__(self, *exc):
        self.e.record()
        self.pairs.append((self.s, self.e))

    def ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gqa_routed_query_amd as gq
    from workloads import (ROUTER_D_MODEL, WORKLOADS, decode_inputs, gqe_inputs, gqe_sweep_points,
                           prefill_inputs, router_inputs, router_logits)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"device {torch.cuda.get_device_name(dev)}, lib {gq.lib_path}")

    wp, wd, wg = WORKLOADS["prefill"], WORKLOADS["decode"], WORKLOADS["gqe"]
    # Cache eviction before every timed call: READ 1 GiB (a write would leave
    # dirty lines whose write-back competes with the timed kernel).
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    if args.only == "copy":
        # calibration for the HBM byte counters: one 1 GiB device copy
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 1 GiB")
        return
    if args.only == "peaks":
        # the peak microbenchmarks alone, e.g. for counters on the attention tile loop
        # (no rocm-smi query: under a profiler, child processes cannot start)
        measured_peaks(torch, gq, dev, smi=False)
        return

    run_prefill = args.only in (None, "prefill")
    run_decode = args.only in (None, "decode")
    run_gqe = args.only in (None, "gqe")
    run_sweep = args.only == "sweep" or (args.only is None and not args.no_sweep)

    # ---- inputs, resident in HBM before any timing ----
    if run_prefill:
        pq, pk, pv = prefill_inputs(wp.B, wp.h, wp.g, wp.T, wp.d, "bf16", seed=wp.seed, device=dev)
        pout = torch.empty_like(pq)
        prefill_flops = 2.0 * wp.B * wp.h * wp.d * wp.T * (wp.T + 1)
    if run_decode:
        dq, dk, dv, dlens = decode_inputs(wd.B, wd.h, wd.g, wd.T, wd.d, wd.lens, seed=wd.seed,
                                          device=dev)
        dout = torch.empty_like(dq)
        dws_bytes = gq.gqa_decode_workspace_bytes(wd.B, wd.h, wd.g, wd.T, wd.d)
        dws = torch.empty(max(dws_bytes, 1), dtype=torch.uint8, device=dev)
        sum_lens = int(dlens.sum().item())
        decode_bytes = (2 * wd.g * wd.d * 2) * sum_lens + 2 * dq.numel() * 2
    if run_gqe:
        gq_, gk, gv, glg = gqe_inputs(wg.B, wg.h, wg.g, wg.T, wg.d, "bf16", seed=wg.seed, device=dev)
        gout = torch.empty_like(gq_)
        gws = {}
        for kk in wg.top_k:
            nb = gq.gqe_workspace_bytes(wg.B, wg.h, wg.g, wg.T, wg.d, kk)
            gws[kk] = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        dense_gqe_flops = 2.0 * wg.B * wg.h * wg.d * wg.T * (wg.T + 1)
    torch.cuda.synchronize()

    t_pre, t_dec = Timer(torch), Timer(torch)
    t_gqe = {k: Timer(torch) for k in wg.top_k}
    t_gqa_same = Timer(torch)  # dense GQA at the GQE shape, for the speedup ratio

    def step(timed):
        # every call starts with no input in the Infinity Cache or the L2s
        if run_prefill:
            flush.sum()
            with (t_pre if timed else Timer(torch)):
                gq.gqa_prefill(pq, pk, pv, causal=True, out=pout)
        if run_decode:
            flush.sum()
            with (t_dec if timed else Timer(torch)):
                gq.gqa_decode(dq, dk, dv, dlens, out=dout, workspace=dws)
        if run_gqe:
            for kk in wg.top_k:
                flush.sum()
                with (t_gqe[kk] if timed else Timer(torch)):
                    gq.gqe_routed_prefill(gq_, gk, gv, glg, kk, causal=True, out=gout,
                                          workspace=gws[kk])
            flush.sum()
            with (t_gqa_same if timed else Timer(torch)):
                gq.gqa_prefill(gq_, gk, gv, causal=True, out=gout)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / max(args.steps, 1)

    def stats(ms):
        ms = sorted(ms)
        return {"mean_ms": sum(ms) / len(ms), "median_ms": ms[len(ms) // 2], "min_ms": ms[0]}

    res = {}
    if run_prefill:
        sp = stats(t_pre.ms())
        tflops = prefill_flops / (sp["mean_ms"] * 1e-3) / 1e12
        res["prefill"] = dict(sp, tflops=tflops, frac_peak=tflops / PEAK_BF16_TFLOPS,
                              flops_per_launch=prefill_flops)
        log(f"prefill: {sp['mean_ms']*1e3:.1f} us/launch, {tflops:.1f} TFLOP/s")
    if run_decode:
        sd = stats(t_dec.ms())
        gbps = decode_bytes / (sd["mean_ms"] * 1e-3) / 1e9
        res["decode"] = dict(sd, GBps=gbps, frac_peak=gbps / PEAK_HBM_GBPS,
                             bytes_per_call=decode_bytes, sum_lens=sum_lens,
                             kv_cache_bytes=gq.gqa_kv_cache_bytes(1, wd.g, sum_lens, wd.d))
        log(f"decode: {sd['mean_ms']*1e3:.1f} us/call, {gbps:.0f} GB/s")
    if run_gqe:
        res["gqe"] = {}
        dense_same = stats(t_gqa_same.ms())
        for kk in wg.top_k:
            sg = stats(t_gqe[kk].ms())
            fl = dense_gqe_flops * kk / (wg.h // wg.g)
            tf = fl / (sg["mean_ms"] * 1e-3) / 1e12
            res["gqe"][f"top{kk}"] = dict(sg, tflops=tf, frac_peak=tf / PEAK_BF16_TFLOPS,
                                          flops_per_call=fl,
                                          speedup_vs_dense=dense_same["mean_ms"] / sg["mean_ms"])
            log(f"gqe k={kk}: {sg['mean_ms']*1e3:.1f} us/call, {tf:.1f} TFLOP/s")

    # ---- GQE routed decode at the decode workload, outside the step ----
    gdec = {}
    if run_decode and run_sweep:
        dlg = router_logits(wd.B, 1, wd.h, seed=wd.seed + 100, device=dev)[:, 0].contiguous()
        for kk in (1, 2):
            tm = Timer(torch)
            for it in range(3 + args.steps):
                flush.sum()
                if it < 3:
                    gq.gqe_routed_decode(dq, dk, dv, dlens, dlg, kk, out=dout, workspace=dws)
                    continue
                with tm:
                    gq.gqe_routed_decode(dq, dk, dv, dlens, dlg, kk, out=dout, workspace=dws)
            torch.cuda.synchronize()
            sg = stats(tm.ms())
            # the K/V stream is the same as plain decode; only the kept heads'
            # queries are read; every output row is written; logits, idx, gates
            nb = (2 * wd.g * wd.d * 2) * sum_lens + wd.B * wd.g * kk * wd.d * 2 + dq.numel() * 2 \
                + dlg.numel() * 4 + 2 * wd.B * wd.g * kk * 4
            gdec[f"top{kk}"] = dict(mean_us=sg["mean_ms"] * 1e3, GBps=nb / (sg["mean_ms"] * 1e-3) / 1e9,
                                    frac=nb / (sg["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                    time_vs_dense_decode=sg["mean_ms"] / res["decode"]["mean_ms"])
            log(f"gqe decode k={kk}: {sg['mean_ms']*1e3:.1f} us/call, {gdec[f'top{kk}']['GBps']:.0f} GB/s")
        del dlg

    # ---- KV-group sweep (decode), outside the step ----
    sweep = []
    if (run_decode or args.only == "sweep") and run_sweep:
        if run_decode:
            del dk, dv
        ws = WORKLOADS["decode_sweep"]
        # profile runs (--only sweep) make two calls per g, in the order of g_sweep
        n_warm, n_time = (1, 1) if args.only == "sweep" else (3, 10)
        kv_mha = gq.gqa_kv_cache_bytes(ws.B, ws.h, ws.T, ws.d)
        for g in ws.g_sweep:
            q, kc0, vc0, lens = decode_inputs(ws.B, ws.h, g, ws.T, ws.d, ws.lens, seed=ws.seed + g,
                                              device=dev)
            # K and V as two halves of one buffer, so that the HBM read
            # microbenchmark can stream exactly the cache bytes in one launch
            kv_buf = torch.empty((2,) + tuple(kc0.shape), dtype=kc0.dtype, device=dev)
            kv_buf[0].copy_(kc0)
            kv_buf[1].copy_(vc0)
            del kc0, vc0
            kc, vc = kv_buf[0], kv_buf[1]
            out = torch.empty_like(q)
            wsb = torch.empty(max(gq.gqa_decode_workspace_bytes(ws.B, ws.h, g, ws.T, ws.d), 1),
                              dtype=torch.uint8, device=dev)
            tm = Timer(torch)
            for it in range(n_warm + n_time):
                flush.sum()
                if it < n_warm:
                    gq.gqa_decode(q, kc, vc, lens, out=out, workspace=wsb)
                    continue
                with tm:
                    gq.gqa_decode(q, kc, vc, lens, out=out, workspace=wsb)
            torch.cuda.synchronize()
            st = stats(tm.ms())
            # the same cache bytes as one plain sequential read (flushed, same
            # timing): what any kernel that must read them can reach at this size
            tr = Timer(torch)
            xr = torch.zeros(1, dtype=torch.int32, device=dev)
            for it in range(n_warm + n_time):
                flush.sum()
                if it < n_warm:
                    gq.peak_hbm_read(kv_buf, xr)
                    continue
                with tr:
                    gq.peak_hbm_read(kv_buf, xr)
            torch.cuda.synchronize()
            rd = stats(tr.ms())
            # the cache-size law 2 * n_kv * d * T * sizeof(bf16) * B, and the HBM
            # bytes the counters measured for one call (null when they were
            # taken on another kernel source)
            kv = gq.gqa_kv_cache_bytes(ws.B, g, ws.T, ws.d)
            nbytes = kv + 2 * q.numel() * 2
            measured = traffic_for(f"decode_sweep_g{g}", "fetch_bytes_per_launch")
            sweep.append(dict(g=g, heads_per_group=ws.h // g, kv_cache_bytes=kv,
                              kv_cache_reduction_vs_mha=kv_mha / kv,
                              measured_read_bytes=measured,
                              measured_read_over_law=(measured / kv) if measured else None,
                              mean_ms=st["mean_ms"], GBps=nbytes / (st["mean_ms"] * 1e-3) / 1e9,
                              frac_peak=nbytes / (st["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                              read_same_bytes_us=rd["mean_ms"] * 1e3,
                              read_same_bytes_GBps=kv / (rd["mean_ms"] * 1e-3) / 1e9,
                              frac_of_read_same_bytes=rd["mean_ms"] / st["mean_ms"]))
            log(f"sweep g={g}: {st['mean_ms']*1e3:.1f} us, {sweep[-1]['GBps']:.0f} GB/s; plain read of the "
                f"same {kv/1e6:.0f} MB {rd['mean_ms']*1e3:.1f} us ({sweep[-1]['read_same_bytes_GBps']:.0f} GB/s)")
            del q, kc, vc, kv_buf, out, wsb
            torch.cuda.empty_cache()

    # ---- GQE router with its projection (x W_r^T + top-k), outside the step ----
    grouter = {}
    if run_gqe and run_sweep:
        n_tok = wg.B * wg.T
        rx, rw = router_inputs(n_tok, ROUTER_D_MODEL, wg.h, seed=wg.seed + 200, device=dev)
        for kk in wg.top_k:
            tm = Timer(torch)
            for it in range(3 + args.steps):
                flush.sum()
                if it < 3:
                    gq.gqe_router(rx, rw, wg.g, kk)
                    continue
                with tm:
                    gq.gqe_router(rx, rw, wg.g, kk)
            torch.cuda.synchronize()
            sr = stats(tm.ms())
            # x and w_r read once; logits, idx and gates written
            nb = rx.numel() * 2 + rw.numel() * 2 + n_tok * wg.h * 4 + 2 * n_tok * wg.g * kk * 4
            grouter[f"top{kk}"] = dict(mean_us=sr["mean_ms"] * 1e3, bytes_per_call=nb,
                                       GBps=nb / (sr["mean_ms"] * 1e-3) / 1e9,
                                       frac=nb / (sr["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS)
            log(f"gqe router k={kk}: {sr['mean_ms']*1e3:.1f} us/call, {grouter[f'top{kk}']['GBps']:.0f} GB/s")
        del rx, rw

    # ---- GQE vs dense GQA over the sequence length, outside the step ----
    gsweep = []
    if run_gqe and run_sweep:
        del gq_, gk, gv, glg, gout, gws
        torch.cuda.empty_cache()
        for (B, h, g, T, d, ks, seed) in gqe_sweep_points():
            q, k, v, lg = gqe_inputs(B, h, g, T, d, "bf16", seed=seed, device=dev)
            out = torch.empty_like(q)
            dense_flops = 2.0 * B * h * d * T * (T + 1)

            def timed(fn, n_warm=2, n=5):
                tm = Timer(torch)
                for it in range(n_warm + n):
                    flush.sum()
                    if it < n_warm:
                        fn()
                        continue
                    with tm:
                        fn()
                torch.cuda.synchronize()
                return stats(tm.ms())["median_ms"]

            dense_ms = timed(lambda: gq.gqa_prefill(q, k, v, causal=True, out=out))
            if h == 16:
                # the pages' configuration: k=1 routed experts in 8 groups plus the
                # shared head (9 of 16 query heads), full output build
                qs = torch.randn(B, T, d, device=dev).to(torch.bfloat16)
                ms = timed(lambda: gq.gqe_prefill_build(q, qs, k, v, lg, 1, shared_kv=0))
                gsweep.append(dict(B=B, h=h, g=g, T=T, d=d, top_k=1, build="concat+wsum+shared",
                                   routed_us=ms * 1e3, dense_us=dense_ms * 1e3,
                                   speedup=dense_ms / ms))
                log(f"gqe build h={h} g={g} T={T} B={B} k=1 +shared: {ms*1e3:.1f} us, "
                    f"speed-up {dense_ms/ms:.2f}")
                del qs
            for kk in ks:
                wsb = gq.gqe_workspace_bytes(B, h, g, T, d, kk)
                ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
                ms = timed(lambda: gq.gqe_routed_prefill(q, k, v, lg, kk, causal=True, out=out,
                                                         workspace=ws))
                fl = dense_flops * kk / (h // g)
                gsweep.append(dict(B=B, h=h, g=g, T=T, d=d, top_k=kk, routed_us=ms * 1e3,
                                   dense_us=dense_ms * 1e3, speedup=dense_ms / ms,
                                   routed_tflops=fl / (ms * 1e-3) / 1e12,
                                   dense_tflops=dense_flops / (dense_ms * 1e-3) / 1e12))
                log(f"gqe sweep h={h} g={g} T={T} B={B} k={kk}: routed {ms*1e3:.1f} us, "
                    f"dense {dense_ms*1e3:.1f} us, speed-up {dense_ms/ms:.2f}")
            del q, k, v, lg, out
            torch.cuda.empty_cache()

    # ---- measured peaks: the rates the path is compared with besides the datasheet ----
    peaks = None
    if args.only is None and not args.no_peaks:
        peaks = measured_peaks(torch, gq, dev)

    # ---- CPU oracle baseline on the whole prefill workload, and its parity ----
    cpu = None
    if run_prefill and not args.no_cpu:
        cpu = cpu_baseline(pq, pk, pv, pout, wp)

    line = {
        "metric": METRIC,
        "value": res["prefill"]["tflops"] if "prefill" in res else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "GQA causal prefill bf16/fp32-acc",
            "B": wp.B, "h": wp.h, "g": wp.g, "T": wp.T, "d": wp.d, "causal": True,
            "step": "prefill + decode(B=64,h=32,g=8,d=128,lens U[1024,8192]) + "
                    "GQE(B=2,T=4096,h=32,g=8,d=128,k=1,2)",
        },
    }
    if "prefill" in res:
        p = res["prefill"]
        line["roofline"] = {
            "kernel": "attn_bf16_kernel<128,12,32,3,false>",
            "bound": "mfma",
            "achieved": p["tflops"],
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": p["tflops"] / PEAK_BF16_TFLOPS,
            "traffic": traffic_for("prefill"),
        }
        if peaks:
            line["roofline"]["measured_peak"] = peaks["mfma_bf16"]["TFLOPs"]
            line["roofline"]["frac_measured_peak"] = p["tflops"] / peaks["mfma_bf16"]["TFLOPs"]
            line["roofline"]["attn_tile_loop_peak"] = peaks["attn_tile"]["TFLOPs"]
            line["roofline"]["frac_attn_tile_loop_peak"] = p["tflops"] / peaks["attn_tile"]["TFLOPs"]
        line["prefill"] = {"mean_us": p["mean_ms"] * 1e3, "median_us": p["median_ms"] * 1e3,
                           "min_us": p["min_ms"] * 1e3, "flops_per_launch": p["flops_per_launch"]}
    if "decode" in res:
        dd = res["decode"]
        line["decode"] = {
            "value": dd["GBps"], "unit": "GB/s", "frac": dd["frac_peak"],
            "roofline": {"kernel": "decode_kernel<128,1> + decode_merge_kernel<128>",
                         "bound": "hbm", "achieved": dd["GBps"], "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": dd["frac_peak"],
                         "traffic": traffic_for("decode")},
            "mean_us": dd["mean_ms"] * 1e3, "median_us": dd["median_ms"] * 1e3,
            "min_us": dd["min_ms"] * 1e3, "bytes_per_call": dd["bytes_per_call"],
        }
        if peaks:
            line["decode"]["roofline"]["measured_peak"] = peaks["hbm_read"]["GBps"]
            line["decode"]["roofline"]["frac_measured_peak"] = dd["GBps"] / peaks["hbm_read"]["GBps"]
    if "gqe" in res:
        line["gqe"] = {k: {"tflops": v["tflops"], "frac": v["frac_peak"],
                           "mean_us": v["mean_ms"] * 1e3,
                           "speedup_vs_dense_gqa": v["speedup_vs_dense"]}
                       for k, v in res["gqe"].items()}
        line["gqe"]["dense_gqa_same_shape_us"] = dense_same["mean_ms"] * 1e3
    if sweep:
        line["decode_sweep"] = sweep
    if gsweep:
        line["gqe_sweep"] = gsweep
    if gdec:
        line["gqe_decode"] = gdec
    if grouter:
        line["gqe_router"] = dict(grouter, n_tokens=wg.B * wg.T, d_model=ROUTER_D_MODEL, h=wg.h, g=wg.g)
    if peaks:
        line["measured_peaks"] = peaks
    if cpu:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def measured_peaks(torch, gq, dev, smi=True):
    """The library's peak microbenchmarks, each timed as the median of 10
    launches with HIP events: an HBM read of a 4 GiB buffer (16 times the
    Infinity Cache), and the MFMA-only loop and the prefill's attention tile
    loop (LDS fragment reads, MFMAs and softmax of one tile staged in LDS),
    each once as long as a prefill launch and once long enough for the clock
    to settle under MFMA load. Also the clocks and power cap rocm-smi reports."""
    out = {}
    buf = torch.randint(0, 256, (1 << 32,), dtype=torch.uint8, device=dev)
    xo = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        gq.peak_hbm_read(buf, xo)
    t = Timer(torch)
    for _ in range(10):
        with t:
            gq.peak_hbm_read(buf, xo)
    torch.cuda.synchronize()
    ms = sorted(t.ms())
    out["hbm_read"] = {"GBps": buf.numel() / (ms[5] * 1e-3) / 1e9, "bytes": buf.numel(),
                       "median_us": ms[5] * 1e3, "min_us": ms[0] * 1e3}
    ops = torch.randn(1024, device=dev).to(torch.bfloat16)
    so = torch.zeros(1, dtype=torch.float32, device=dev)
    # 1000 rounds last about as long as one prefill launch (~150 us); 40000
    # rounds (~6 ms) show the rate once the clock has settled under MFMA load.
    for key, iters in (("mfma_bf16", 1000), ("mfma_bf16_sustained", 40000)):
        for _ in range(3):
            gq.peak_mfma_bf16(ops, iters, so)
        t = Timer(torch)
        flops = 0.0
        for _ in range(10):
            gq.peak_hbm_read(buf[: 1 << 30], xo)  # as in the bench step: HBM-bound work between launches
            with t:
                _, flops = gq.peak_mfma_bf16(ops, iters, so)
        torch.cuda.synchronize()
        ms = sorted(t.ms())
        out[key] = {"TFLOPs": flops / (ms[5] * 1e-3) / 1e12, "flops": flops, "iters": iters,
                    "median_us": ms[5] * 1e3, "min_us": ms[0] * 1e3}
    # The prefill's attention tile loop with its operands staged in LDS once:
    # the rate any kernel doing this per-tile work reaches on the chip, with
    # no global memory traffic and no barrier.
    g = torch.Generator(device=dev).manual_seed(12)
    qkv = torch.randn(3, 32, 128, generator=g, device=dev).to(torch.bfloat16)
    for key, iters in (("attn_tile", 300), ("attn_tile_sustained", 8000)):
        for _ in range(3):
            gq.peak_attn_tile(qkv, iters)
        t = Timer(torch)
        flops = 0.0
        for _ in range(10):
            gq.peak_hbm_read(buf[: 1 << 30], xo)
            with t:
                _, flops = gq.peak_attn_tile(qkv, iters)
        torch.cuda.synchronize()
        ms = sorted(t.ms())
        out[key] = {"TFLOPs": flops / (ms[5] * 1e-3) / 1e12, "flops": flops, "iters": iters,
                    "median_us": ms[5] * 1e3, "min_us": ms[0] * 1e3}
    del buf
    torch.cuda.empty_cache()
    log(f"measured peaks: HBM read {out['hbm_read']['GBps']:.0f} GB/s, "
        f"bf16 MFMA {out['mfma_bf16']['TFLOPs']:.0f} TFLOP/s "
        f"({out['mfma_bf16_sustained']['TFLOPs']:.0f} sustained), attention tile loop "
        f"{out['attn_tile']['TFLOPs']:.0f} TFLOP/s ({out['attn_tile_sustained']['TFLOPs']:.0f} sustained)")
    out["rocm_smi"] = rocm_smi_clocks() if smi else None
    return out


def rocm_smi_clocks():
    """sclk/mclk and power lines of rocm-smi (None where it is unavailable)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showmaxpower"],
                           capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    keep = ("sclk", "mclk", "fclk", "power", "Power")
    lines = [ln.strip() for ln in r.stdout.splitlines() if any(k in ln for k in keep)]
    return lines or None


def cpu_baseline(pq, pk, pv, pout, wp):
    """Time the float64 oracle on the whole prefill workload (B=4, h=32, g=8,
    T=2048, d=128, causal: 137.5 GFLOP of algorithmic work), on the same
    inputs the GPU used, then compare its output with the GPU's last timed
    output element by element (outside the timed region)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q, k, v = pq.cpu(), pk.cpu(), pv.cpu()
    flops = 2.0 * wp.B * wp.h * wp.d * wp.T * (wp.T + 1)
    log("cpu baseline: oracle on the whole prefill workload")
    t0 = time.perf_counter()
    out = oracle.gqa_ref(q, k, v, causal=True)
    dt = time.perf_counter() - t0
    gpu = pout.cpu().to(dtype=__import__("torch").float64).numpy()
    err = float(np.abs(gpu - out).max())
    tol = 2e-2  # bf16 inputs, fp32 accumulation
    log(f"cpu baseline: {dt:.2f} s; GPU output vs oracle, all {out.size} elements: "
        f"max|err| = {err:.3e} (tolerance {tol})")
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = None
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": dt, "blas_threads": threads, "cpu_count": os.cpu_count(),
            "sched_affinity": affinity, "cpu_model": cpu_model(),
            "parity": {"max_abs_err": err, "tol": tol, "ok": err <= tol, "elements": int(out.size),
                       "compared": "GPU bf16 output of the timed prefill launch vs the float64 oracle"},
            "sample": "float64 oracle, whole prefill workload B=4 h=32 g=8 T=2048 d=128 causal "
                      f"({flops/1e9:.2f} GFLOP algorithmic); host cpu_count={os.cpu_count()}"}


def cpu_model():
    """The host CPU's model string (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


if __name__ == "__main__":
    main()

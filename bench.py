#!/usr/bin/env python3
"""Benchmark of the reshaped-softmax causal attention hot path on one MI355X.

One step runs the whole path once over resident synthetic inputs:
  * dilution attention forward (three stages) at B=1, H=16, T=16384, d=64,
    bf16, eps=1e-6, 5 % heavy keys -- the per-layer shape of the 24-layer,
    ~209M-parameter decoder at its 16K training context;
  * tempered causal attention forward on the same inputs, tau = YaRN(s=4);
  * one cached dilution decode step: 64 sequences x 32768-key bf16 cache,
    H=16, d=64, fp32 demand updated in place (the 128 queries of the decode
    workload are used in turn).

After the timed steps, the exact backward of both operators (attn_bwd, from
the forward's saved out / lse / row sums and a synthetic dO) is timed the same
way and reported under ``components`` at 10*d flops per causal pair (the
usual 2.5x of the forward's 4*d).  Then, also under ``components``:
  * chunked prefill: the same 16K dilution forward run as 8 chunks of 2048
    rows through attn_prefill, the demand carried in place between chunks;
  * head dimension 128: dilution and tempered forward at B=1, H=20,
    T=16384, d=128 (a 2.7B focal model's attention) with per-head learned
    temperature multipliers, their backward (attn_bwd_ex with those
    multipliers, returning dL/dtau per head as well), and one decode step
    over a 32-sequence x
    32768-key cache at H=20, d=128 with per-(sequence, head) multipliers.

Printed: one JSON line.  ``value`` is the dilution forward's algorithmic
TFLOP/s (4*d flops per causal (query, key) pair: q.k and the weighted v, once)
over the sum of its three launches' median durations; ``roofline`` is that
whole forward against the bf16 matrix peak, with each stage's figures under
``components.dilution_fwd.stages``.  The tempered forward TFLOP/s and the
decode step's HBM GB/s (K + V + demand read + demand write) are reported
under ``components``.  Kernel durations are medians over the timed steps of
HIP events recorded on the stream the library launches on, inside the timed
region.  ``parity`` holds the device's errors against the oracle on the
CPU baseline's sample (the full-size comparisons are the GPU tests').

``executed_mfma_busy_rocprof`` is rocprof's matrix-core busy fraction of the
dilution stages (SQ_VALU_MFMA_BUSY_CYCLES over 4 x SQ_BUSY_CU_CYCLES), read
from the committed counter summary under the same digest rule as
``traffic``.  ``roofline.traffic`` is the measured HBM bytes per launch of the roofline
kernel, read from the committed counter summary under ``profiles/`` when that
summary was taken from the same kernel sources and build flags (a SHA-256 over
them is stored with it), else null.  ``--copy-calibration-mib N`` appends a
plain streaming fp32 copy kernel of N MiB read and N MiB written after the
timed steps: the known-size reference that scales the HBM byte counters.

The MI355X ceilings the roofline fractions use are the published ones (bf16
MFMA 2.5 PFLOP/s, HBM 8 TB/s); each roofline object also carries the same
fraction against ceilings measured in the run (``measured_peaks``: a loop of
independent MFMAs and a streaming read of 8 GiB, libattn_peaks.so).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--copy-calibration-mib N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd TFLOP/s (dilution & tempered) at T=16K; decode HBM GB/s at 32K cache"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E peak
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_dilution_t16k_decode_32k.md")
BUSY_SUMMARY = os.path.join(ROOT, "profiles", "mfma_utilisation_dilution_t16k.md")
CSRC = os.path.join(ROOT, "transformer_attention_causal_amd", "csrc")
FWD_SOURCES = ("attn_common.hpp", "launch.hpp", "tiles.hpp", "fwd_bf16.hip")
DEC_SOURCES = ("attn_common.hpp", "launch.hpp", "decode.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def causal_pairs(B, H, T):
    return B * H * T * (T + 1) // 2


def source_digest(files):
    """SHA-256 over the kernel sources and the hipcc flags they are built with."""
    from transformer_attention_causal_amd.build import FLAGS
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _record(path, tag, key, field, files):
    """Field ``field`` of entry ``key`` of the ``tag`` line of a committed
    counter summary, or None when absent or taken from other sources."""
    try:
        with open(path) as fh:
            for line in fh:
                if line.startswith(tag + ": "):
                    rec = json.loads(line[len(tag) + 2:])
                    ent = rec.get(key)
                    if ent and ent.get("sources_sha256") == source_digest(files):
                        return ent[field]
    except OSError:
        pass
    return None


def measured_traffic(key, files):
    """HBM bytes per launch of kernel ``key`` from the committed counter summary."""
    return _record(TRAFFIC_SUMMARY, "traffic-record", key, "bytes_per_launch", files)


def measured_busy(key, files):
    """rocprof MFMA-busy fraction of ``key`` from the committed counter summary."""
    return _record(BUSY_SUMMARY, "utilisation-record", key, "mfma_busy", files)


def measured_peaks(torch, dev, stream):
    """The GPU's own ceilings, measured in this process with events on the
    library's stream: a loop of independent bf16 32x32x16 MFMAs (8 waves per
    SIMD) and a non-temporal streaming read of an 8 GiB buffer
    (libattn_peaks.so)."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_causal_amd", "libattn_peaks.so"))
    lib.attn_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_peak_mfma_bf16_flops.restype = ctypes.c_double
    lib.attn_peak_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.attn_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    h = stream.cuda_stream

    def timed(fn, reps=3):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    wgs, iters = 256 * 8, 4096
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)

    def mfma():
        if lib.attn_peak_mfma_bf16(iters, wgs, out.data_ptr(), h) != 0:
            raise RuntimeError("attn_peak_mfma_bf16 failed")

    mfma_ms = timed(mfma)
    mfma_tflops = lib.attn_peak_mfma_bf16_flops(iters, wgs) / (mfma_ms * 1e-3) / 1e12
    nbytes = 8 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)

    def read():
        if lib.attn_peak_stream_read(buf.data_ptr(), nbytes, flag.data_ptr(), 256 * 8, h) != 0:
            raise RuntimeError("attn_peak_stream_read failed")

    read_ms = timed(read)
    del buf
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma_tflops, 1),
            "hbm_stream_read_gbps": round(nbytes / (read_ms * 1e-3) / 1e9, 1),
            "how": "independent 32x32x16 bf16 MFMA loop at 8 waves/SIMD; non-temporal "
                   "16-byte streaming read of 8 GiB; events on the bench stream"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps; every figure is the median over them (>= 20 by default)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a streaming fp32 copy of this many MiB three times")
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="heads of the T=16384 dilution workload the oracle runs for the CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path has no multi-GPU form here "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from transformer_attention_causal_amd import binding as ab
    from transformer_attention_causal_amd.workloads import (DECODE, PREFILL, decode_cache_device,
                                                            decode_initial_demand,
                                                            decode_queries, prefill_inputs)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ab.load()

    # ---------------------------------------------------------------- inputs
    w = PREFILL["dilution_t16k"]
    log(f"bench: drawing {w.name} inputs B={w.B} H={w.H} T={w.T}")
    inp = prefill_inputs(w)

    def dev_bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    tau_t = ab.attn_yarn_tau(w.yarn_s)
    out_d = torch.empty_like(q)
    out_t = torch.empty_like(q)
    ws, ws_bytes = ab.fwd_workspace(w.B, w.H, w.T, ab.ATTN_DILUTION, ab.ATTN_BF16, dev)
    stages, _ = ab.dilution_stages(q, k, v, tau=1.0, eps=w.eps, out=out_d, workspace=ws)

    dw = DECODE["decode_32k"]
    log(f"bench: drawing {dw.name} cache S={dw.S} H={dw.H} L={dw.L}")
    kc, vc = decode_cache_device(dw.S, dw.H, dw.L, dw.d, dw.seed, device=dev)
    demand = torch.from_numpy(decode_initial_demand(dw.S, dw.H, dw.L, dw.seed, dw.demand_max)).to(dev)
    qs = dev_bf16(decode_queries(dw.steps, dw.S, dw.H, dw.d, dw.seed))
    dec_out = torch.empty((dw.S, dw.H, dw.d), dtype=torch.bfloat16, device=dev)
    dws, _ = ab.decode_workspace(dw.S, dw.H, dw.L, dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    names = ["dil_lse", "dil_committed", "dil_shares", "tempered", "decode"]

    def step(i, events=None):
        def mark(j):
            if events is not None:
                events[j].record(stream)
        mark(0)
        for j, st in enumerate(stages):
            st()
            mark(j + 1)
        ab.fwd(q, k, v, tau=tau_t, mode=ab.ATTN_TEMPERED, out=out_t)
        mark(4)
        ab.decode(qs[i % dw.steps], kc, vc, demand, tau=dw.tau, eps=dw.eps, out=dec_out,
                  workspace=dws)
        mark(5)

    log(f"bench: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    log(f"bench: timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    seg = {n: [] for n in names}
    for e in evs:
        for j, n in enumerate(names):
            seg[n].append(e[j].elapsed_time(e[j + 1]))
    ms = {n: float(np.median(seg[n])) for n in names}
    ms_min = {n: float(np.min(seg[n])) for n in names}
    # the three dilution launches as one call: first launch's start to the
    # last one's end, the gaps between launches included
    dil_call_ms = float(np.median([e[0].elapsed_time(e[3]) for e in evs]))
    log("bench: per-launch ms " + json.dumps({n: round(ms[n], 4) for n in names}))

    # ------------------------------------------------------------- backward
    from transformer_attention_causal_amd.workloads import draw_grad

    dout = dev_bf16(draw_grad(w.B, w.H, w.T, w.d, w.seed))
    lse_d = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    rs_d = torch.empty_like(lse_d)
    lse_t = torch.empty_like(lse_d)
    ab.fwd(q, k, v, tau=1.0, mode=ab.ATTN_DILUTION, eps=w.eps, out=out_d, workspace=ws,
           lse_out=lse_d, rowsum_out=rs_d)
    ab.fwd(q, k, v, tau=tau_t, mode=ab.ATTN_TEMPERED, out=out_t, lse_out=lse_t)
    bws, _ = ab.bwd_workspace(w.B, w.H, w.T, ab.ATTN_DILUTION, ab.ATTN_BF16, dev)
    grads = [torch.empty_like(q) for _ in range(3)]

    def bwd_step(events=None):
        if events is not None:
            events[0].record(stream)
        ab.bwd(q, k, v, out_d, dout, lse_d, rs_d, tau=1.0, mode=ab.ATTN_DILUTION, eps=w.eps,
               dq=grads[0], dk=grads[1], dv=grads[2], workspace=bws)
        if events is not None:
            events[1].record(stream)
        ab.bwd(q, k, v, out_t, dout, lse_t, None, tau=tau_t, mode=ab.ATTN_TEMPERED,
               dq=grads[0], dk=grads[1], dv=grads[2], workspace=bws)
        if events is not None:
            events[2].record(stream)
        # the same dilution backward reading the forward's committed-demand
        # table (ws still holds the forward's for these inputs) instead of
        # recomputing it
        ab.bwd(q, k, v, out_d, dout, lse_d, rs_d, tau=1.0, mode=ab.ATTN_DILUTION, eps=w.eps,
               dq=grads[0], dk=grads[1], dv=grads[2], workspace=bws, fwd_workspace=ws)
        if events is not None:
            events[3].record(stream)

    for _ in range(args.warmup):
        bwd_step()
    bevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        bwd_step(bevs[i])
    torch.cuda.synchronize()
    bwd_ms = {"dilution_bwd": float(np.median([e[0].elapsed_time(e[1]) for e in bevs])),
              "tempered_bwd": float(np.median([e[1].elapsed_time(e[2]) for e in bevs])),
              "dilution_bwd_fwd_table": float(np.median([e[2].elapsed_time(e[3]) for e in bevs]))}
    log("bench: backward ms " + json.dumps({n: round(x, 4) for n, x in bwd_ms.items()}))
    del bws, grads

    def time_launches(fn, n_marks):
        """Median ms between consecutive marks of ``fn(events)`` over the timed
        iterations (warm-up iterations first)."""
        for _ in range(args.warmup):
            fn(None)
        evs_ = [[torch.cuda.Event(enable_timing=True) for _ in range(n_marks)]
                for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            fn(evs_[i])
        torch.cuda.synchronize()
        return [float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs_]))
                for j in range(n_marks - 1)]

    # ------------------------------------------------------- chunked prefill
    chunk = 2048
    dem_c = torch.zeros((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    pws_need = [ab.attn_prefill_workspace_bytes(w.B, w.H, chunk, e, w.d, 1, 1)
                for e in range(chunk, w.T + 1, chunk)]
    pws = torch.empty(max(pws_need), dtype=torch.uint8, device=dev)
    q_chunks = [q[:, :, a:a + chunk].contiguous() for a in range(0, w.T, chunk)]
    out_c = torch.empty_like(q_chunks[0])

    def chunked(events):
        if events is not None:
            events[0].record(stream)
        dem_c.zero_()
        for c, qc in enumerate(q_chunks):
            ab.prefill(qc, k, v, (c + 1) * chunk, tau=1.0, mode=ab.ATTN_DILUTION, eps=w.eps,
                       demand_in=dem_c, demand_out=dem_c, out=out_c, workspace=pws)
        if events is not None:
            events[1].record(stream)

    chunk_ms = time_launches(chunked, 2)[0]
    log(f"bench: chunked prefill ({w.T // chunk} x {chunk} rows) {chunk_ms:.4f} ms")
    del pws, q_chunks, out_c, dem_c

    # ------------------------------------------------------ head dimension 128
    from transformer_attention_causal_amd.workloads import learned_tau

    w8 = PREFILL["focal_d128_t16k"]
    log(f"bench: drawing {w8.name} inputs B={w8.B} H={w8.H} T={w8.T} d={w8.d}")
    inp8 = prefill_inputs(w8)
    q8, k8, v8 = dev_bf16(inp8.q), dev_bf16(inp8.k), dev_bf16(inp8.v)
    del inp8
    tau8 = torch.from_numpy(learned_tau(w8.B, w8.H, w8.d, seed=w8.seed)).to(dev)
    out8 = torch.empty_like(q8)
    ws8 = torch.empty(ab.attn_prefill_workspace_bytes(w8.B, w8.H, w8.T, w8.T, w8.d, 1, 1),
                      dtype=torch.uint8, device=dev)

    def d128(events):
        if events is not None:
            events[0].record(stream)
        ab.prefill(q8, k8, v8, w8.T, tau=1.0, mode=ab.ATTN_DILUTION, eps=w8.eps, out=out8,
                   workspace=ws8, tau_bh=tau8)
        if events is not None:
            events[1].record(stream)
        ab.prefill(q8, k8, v8, w8.T, tau=1.0, mode=ab.ATTN_TEMPERED, out=out8, tau_bh=tau8)
        if events is not None:
            events[2].record(stream)

    d128_ms = time_launches(d128, 3)
    log(f"bench: d=128 forward ms dilution {d128_ms[0]:.4f} tempered {d128_ms[1]:.4f}")

    # d = 128 backward with the per-head multipliers and their gradient
    g8 = dev_bf16(draw_grad(w8.B, w8.H, w8.T, w8.d, w8.seed))
    lse8 = torch.empty((w8.B, w8.H, w8.T), dtype=torch.float32, device=dev)
    rs8, lse8t = torch.empty_like(lse8), torch.empty_like(lse8)
    out8t = torch.empty_like(q8)
    dtau8 = torch.empty((w8.B, w8.H), dtype=torch.float32, device=dev)
    ab.prefill(q8, k8, v8, w8.T, tau=1.0, mode=ab.ATTN_DILUTION, eps=w8.eps, out=out8,
               workspace=ws8, tau_bh=tau8, lse_out=lse8, rowsum_out=rs8)
    ab.prefill(q8, k8, v8, w8.T, tau=1.0, mode=ab.ATTN_TEMPERED, out=out8t, tau_bh=tau8,
               lse_out=lse8t)
    bws8, _ = ab.bwd_workspace(w8.B, w8.H, w8.T, ab.ATTN_DILUTION, ab.ATTN_BF16, dev, w8.d)
    grads8 = [torch.empty_like(q8) for _ in range(3)]

    def bwd128(events):
        if events is not None:
            events[0].record(stream)
        ab.bwd(q8, k8, v8, out8, g8, lse8, rs8, mode=ab.ATTN_DILUTION, eps=w8.eps,
               dq=grads8[0], dk=grads8[1], dv=grads8[2], workspace=bws8, tau_bh=tau8,
               dtau_out=dtau8)
        if events is not None:
            events[1].record(stream)
        ab.bwd(q8, k8, v8, out8t, g8, lse8t, None, mode=ab.ATTN_TEMPERED,
               dq=grads8[0], dk=grads8[1], dv=grads8[2], workspace=bws8, tau_bh=tau8,
               dtau_out=dtau8)
        if events is not None:
            events[2].record(stream)
        # dilution again, reading the forward's committed-demand table from ws8
        ab.bwd(q8, k8, v8, out8, g8, lse8, rs8, mode=ab.ATTN_DILUTION, eps=w8.eps,
               dq=grads8[0], dk=grads8[1], dv=grads8[2], workspace=bws8, tau_bh=tau8,
               dtau_out=dtau8, fwd_workspace=ws8)
        if events is not None:
            events[3].record(stream)

    bwd8_ms = time_launches(bwd128, 4)
    log(f"bench: d=128 backward ms (per-head tau, dL/dtau) dilution {bwd8_ms[0]:.4f} "
        f"tempered {bwd8_ms[1]:.4f} dilution reading the forward's table {bwd8_ms[2]:.4f}")
    del q8, k8, v8, out8, out8t, g8, bws8, grads8, lse8, rs8, lse8t, ws8

    S8, H8, L8 = 32, 20, 32768
    kc8, vc8 = decode_cache_device(S8, H8, L8, 128, dw.seed + 1, device=dev)
    dem8 = torch.from_numpy(decode_initial_demand(S8, H8, L8, dw.seed + 1)).to(dev)
    qs8 = dev_bf16(decode_queries(dw.steps, S8, H8, 128, dw.seed + 1))
    tsh8 = torch.from_numpy(learned_tau(S8, H8, 128, seed=dw.seed + 1)).to(dev)
    dws8, _ = ab.decode_workspace(S8, H8, L8, dev, 128)
    dout8 = torch.empty((S8, H8, 128), dtype=torch.bfloat16, device=dev)
    dstep = [0]

    def dec128(events):
        if events is not None:
            events[0].record(stream)
        ab.decode(qs8[dstep[0] % dw.steps], kc8, vc8, dem8, tau=1.0, eps=dw.eps, out=dout8,
                  workspace=dws8, tau_sh=tsh8)
        dstep[0] += 1
        if events is not None:
            events[1].record(stream)

    dec8_ms = time_launches(dec128, 2)[0]
    dec8_bytes = (2.0 * S8 * H8 * L8 * 128 * 2 + 2.0 * S8 * H8 * L8 * 4 + 2.0 * S8 * H8 * 128 * 2)
    log(f"bench: d=128 decode step {dec8_ms:.4f} ms")
    del kc8, vc8, dem8, dws8

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        log(f"bench: calibration copy {args.copy_calibration_mib} MiB read + written, 3 launches")
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    log("bench: measured peaks (MFMA loop, 8 GiB streaming read)")
    peaks = measured_peaks(torch, dev, stream)
    log("bench: measured peaks " + json.dumps({k: v for k, v in peaks.items() if k != "how"}))

    # ------------------------------------------------------------ throughputs
    d = w.d
    flops = 4.0 * d * causal_pairs(w.B, w.H, w.T)            # algorithmic, per forward
    dil_ms = ms["dil_lse"] + ms["dil_committed"] + ms["dil_shares"]
    dil_tflops = flops / (dil_ms * 1e-3) / 1e12
    tmp_tflops = flops / (ms["tempered"] * 1e-3) / 1e12
    dec_bytes = (2.0 * dw.S * dw.H * dw.L * dw.d * 2        # K and V caches, bf16
                 + 2.0 * dw.S * dw.H * dw.L * 4             # demand read + write, fp32
                 + 2.0 * dw.S * dw.H * dw.d * 2)            # query in, output out
    dec_gbps = dec_bytes / (ms["decode"] * 1e-3) / 1e9
    flops8 = 4.0 * w8.d * causal_pairs(w8.B, w8.H, w8.T)
    # per-stage figures of the dilution forward: each stage's share of the
    # forward's time, its executed matrix-core busy fraction and measured HBM
    # bytes per launch (counter summaries), and the forward's algorithmic
    # flops over the stage's own time (what the forward would reach if every
    # stage ran as fast as this one)
    stage_kernels = {"dil_lse": "rows_bf16_kernel<kRowLse>",
                     "dil_committed": "colsum_bf16_kernel",
                     "dil_shares": "rows_bf16_kernel<kRowShare>"}
    stages_out = {}
    for n, kname in stage_kernels.items():
        stages_out[n] = {
            "kernel": kname, "ms": round(ms[n], 4), "min_ms": round(ms_min[n], 4),
            "share_of_forward": round(ms[n] / dil_ms, 4),
            "executed_mfma_busy_rocprof": measured_busy(kname, FWD_SOURCES),
            "traffic": measured_traffic(kname, FWD_SOURCES)}
    tr = [stages_out[n]["traffic"] for n in stage_kernels]
    fwd_traffic = sum(tr) if all(t is not None for t in tr) else None

    result = {
        "metric": METRIC,
        "value": round(dil_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "dilution_t16k (value) + tempered_t16k + decode_32k step",
            "B": w.B, "H": w.H, "T": w.T, "d": d, "eps": w.eps, "heavy_key_frac": w.heavy_frac,
            "tempered_tau": tau_t,
            "decode": {"S": dw.S, "H": dw.H, "L": dw.L, "d": dw.d, "steps_in_workload": dw.steps},
        },
        "components": {
            "dilution_fwd": {"ms": round(dil_ms, 4), "tflops": round(dil_tflops, 3),
                             "frac_of_bf16_peak": round(dil_tflops / PEAK_BF16_TFLOPS, 4),
                             "stages": stages_out,
                             "whole_call_ms": round(dil_call_ms, 4),
                             "whole_call_tflops": round(flops / (dil_call_ms * 1e-3) / 1e12, 3),
                             "executed_mfma_busy_rocprof": measured_busy("dilution_fwd", FWD_SOURCES)},
            "tempered_fwd": {"ms": round(ms["tempered"], 4), "tflops": round(tmp_tflops, 3),
                             "frac_of_bf16_peak": round(tmp_tflops / PEAK_BF16_TFLOPS, 4),
                             "kernel": "rows_bf16_kernel<kRowTempered>",
                             "executed_mfma_busy_rocprof": measured_busy(
                                 "rows_bf16_kernel<kRowTempered>", FWD_SOURCES),
                             "traffic": measured_traffic("rows_bf16_kernel<kRowTempered>",
                                                         FWD_SOURCES)},
            "decode_step": {"ms": round(ms["decode"], 4), "gbps": round(dec_gbps, 2),
                            "bytes": dec_bytes,
                            "frac_of_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4)},
            "min_ms": {n: round(ms_min[n], 4) for n in names},
            "dilution_bwd": {"ms": round(bwd_ms["dilution_bwd"], 4),
                             "tflops": round(2.5 * flops / (bwd_ms["dilution_bwd"] * 1e-3) / 1e12, 3)},
            "dilution_bwd_reading_fwd_table": {
                "ms": round(bwd_ms["dilution_bwd_fwd_table"], 4),
                "tflops": round(2.5 * flops / (bwd_ms["dilution_bwd_fwd_table"] * 1e-3) / 1e12, 3),
                "note": "attn_bwd_ex given the forward's workspace: no committed-demand pass"},
            "tempered_bwd": {"ms": round(bwd_ms["tempered_bwd"], 4),
                             "tflops": round(2.5 * flops / (bwd_ms["tempered_bwd"] * 1e-3) / 1e12, 3)},
            "dilution_chunked_prefill": {
                "chunks": w.T // chunk, "rows_per_chunk": chunk, "ms": round(chunk_ms, 4),
                "tflops": round(flops / (chunk_ms * 1e-3) / 1e12, 3),
                "vs_whole_prefill": round(dil_ms / chunk_ms, 4)},
            "focal_d128_t16k": {
                "B": w8.B, "H": w8.H, "T": w8.T, "d": w8.d, "tau": "per head, sqrt(d)/U[5,10]",
                "dilution_ms": round(d128_ms[0], 4),
                "dilution_tflops": round(flops8 / (d128_ms[0] * 1e-3) / 1e12, 3),
                "tempered_ms": round(d128_ms[1], 4),
                "tempered_tflops": round(flops8 / (d128_ms[1] * 1e-3) / 1e12, 3),
                "dilution_bwd_ms": round(bwd8_ms[0], 4),
                "dilution_bwd_tflops": round(2.5 * flops8 / (bwd8_ms[0] * 1e-3) / 1e12, 3),
                "dilution_bwd_reading_fwd_table_ms": round(bwd8_ms[2], 4),
                "tempered_bwd_ms": round(bwd8_ms[1], 4),
                "tempered_bwd_tflops": round(2.5 * flops8 / (bwd8_ms[1] * 1e-3) / 1e12, 3),
                "bwd_outputs": "dq, dk, dv and dL/dtau per head"},
            "decode_d128_32k": {
                "S": S8, "H": H8, "L": L8, "d": 128, "ms": round(dec8_ms, 4),
                "gbps": round(dec8_bytes / (dec8_ms * 1e-3) / 1e9, 2), "bytes": dec8_bytes,
                "frac_of_hbm_peak": round(dec8_bytes / (dec8_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "dilution forward, its three launches: rows_bf16_kernel<kRowLse> "
                      "(log-sum-exp), colsum_bf16_kernel (committed demand), "
                      "rows_bf16_kernel<kRowShare> (shares and share@V)",
            "achieved": round(dil_tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dil_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": fwd_traffic,
            "measured_peak": peaks["mfma_bf16_tflops"],
            "frac_of_measured_peak": round(dil_tflops / peaks["mfma_bf16_tflops"], 4),
            "executed_mfma_busy_rocprof": measured_busy("dilution_fwd", FWD_SOURCES),
            "units": f"{causal_pairs(w.B, w.H, w.T)} causal pairs x {4 * d} flops (q.k and the "
                     f"weighted v, once) over the sum of the three launches' median durations",
        },
        "roofline_decode": {
            "bound": "hbm",
            "kernel": "attn_decode step (dec_fused<64>: one workgroup per (sequence, head), "
                      "scores in LDS)",
            "achieved": round(dec_gbps, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
            "measured_peak": peaks["hbm_stream_read_gbps"],
            "frac_of_measured_peak": round(dec_gbps / peaks["hbm_stream_read_gbps"], 4),
            "traffic": measured_traffic("attn_decode", DEC_SOURCES),
        },
        "measured_peaks": peaks,
    }

    if not args.no_cpu_baseline:
        # the device's results on the oracle's sample, for the parity figures:
        # the first heads of the 16K forward (both operators, with LSE and
        # final demand) and one decode step from the initial demand on the
        # first sequences of the device's own cache
        heads = list(range(min(args.cpu_heads, w.H)))
        ns = 4
        lse_s = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
        dem_s = torch.empty_like(lse_s)
        ab.fwd(q, k, v, tau=1.0, mode=ab.ATTN_DILUTION, eps=w.eps, out=out_d, workspace=ws,
               lse_out=lse_s, demand_out=dem_s)
        ab.fwd(q, k, v, tau=tau_t, mode=ab.ATTN_TEMPERED, out=out_t)
        dem0 = torch.from_numpy(decode_initial_demand(dw.S, dw.H, dw.L, dw.seed,
                                                      dw.demand_max)).to(dev)
        ab.decode(qs[0], kc, vc, dem0, tau=dw.tau, eps=dw.eps, out=dec_out, workspace=dws)
        torch.cuda.synchronize()
        got = {"dil": out_d[:, heads].float().cpu().numpy(),
               "dil_lse": lse_s[:, heads].cpu().numpy(),
               "dil_dem": dem_s[:, heads].cpu().numpy(),
               "tmp": out_t[:, heads].float().cpu().numpy(),
               "dec": dec_out[:ns].float().cpu().numpy(),
               "dec_dem": dem0[:ns].cpu().numpy(),
               "kc": kc[:ns].contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
               "vc": vc[:ns].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)}
        del dem0
        result["cpu_baseline"], result["parity"] = cpu_baseline(inp, w, heads, tau_t, dw, ns, got)
    print(json.dumps(result), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _parity(got, ref):
    import numpy as np

    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    return {"max_abs": float(np.max(np.abs(diff))),
            "rel_rms": float(np.linalg.norm(diff) / np.linalg.norm(ref))}


def cpu_baseline(inp, w, heads, tau_t, dw, ns, got):
    """The fp64 oracle (untuned) on a bounded sample of the same workloads:
    the dilution forward (the headline figure) on the first heads of the 16K
    workload, and beside it the tempered forward on the same heads and one
    decode step over the first sequences of the device's cache.  The oracle's
    results on that sample also give the device's parity figures."""
    import numpy as np

    import oracle
    from transformer_attention_causal_amd.workloads import (decode_initial_demand,
                                                            decode_queries)

    log(f"bench: cpu baseline (oracle) on {len(heads)} head(s) of T={w.T} dilution")
    sub = [oracle.Bf16(np.ascontiguousarray(x[:, heads])) for x in (inp.q, inp.k, inp.v)]
    t0 = time.perf_counter()
    ref_d, lse_d, dem_d = oracle.dilution_fwd(*sub, 1.0, w.eps)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * causal_pairs(1, len(heads), w.T)
    t0 = time.perf_counter()
    ref_t, _ = oracle.tempered_fwd(*sub, tau_t)
    dt_t = time.perf_counter() - t0
    # one decode step: the first sequences of the device's cache, from the
    # initial demand, with the first step's queries
    dem = decode_initial_demand(dw.S, dw.H, dw.L, dw.seed, dw.demand_max)[:ns].astype(np.float64)
    qd = np.ascontiguousarray(decode_queries(1, dw.S, dw.H, dw.d, dw.seed)[0][:ns])
    t0 = time.perf_counter()
    ref_dec = oracle.dilution_decode_step(oracle.Bf16(qd), oracle.Bf16(got["kc"]),
                                          oracle.Bf16(got["vc"]), dem, dw.tau, dw.eps)
    dt_d = time.perf_counter() - t0
    dec_bytes = ns * dw.H * (2.0 * dw.L * dw.d * 2 + 2.0 * dw.L * 4 + 2.0 * dw.d * 2)
    log(f"bench: cpu baseline {dt:.2f} s dilution, {dt_t:.2f} s tempered, {dt_d:.3f} s decode")
    dem_tot = np.max(np.abs(got["dil_dem"].astype(np.float64).sum(-1) / w.T - 1.0))
    dec_tot = np.max(np.abs(got["dec_dem"].astype(np.float64).sum(-1) / dem.sum(-1) - 1.0))
    parity = {
        "bars": {"bf16_max_abs": 2e-2, "bf16_rel_rms": 1e-2, "demand_total_rel": 1e-4},
        "dilution_t16k": {"heads": heads, "rows": "all",
                          **_parity(got["dil"], ref_d),
                          "lse_max_abs": float(np.max(np.abs(got["dil_lse"] - lse_d))),
                          "demand_total_rel": float(dem_tot),
                          "demand_per_key_max_abs": float(np.max(np.abs(got["dil_dem"] - dem_d)))},
        "tempered_t16k": {"heads": heads, "rows": "all", "tau": tau_t,
                          **_parity(got["tmp"], ref_t)},
        "decode_32k": {"sequences": ns, "heads": dw.H, "step": "first, from the initial demand",
                       **_parity(got["dec"], ref_dec),
                       "demand_total_rel": float(dec_tot),
                       "demand_per_key_max_abs": float(np.max(np.abs(got["dec_dem"] - dem)))},
        "full_coverage": "tests/test_gpu_workloads.py: every row of every head at T=16384, "
                         "every row of head 0 at T=131072, every decode pair at every step",
    }
    threads = oracle.num_threads()
    base = {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cores_available": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": f"dilution forward, {len(heads)} of {w.H} heads at T={w.T} (all rows), "
                  f"{dt:.2f} s, fp64, {threads} OpenMP threads; a bounded sample, not the "
                  f"whole workload",
        "also": {
            "tempered_fwd": {"value": round(flops / dt_t / 1e12, 6), "unit": "TFLOP/s",
                             "sample": f"the same {len(heads)} heads, tau={tau_t:.7f}, "
                                       f"{dt_t:.2f} s"},
            "decode_step": {"value": round(dec_bytes / dt_d / 1e9, 3), "unit": "GB/s",
                            "sample": f"one step, {ns} of {dw.S} sequences x {dw.H} heads x "
                                      f"{dw.L} keys, {dt_d:.3f} s"},
        },
    }
    return base, parity


if __name__ == "__main__":
    main()

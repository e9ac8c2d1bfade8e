#!/usr/bin/env python3
"""Benchmark: HCA attention forward + backward on one MI355X.

A step is one pass of the whole hot path on one batch of synthetic input
already resident in device memory: hca_attn_fwd (KV transposes + forward
kernel) then hca_attn_bwd (transposes, dQ kernel, dKV kernel, reduction).  The
block table is built once per sequence layout, outside the timed region
(it depends only on S, r, W and the document starts), and its build time is
reported as plan_build_ms.

Prints one JSON line.  value = effective TFLOP/s of forward + backward
= 14 * D * H * P / time, where P is the number of visible (position, key)
pairs (forward 4 * D * H * P, backward 10 * D * H * P; masked work excluded).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_F32_TFLOPS = 157.3  # MI355X fp32 vector ALU, published
PEAK_HBM_GBS = 8000.0

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_sparse_compressed_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# HBM bytes per launch measured with rocprofv3's L2-to-memory request counters
# (TCC_EA0_RDREQ_32B / _64B / _128B times their sizes for reads, TCC_EA0_WRREQ_64B
# and TCC_EA0_WRREQ for writes; the same arithmetic on a plain copy of known size
# gives its size back): "traffic:" JSON lines, one per kernel and workload, in
# profiles/hbm_traffic_<workload>.md.  MFMA and LDS utilisation from rocprofv3's
# derived counters: "mfma:" JSON lines in profiles/mfma_util.md.
MFMA_FILE = os.path.join(PROFILES, "mfma_util.md")
KERNEL_SOURCES = {"fwd": "hca_fwd.hip", "bwd_pds": "hca_bwd.hip", "bwd_dq": "hca_bwd.hip",
                  "bwd_dkv": "hca_bwd.hip", "dkv_reduce": "hca_bwd.hip",
                  "transpose": "hca_fwd.hip"}


def source_hash(kernel):
    """Hash of the sources that decide a kernel's memory traffic: its .hip file, the
    shared device headers and the planner (launch order)."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "hca_stage.h", "hca_device.h", "hca_internal.h",
              "hca_plan.cpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _records(path, tag, kernel, workload):
    """The "tag:" JSON record of this kernel and workload in a profile summary, or
    None when there is none for the kernel's current sources."""
    try:
        with open(path) as fh:
            lines = [ln[len(tag):] for ln in fh if ln.startswith(tag)]
    except OSError:
        return None
    want = source_hash(kernel) if kernel in KERNEL_SOURCES else None
    for ln in lines:
        rec = json.loads(ln)
        if rec.get("kernel") == kernel and rec.get("workload") == workload and \
                rec.get("source") == want:
            return rec
    return None


def recorded_traffic(kernel, workload):
    """Measured HBM bytes per launch for this kernel and workload, or None."""
    rec = _records(os.path.join(PROFILES, "hbm_traffic_%s.md" % workload), "traffic:",
                   kernel, workload)
    return rec["bytes_per_launch"] if rec else None


def recorded_util(kernel, workload):
    """Measured MfmaUtil / LdsUtil / LDSBankConflict (fractions) or None."""
    rec = _records(MFMA_FILE, "mfma:", kernel, workload)
    return {k: rec[k] for k in ("mfma_util", "lds_util", "lds_bank_conflict")} if rec else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_bf16",
                    help="tiny_fp32 | packed_bf16 | mid_bf16 | long_bf16 | max_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the CPU oracle sample")
    ap.add_argument("--comp-item-chunks", type=int, default=0,
                    help="64-position chunks per compressed-tile work item of the key-"
                         "stationary backward (0 = library choice)")
    ap.add_argument("--half-items-min", type=int, default=0,
                    help="item count from which half-tile items are used (0 = library "
                         "choice, -1 = never)")
    ap.add_argument("--kv-keys", type=int, default=0,
                    help="keys per key tile of the key-stationary backward (0 = library "
                         "choice; 64 or 128 at head dim 512)")
    ap.add_argument("--comp-pattern", default="rule", choices=("rule", "dense", "topk"),
                    help="rule: the analytic plan; dense: the same pattern materialised as a "
                         "dense compressed-key mask kept in device memory, planned from the "
                         "mask (the dynamic-mask comparison); topk: the CSA form, per-query "
                         "compressed-entry selections (workload csa_topk_bf16)")
    ap.add_argument("--source-hashes", action="store_true",
                    help="print the source hash of each kernel and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times), the "
                         "reference kernel that checks the HBM request-counter arithmetic")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")
    return args


def copy_probe(mib):
    """A plain copy kernel of known size: reads and writes exactly mib MiB per launch."""
    import torch

    n = mib * 2**20 // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert bool((dst[-4:] == src[-4:]).all())
    print(json.dumps({"copy_probe_bytes": n * 4, "launches": 3}), flush=True)


def cpu_baseline(wl, target_s):
    """Times the oracle on the first S' positions of the workload (all heads), full
    forward + backward in fp64, doubling S' until the run takes target_s."""
    import numpy as np

    import oracle
    from hca_inputs import draw, segment_ids

    oracle.build()
    Sp = 64
    best = None
    while True:
        Sp = min(Sp, wl.S)
        Sc = Sp // wl.r
        q, kv, kvc, dout = draw(1, Sp, wl.H, wl.D, Sc, wl.dtype, wl.seed, wl.value_scale, "cpu")
        from hca_inputs import to_host_bits

        host = [to_host_bits(t) for t in (q, kv, kvc, dout)]
        prob = oracle.Problem(1, Sp, wl.H, wl.D, wl.r, wl.W, Sc, 1.0 / math.sqrt(wl.D),
                              segment_ids(None, 1, Sp), oracle.STRICT, wl.dtype)
        t0 = time.perf_counter()
        oracle.full(prob, *host)
        dt = time.perf_counter() - t0
        pairs = oracle.count_pairs(prob, 0) + oracle.count_pairs(prob, 1)
        flops = 14.0 * wl.D * wl.H * pairs
        best = (Sp, dt, flops)
        if dt >= target_s or Sp >= wl.S or Sp >= 8192:
            break
        Sp *= 2
    Sp, dt, flops = best
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh
                              if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model, "kind": "oracle",
            "sample": "first %d positions of %s (1 document, all %d heads), full forward + "
                      "backward in fp64, %.1f s" % (Sp, wl.name, wl.H, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the library runs on exactly one GPU; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.source_hashes:
        print(json.dumps({k: source_hash(k) for k in KERNEL_SOURCES}))
        return
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    import torch

    import numpy as np

    import block_sparse_compressed_amd as hca
    from hca_inputs import (CSA_TOPK, CSA_TOPK_K, WORKLOADS, doc_lengths, draw_workload,
                            starts_csr, topk_indices)

    if args.comp_pattern == "topk":
        args.workload = CSA_TOPK.name
    wl = {w.name: w for w in list(WORKLOADS.values()) + [CSA_TOPK]}[args.workload]
    if (wl is CSA_TOPK) != (args.comp_pattern == "topk"):
        print("bench.py: workload %s goes with --comp-pattern %s" % (
            wl.name, "topk" if wl is CSA_TOPK else "rule or dense"), file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lengths = doc_lengths(wl)
    starts, counts = starts_csr(lengths, wl.B)
    dt = hca.HCA_BF16 if wl.dtype == "bf16" else hca.HCA_F32
    tiles = None
    if args.comp_item_chunks or args.half_items_min or args.kv_keys:
        tiles = (0, 0, 0, args.half_items_min, args.comp_item_chunks, args.kv_keys)

    # Plan build (host), timed once outside the step loop.  dense: the analytic
    # plan's per-position intervals give the dense mask of the same pattern,
    # which is then planned from the mask (every element read).
    comp_mask = topk = None
    if args.comp_pattern == "dense":
        rows = hca.hca_plan_export_rows(hca.hca_block_mask_build(
            wl.B, wl.S, wl.r, wl.W, wl.Sc, starts, counts, wl.H, wl.D, dt))
        c = np.arange(wl.Sc, dtype=np.int32)[None, None, :]
        comp_mask = ((c >= rows[:, :, 1:2]) & (c < rows[:, :, 2:3])).astype(np.uint8)
    if args.comp_pattern == "topk":
        topk = topk_indices(wl, CSA_TOPK_K)

    def build_plan():
        if comp_mask is not None:
            return hca.hca_block_mask_build_masked(wl.B, wl.S, wl.W, wl.Sc, comp_mask, starts,
                                                   counts, wl.H, wl.D, dt, tiles)
        if topk is not None:
            return hca.hca_block_mask_build_topk(wl.B, wl.S, wl.W, wl.Sc, topk, starts, counts,
                                                 wl.H, wl.D, dt, tiles)
        return hca.hca_block_mask_build(wl.B, wl.S, wl.r, wl.W, wl.Sc, starts, counts, wl.H,
                                        wl.D, dt, hca.HCA_COMPSEG_STRICT, tiles)

    t0 = time.perf_counter()
    plan = build_plan()
    plan_ms = (time.perf_counter() - t0) * 1e3

    q, kv, kvc, dout = draw_workload(wl, device=dev)
    torch.cuda.reset_peak_memory_stats()
    # dense: the materialised mask stays resident in device memory, as in a
    # pipeline that hands the attention a dense mask each step.
    mask_dev = torch.from_numpy(comp_mask).to(dev) if comp_mask is not None else None
    att = hca.HcaAttention(wl.B, wl.S, wl.H, wl.D, wl.r, wl.W, wl.dtype, starts, counts,
                           tiles=tiles, plan=plan)
    info = att.info
    scale = 1.0 / math.sqrt(wl.D)
    o, lse = att.new_outputs()
    grads = att.new_grads()

    def step():
        att.forward(q, kv, kvc, scale, o, lse)
        att.backward(q, kv, kvc, o, lse, dout, scale, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Forward alone, for the forward-only figure.
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        att.forward(q, kv, kvc, scale, o, lse)
    ev[1].record(stream)
    torch.cuda.synchronize()
    fwd_ms = ev[0].elapsed_time(ev[1]) / args.steps

    # Timed region: K full steps, nothing else on the GPU or the host in between.
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(stop) / args.steps
    # The same K steps again with the library's per-kernel HIP events (recorded on
    # the stream each kernel runs on): the per-kernel durations of the roofline
    # object.  The event records add a little time per kernel, so the headline
    # step time comes from the uninstrumented pass above.
    hca.hca_timing_read()
    hca.hca_timing_enable(True)
    torch.cuda.synchronize()
    start_i = torch.cuda.Event(enable_timing=True)
    stop_i = torch.cuda.Event(enable_timing=True)
    start_i.record(stream)
    for _ in range(args.steps):
        step()
    stop_i.record(stream)
    torch.cuda.synchronize()
    hca.hca_timing_enable(False)
    kernels = hca.hca_timing_read()
    ms_instrumented = start_i.elapsed_time(stop_i) / args.steps
    peak_mem = torch.cuda.max_memory_allocated() / 2**30

    P = info.pairs_raw + info.pairs_comp
    fl_fwd = 4.0 * wl.D * wl.H * P
    fl_all = 14.0 * wl.D * wl.H * P
    # Algorithmic work per launch of each kernel: flops, and the bytes it must move
    # (inputs read once, outputs written once; transposed copies and fp32 partial
    # sums are workspace, not counted).  A kernel's roofline is whichever of
    # flops / peak and bytes / HBM bandwidth takes longer.
    e = 2 if wl.dtype == "bf16" else 4
    qb = wl.B * wl.H * wl.S * wl.D * e          # one [B,H,S,D] tensor
    kb = (wl.B * wl.S + wl.B * wl.Sc) * wl.D * e  # kv and kv_comp
    rb = 4 * wl.B * wl.H * wl.S                  # one fp32 value per row (LSE, delta)
    DHP = wl.D * wl.H * P
    per_kernel = {  # kernel: (flops, bytes)
        "fwd": (fl_fwd, 2 * qb + kb + rb),                          # Q, K -> O, LSE
        "bwd_dq": (6.0 * DHP, 4 * qb + kb + 2 * rb),                # Q, dO, O, LSE, K -> dQ, delta
        "bwd_dkv": (4.0 * DHP, 2 * qb + kb + 2 * rb),               # Q, dO, LSE, delta, K
        "fwd_f32": (fl_fwd, 2 * qb + kb + rb),
        "bwd_f32": (10.0 * DHP, 5 * qb + 2 * kb + rb),
    }
    if info.ws_pds_bytes:
        # Stored P / dS: the first pass forms S, dP, P and dS (Q, dO, O, LSE, K ->
        # delta), the dQ pass only dQ = sum dS K (K -> dQ); the stored tiles are
        # workspace, not algorithmic bytes.
        per_kernel["bwd_pds"] = (4.0 * DHP, 3 * qb + kb + 2 * rb)
        per_kernel["bwd_dq"] = (2.0 * DHP, qb + kb)
    kavg = {k: v[1] / v[0] for k, v in kernels.items() if v[0]}
    per_step = {k: kernels[k][1] / args.steps for k in kernels}
    # With stored P / dS the dQ pass runs on the library's second stream while
    # the key-stationary pass runs on the caller's: its event span covers the
    # whole overlap and is no exclusive time, so the dominant kernel is taken
    # among the kernels of the caller's stream, whose spans add up to the step.
    concurrent = {"bwd_dq"} if info.ws_pds_bytes else set()
    dom = max((k for k in per_step if k in per_kernel and k not in concurrent),
              key=lambda k: per_step[k])
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS

    def roof(flops, nbytes, t_ms):
        t_mfma = flops / (peak * 1e12)
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
        if t_hbm > t_mfma:
            return dict(bound="hbm", achieved=round(nbytes / (t_ms * 1e-3) / 1e9, 2),
                        peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(t_hbm / (t_ms * 1e-3), 4))
        # bf16 runs on the matrix cores; the float32 path is vector-ALU code
        # (peak: fp32 vector rate of 256 CUs at 2.4 GHz).
        return dict(bound="mfma" if wl.dtype == "bf16" else "alu",
                    achieved=round(flops / (t_ms * 1e-3) / 1e12, 2), peak=peak,
                    unit="TFLOP/s", frac=round(t_mfma / (t_ms * 1e-3), 4))

    roofline = roof(*per_kernel[dom], kavg[dom])
    util = recorded_util(dom, wl.name)
    roofline.update(kernel=dom, traffic=recorded_traffic(dom, wl.name),
                    mfma_util=util["mfma_util"] if util else None,
                    avg_ms=round(kavg[dom], 4), alg_flops=per_kernel[dom][0],
                    alg_bytes=per_kernel[dom][1])
    # The whole step (forward + backward) against the same two limits.
    step_bytes = (2 * qb + kb + rb) + (4 * qb + 2 * kb + rb)
    step_roof = roof(fl_all, step_bytes, ms)
    step_roof.update(alg_flops=fl_all, alg_bytes=step_bytes)

    out = {
        "metric": "HCA attn fwd+bwd effective TFLOP/s",
        "value": round(fl_all / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_with_kernel_events": round(ms_instrumented, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "S": wl.S, "H": wl.H, "D": wl.D, "r": wl.r,
                   "W": wl.W, "S_c": wl.Sc,
                   "documents": 1 if lengths is None else sum(len(x) for x in lengths),
                   "comp_pattern": args.comp_pattern,
                   "topk": None if topk is None else int(topk.shape[2]),
                   "parallelism": "single GPU"},
        "tokens_per_s": round(wl.B * wl.S / (ms * 1e-3), 1),
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tflops": round(fl_fwd / (fwd_ms * 1e-3) / 1e12, 3),
        "fwd_tokens_per_s": round(wl.B * wl.S / (fwd_ms * 1e-3), 1),
        "visible_pairs": P,
        "plan_build_ms": round(plan_ms, 2),
        "comp_pattern": args.comp_pattern,
        "plan_device_bytes": info.device_bytes,
        "comp_mask_bytes": 0 if mask_dev is None else mask_dev.numel(),
        "peak_mem_gib": round(peak_mem, 3),
        "ws_bytes": max(info.ws_fwd_bytes, info.ws_bwd_bytes),
        "bwd_items": {"items": info.items, "half": info.items_half,
                      "partial_blocks": info.part_blocks,
                      "comp_item_chunks": info.comp_item_chunks, "kv_keys": info.kv_keys},
        "wall_s": round(wall, 3),
        "kernels_ms_per_step": {k: round(v, 4) for k, v in per_step.items()},
        "concurrent_kernels": sorted(concurrent & set(per_step)),
        "kernel_rooflines": {k: roof(*per_kernel[k], kavg[k]) for k in per_step
                             if k in per_kernel and k in kavg},
        "roofline": roofline,
        "step_roofline": step_roof,
        # rocprofv3 counters recorded for these kernel sources (separate runs).
        "counters": {k: dict(recorded_util(k, wl.name) or {},
                             hbm_bytes=recorded_traffic(k, wl.name))
                     for k in per_step if recorded_util(k, wl.name) or
                     recorded_traffic(k, wl.name)},
    }
    if not args.no_cpu_baseline and args.comp_pattern == "rule":
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

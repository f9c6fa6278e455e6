#!/usr/bin/env python3
"""Benchmark of the SLA hot path on one MI355X.

One step = one ``sla_forward`` plus one ``sla_backward`` (every stage of the
method: states, pooling, classification, aggregation, fused attention, and the
backward) on one batch of seeded synthetic input already resident in HBM.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--mode fwd|fwdbwd] [--no-cpu-baseline] [--no-side-runs]
                    [--traffic-probe]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "video_dit_b2_h12_n32768_d128"
DOMINANT = {"fwd": "attention", "fwdbwd": "bwd_kv"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", choices=("fwd", "fwdbwd"), default="fwdbwd")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side-runs", action="store_true",
                    help="skip the linear-branch and dense-baseline side measurements")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="after the timed region, run one device copy of 256 MiB (known bytes) "
                         "to calibrate hardware traffic counters")
    ap.add_argument("--dense", action="store_true",
                    help="time the same library as dense attention (all blocks critical)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t arrays created through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventQuery.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def array(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            self.hip.hipGetLastError()   # a stage the call did not run: clear the sticky error
            return None
        return out.value


def kernel_sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_linear_attention_mean_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, workload, digest):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, wl, k_c, k_n):
    """The oracle as it stands, on a bounded sample of the same workload:
    classification, states and forward of one full head, and the backward
    of one full head."""
    import oracle as orc

    scale = orc.default_scale(wl.head_dim)
    q = orc.decode_bf16(inp["q"][0, 0])
    k = orc.decode_bf16(inp["k"][0, 0])
    v = orc.decode_bf16(inp["v"][0, 0])
    w = orc.decode_bf16(inp["w"])
    t = wl.num_blocks
    t0 = time.perf_counter()
    scores = orc.compressed_scores(q, k, wl.valid_len, scale)
    mask = orc.classify(scores, k_c, k_n)
    blocks = list(range(t))
    orc.forward_head(q, k, v, w, mask, wl.valid_len, scale, blocks=blocks)
    t_fwd = time.perf_counter() - t0
    flops_fwd = 4.0 * 64 * 64 * wl.head_dim * k_c * len(blocks)
    # backward of the same head
    nq = wl.seq_len
    mq = mask
    do = orc.decode_bf16(inp["do"][0, 0]) if "do" in inp else np.ones((nq, wl.head_dim))
    t1 = time.perf_counter()
    orc.backward_head(q, k, v, w, do, mq, wl.valid_len, scale)
    t_bwd = time.perf_counter() - t1
    flops_bwd = 10.0 * 64 * 64 * wl.head_dim * k_c * t
    tflops = (flops_fwd + flops_bwd) / (t_fwd + t_bwd) / 1e12
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {
        "value": tflops,
        "unit": "TFLOP/s (critical-block FLOPs, fp64 oracle)",
        "cores": min(cores, threads),
        "kind": "oracle",
        "sample": (f"head (0,0) of {wl.batch * wl.heads}: scores, classification, states and "
                   f"forward of all {len(blocks)} query blocks ({t_fwd:.1f} s); backward of the "
                   f"same head ({t_bwd:.1f} s)"),
    }


def _timed(fn, warmup, steps):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def linear_branch_rate(wl, inp, q, k, v, w, dev):
    """Forward with no critical blocks (same negligible fraction): the linear
    branch alone.  Algorithmic bytes: K, V read, the per-block states h, z
    written and read once (bf16 as stored), Q read, O written."""
    import torch

    from sparse_linear_attention_mean_amd.attention import SlaProblem

    prob = SlaProblem.create(wl.batch, wl.heads, wl.seq_len, wl.head_dim, 0.0,
                             wl.frac_negligible, valid_len=wl.valid_len, device=dev)
    o = torch.empty(prob.shape(), dtype=torch.bfloat16, device=dev)
    mask = prob.new_mask()
    ms = _timed(lambda: prob.forward(q, k, v, w, o=o, mask=mask), 2, 5)
    bh, n, d, t = wl.batch * wl.heads, wl.seq_len, wl.head_dim, wl.num_blocks
    tok = 2 * bh * n * d                         # one bf16 [B,H,N,d] tensor
    states = bh * t * (d * d + 2 * d) * 2        # h (d x d) and z (two bf16 parts) per block
    nbytes = 2 * tok + 2 * states + tok + tok
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "note": "sla_forward with frac_critical = 0 and the same frac_negligible"}


def dense_ratio(wl, q, k, v, w, do, dev, with_bwd, sla_ms):
    """The same library and kernels with every block critical (frac_critical
    = 1, frac_negligible = 0): the dense attention baseline of the same shape."""
    import torch

    from sparse_linear_attention_mean_amd.attention import SlaProblem

    prob = SlaProblem.create(wl.batch, wl.heads, wl.seq_len, wl.head_dim, 1.0, 0.0,
                             valid_len=wl.valid_len, device=dev)
    o = torch.empty(prob.shape(), dtype=torch.bfloat16, device=dev)
    mask = prob.new_mask()
    grads = None
    if with_bwd:
        shp = prob.shape()
        grads = tuple(torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3)) + (
            torch.empty((wl.head_dim, wl.head_dim), dtype=torch.float32, device=dev),)

    def step():
        prob.forward(q, k, v, w, o=o, mask=mask)
        if with_bwd:
            prob.backward(q, k, v, w, o, do, mask, grads=grads)

    ms = _timed(step, 1, 2)
    return {"dense_ms_per_step": round(ms, 3), "sla_ms_per_step": round(sla_ms, 4),
            "speedup": round(ms / sla_ms, 2),
            "note": "frac_critical = 1, frac_negligible = 0 through the same entry points"}


def mask_reuse_rate(wl, q, k, v, w, dev, mask):
    """Forward with the mask of the timed run passed back in (given-mask mode:
    no pooling, scores or classification) against the computed-mask forward."""
    import torch

    from sparse_linear_attention_mean_amd import _binding as B
    from sparse_linear_attention_mean_amd.attention import SlaProblem

    out = {}
    for name, mode in (("fwd_ms_computed_mask", B.SLA_MASK_COMPUTE),
                       ("fwd_ms_given_mask", B.SLA_MASK_GIVEN)):
        prob = SlaProblem.create(wl.batch, wl.heads, wl.seq_len, wl.head_dim, wl.frac_critical,
                                 wl.frac_negligible, valid_len=wl.valid_len, mask_mode=mode,
                                 device=dev)
        o = torch.empty(prob.shape(), dtype=torch.bfloat16, device=dev)
        m = mask.clone() if mode == B.SLA_MASK_GIVEN else prob.new_mask()
        out[name] = round(_timed(lambda: prob.forward(q, k, v, w, o=o, mask=m), 2, 5), 4)
    return out


def global_linear_rate(wl, q, k, v, w, do, dev, with_bwd, gate=0.5):
    """The SALAD-style variant: linear branch over every key block (one state
    sum per head instead of the per-row marginal aggregation), gated output."""
    import torch

    from sparse_linear_attention_mean_amd import _binding as B
    from sparse_linear_attention_mean_amd.attention import SlaProblem

    prob = SlaProblem.create(wl.batch, wl.heads, wl.seq_len, wl.head_dim, wl.frac_critical,
                             wl.frac_negligible, valid_len=wl.valid_len, device=dev,
                             linear_mode=B.SLA_LINEAR_GLOBAL, linear_gate=gate)
    o = torch.empty(prob.shape(), dtype=torch.bfloat16, device=dev)
    mask = prob.new_mask()
    grads = None
    if with_bwd:
        shp = prob.shape()
        grads = tuple(torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3)) + (
            torch.empty((wl.head_dim, wl.head_dim), dtype=torch.float32, device=dev),)

    def step():
        prob.forward(q, k, v, w, o=o, mask=mask)
        if with_bwd:
            prob.backward(q, k, v, w, o, do, mask, grads=grads)

    return {"ms_per_step": round(_timed(step, 2, 5), 4), "gate": gate,
            "note": "linear_mode = SLA_LINEAR_GLOBAL, same fractions"}


def two_level_selection(dev, hip, group=8, keep=8, steps=5):
    """Flat against two-level key-block selection on the long-sequence workload
    (N = 65536, T = 1024): the selection stage (score map and classification,
    or group means and the two-level classifier) and the whole forward, from
    the library's stage events.  Also the share of critical blocks the two
    splits have in common."""
    import torch

    from sparse_linear_attention_mean_amd import _binding as B
    from sparse_linear_attention_mean_amd.attention import SlaProblem, bf16_from_bits
    from sparse_linear_attention_mean_amd.inputs import WORKLOADS, make_workload_inputs

    wl = WORKLOADS["pixel_b1_h8_n65536_d64"]
    inp = make_workload_inputs(wl.name, seed=0, with_grad=False)
    q, k, v, w = (bf16_from_bits(inp[x], dev) for x in ("q", "k", "v", "w"))
    out = {"workload": wl.name, "select_group": group, "select_keep": keep}
    masks = {}
    si = B.STAGES.index("classify")
    for label, g, kp in (("flat", 0, 0), ("two_level", group, keep)):
        prob = SlaProblem.create(wl.batch, wl.heads, wl.seq_len, wl.head_dim, wl.frac_critical,
                                 wl.frac_negligible, valid_len=wl.valid_len, device=dev,
                                 select_group=g, select_keep=kp)
        o = torch.empty(prob.shape(), dtype=torch.bfloat16, device=dev)
        mask = prob.new_mask()
        evs = [hip.array(2 * B.SLA_NUM_STAGES) for _ in range(steps)]
        prob.forward(q, k, v, w, o=o, mask=mask)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for ev in evs:
            prob.cfg.stage_events = ctypes.cast(ev, ctypes.c_void_p).value
            prob.forward(q, k, v, w, o=o, mask=mask)
        b.record()
        torch.cuda.synchronize()
        prob.cfg.stage_events = None
        sel = [hip.elapsed_ms(ev[2 * si], ev[2 * si + 1]) for ev in evs]
        sel = [x for x in sel if x is not None]
        out[label] = {"selection_ms": round(sum(sel) / len(sel), 4),
                      "fwd_ms": round(a.elapsed_time(b) / steps, 4)}
        masks[label] = mask
    crit_f, crit_h = masks["flat"] == 1, masks["two_level"] == 1
    out["critical_overlap"] = round(float((crit_f & crit_h).sum()) / max(1, int(crit_f.sum())), 4)
    out["selection_speedup"] = round(out["flat"]["selection_ms"] /
                                     out["two_level"]["selection_ms"], 2)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; it has no multi-GPU path, "
                                   "so --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from sparse_linear_attention_mean_amd import _binding as B
    from sparse_linear_attention_mean_amd.attention import SlaProblem, bf16_from_bits
    from sparse_linear_attention_mean_amd.inputs import WORKLOADS, make_workload_inputs

    wl = WORKLOADS[args.workload]
    fc, fn = (1.0, 0.0) if args.dense else (wl.frac_critical, wl.frac_negligible)
    with_bwd = args.mode == "fwdbwd"
    inp = make_workload_inputs(wl.name, seed=args.seed, with_grad=with_bwd)
    dev = torch.device("cuda:0")
    q, k, v, w = (bf16_from_bits(inp[x], dev) for x in ("q", "k", "v", "w"))
    do = bf16_from_bits(inp["do"], dev) if with_bwd else None
    prob = SlaProblem.create(wl.batch, wl.heads, wl.seq_len, wl.head_dim, fc, fn,
                             valid_len=wl.valid_len, device=dev)
    k_c, k_n, k_m = B.sla_block_counts(prob.cfg)
    o = torch.empty(prob.shape(), dtype=torch.bfloat16, device=dev)
    mask = prob.new_mask()
    shp = prob.shape()
    grads = None
    if with_bwd:
        grads = tuple(torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3)) + (
            torch.empty((wl.head_dim, wl.head_dim), dtype=torch.float32, device=dev),)

    hip = HipEvents()
    nstage = B.SLA_NUM_STAGES
    ev_sets = [hip.array(2 * nstage) for _ in range(args.steps)]
    warm_ev = hip.array(2 * nstage)

    def step(ev):
        prob.cfg.stage_events = ctypes.cast(ev, ctypes.c_void_p).value
        prob.forward(q, k, v, w, o=o, mask=mask)
        if with_bwd:
            prob.backward(q, k, v, w, o, do, mask, grads=grads)

    for _ in range(args.warmup):
        step(warm_ev)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.steps):
        step(ev_sets[s])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps

    stage_ms = {}
    for si, name in enumerate(B.STAGES):
        if not with_bwd and si >= 5:   # backward stages are not recorded in forward-only runs
            continue
        vals = [hip.elapsed_ms(ev_sets[s][2 * si], ev_sets[s][2 * si + 1]) for s in range(args.steps)]
        vals = [x for x in vals if x is not None]
        if vals:
            stage_ms[name] = sum(vals) / len(vals)

    bh = wl.batch * wl.heads
    t = wl.num_blocks
    d = wl.head_dim
    pairs = bh * t * k_c
    flops_fwd_crit = 4.0 * 64 * 64 * d * pairs
    flops_bwd_crit = 10.0 * 64 * 64 * d * pairs if with_bwd else 0.0
    flops = flops_fwd_crit + flops_bwd_crit
    dense_flops = (4.0 + (10.0 if with_bwd else 0.0)) * bh * wl.seq_len ** 2 * d
    value = flops / (ms * 1e-3) / 1e12

    # Rooflines of the two MFMA-bound kernels, each from its own stage events
    # (one launch per stage).  Algorithmic flops per launch:
    #   fused forward attention: 4 b^2 d per critical pair, plus the linear
    #     branch phi(Q) H_i and Y W^T (2 x 2 b d^2 per query block);
    #   key-block backward (dK, dV): its share of the 10 b^2 d per critical
    #     pair, S, dP, P^T dO and dS^T Q (8 b^2 d), plus the linear-branch
    #     terms phi(K) dh and V dh^T (2 x 2 b d^2 per key block).
    linear = k_m > 0
    lin_blk = (2 * 2.0 * 64 * d * d * bh * t) if linear else 0.0

    def roofline(stage, flops_k, label, tag, sources):
        kms = stage_ms.get(stage)
        ach = flops_k / (kms * 1e-3) / 1e12 if kms else None
        return {
            "kernel": label,
            "bound": "mfma",
            "achieved": round(ach, 2) if ach else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4) if ach else None,
            "traffic": traffic_from_profile(tag, wl.name, kernel_sources_digest(sources)),
        }

    rl_fwd = roofline("attention", flops_fwd_crit + lin_blk,
                      "attn_fwd_kernel (fused sparse + linear + projection)", "attn_fwd",
                      ["attn_fwd.hip", "sla_device.h"])
    rl_kv = roofline("bwd_kv", 8.0 * 64 * 64 * d * pairs + lin_blk,
                     "bwd_kv_kernel (key-block backward: dK, dV)", "bwd_kv",
                     ["bwd.hip", "sla_device.h"]) if with_bwd else None

    rec = {
        "metric": "SLA fwd/bwd effective TFLOPS + % bf16 MFMA peak at N=32768,H=12,d=128",
        "value": round(value, 2),
        "unit": "TFLOP/s (critical-block FLOPs)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded grid-structured Q/K, Gaussian V and dO)",
        "config": {
            "workload": wl.name,
            "batch": wl.batch, "heads": wl.heads, "seq_len": wl.seq_len,
            "valid_len": wl.valid_len, "head_dim": d, "block": 64,
            "frac_critical": fc, "frac_negligible": fn,
            "k_c": k_c, "k_n": k_n, "k_m": k_m, "mode": args.mode,
        },
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "tflops_dense_equivalent": round(dense_flops / (ms * 1e-3) / 1e12, 1),
        "stages_ms": {kk: round(vv, 4) for kk, vv in stage_ms.items()},
        "roofline": rl_kv if DOMINANT[args.mode] == "bwd_kv" else rl_fwd,
    }
    if DOMINANT[args.mode] == "bwd_kv":
        rec["roofline_attention_fwd"] = rl_fwd
    if with_bwd:
        fwd_ms = sum(stage_ms.get(s, 0.0) for s in B.STAGES[:5])
        bwd_ms = sum(stage_ms.get(s, 0.0) for s in B.STAGES[5:])
        if fwd_ms > 0:
            rec["fwd_tflops"] = round(flops_fwd_crit / (fwd_ms * 1e-3) / 1e12, 2)
        if bwd_ms > 0:
            rec["bwd_tflops"] = round(flops_bwd_crit / (bwd_ms * 1e-3) / 1e12, 2)
    if not args.no_side_runs and not args.dense:
        rec["linear_branch"] = linear_branch_rate(wl, inp, q, k, v, w, dev)
        rec["vs_dense"] = dense_ratio(wl, q, k, v, w, do, dev, with_bwd, ms)
        rec["mask_reuse"] = mask_reuse_rate(wl, q, k, v, w, dev, mask)
        rec["global_linear"] = global_linear_rate(wl, q, k, v, w, do, dev, with_bwd)
        rec["two_level_selection"] = two_level_selection(dev, hip)
    if args.traffic_probe:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)   # reads and writes 256 MiB each
        torch.cuda.synchronize()
        rec["traffic_probe_bytes"] = 2 * src.numel()
    if not args.no_cpu_baseline:
        sys.path.insert(0, ROOT)
        rec["cpu_baseline"] = cpu_baseline(inp, wl, k_c, k_n)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the SLA hot path on one MI355X.

One step = one ``sla_forward`` plus one ``sla_backward`` (every stage of the
method: states, pooling, classification, aggregation, fused attention, and the
backward) on one batch of seeded synthetic input already resident in HBM.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--mode fwd|fwdbwd] [--no-cpu-baseline] [--no-side-runs]
                    [--traffic-probe]
    python bench.py --trace-summary KERNEL_TRACE_CSV --warmup W --steps K
    python bench.py --counter-summary FETCH_CSV WRITE_CSV GRBM_CSV

`ms_per_step` / `value` come from the K timed steps bracketed by
synchronisations; `step_ms` gives median / min / p90 / mean per step and
`stages_ms` the median per stage.  The roofline of a kernel uses the median
of the HIP events around its stage's single launch; `clock` is the engine
clock while the step repeats (amdsmi), and the roofline also states the
fraction of the peak rescaled to it.  --trace-summary turns a rocprofv3
kernel trace of this script into per-kernel median / min / p90 with the
warm-up launches dropped; --counter-summary turns three rocprofv3 --pmc runs
into HBM bytes and engine clock per kernel and writes the traffic records
under profiles/.
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
PEAK_CLOCK_MHZ = 2400.0     # engine clock the published MFMA peak is quoted at
DEFAULT_WORKLOAD = "video_dit_b2_h12_n32768_d128"
DOMINANT = {"fwd": "attention", "fwdbwd": "bwd_kv"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
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
    ap.add_argument("--sq-summary", nargs=2, metavar=("PASS_A_CSV", "PASS_B_CSV"),
                    help="summarise two rocprofv3 --pmc runs of the SQ_PASSES counters")
    ap.add_argument("--pairs", type=int, default=319488,
                    help="critical pairs per launch for --sq-summary (default: the bench workload)")
    ap.add_argument("--counter-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "GRBM_CSV"),
                    help="summarise three rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, "
                         "GRBM_COUNT GRBM_GUI_ACTIVE) and write the traffic records under profiles/")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="no GPU run: summarise a rocprofv3 kernel trace of a run of this script "
                         "(--warmup / --steps as in that run): per kernel, the launches of the "
                         "timed steps only (warm-up launches dropped), median / min / p90 / mean")
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
    cpu0 = time.process_time()
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
    cpu_s = time.process_time() - cpu0
    wall_s = t_fwd + t_bwd
    tflops = (flops_fwd + flops_bwd) / wall_s / 1e12
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": tflops,
        "unit": "TFLOP/s (critical-block FLOPs, fp64 oracle)",
        # threads actually busy: process CPU time over wall time of the sample
        "cores": round(cpu_s / wall_s, 1),
        "cores_available": cores,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": (f"head (0,0) of {wl.batch * wl.heads}: scores, classification, states and "
                   f"forward of all {len(blocks)} query blocks ({t_fwd:.1f} s); backward of the "
                   f"same head ({t_bwd:.1f} s)"),
        "one_thread": _oracle_one_thread(wl, k_c, k_n),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


_ONE_THREAD_SNIPPET = """
import sys, time, json
sys.path.insert(0, {root!r})
import oracle as orc
from sparse_linear_attention_mean_amd.inputs import make_workload_inputs
wl_name, k_c, k_n, nblk = {name!r}, {k_c}, {k_n}, {nblk}
from sparse_linear_attention_mean_amd.inputs import WORKLOADS
wl = WORKLOADS[wl_name]
inp = make_workload_inputs(wl_name, seed=0, with_grad=False)
scale = orc.default_scale(wl.head_dim)
q, k, v = (orc.decode_bf16(inp[x][0, 0]) for x in ("q", "k", "v"))
w = orc.decode_bf16(inp["w"])
t0 = time.perf_counter()
mask = orc.classify(orc.compressed_scores(q, k, wl.valid_len, scale), k_c, k_n)
orc.forward_head(q, k, v, w, mask, wl.valid_len, scale, blocks=list(range(nblk)))
print(json.dumps({{"s": time.perf_counter() - t0}}))
"""


def _oracle_one_thread(wl, k_c, k_n, nblk=64):
    """The oracle forward of the first nblk query blocks of head (0, 0) (plus
    the scores and classification of the head) in a child process whose BLAS
    and OpenMP pools are limited to one thread."""
    import subprocess

    env = dict(os.environ)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        env[var] = "1"
    code = _ONE_THREAD_SNIPPET.format(root=ROOT, name=wl.name, k_c=k_c, k_n=k_n, nblk=nblk)
    try:
        res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                             timeout=600)
        sec = json.loads(res.stdout.strip().splitlines()[-1])["s"]
    except Exception as exc:   # reported, not fatal: the baseline is context
        return {"error": str(exc)[:200]}
    flops = 4.0 * 64 * 64 * wl.head_dim * k_c * nblk
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s (critical-block FLOPs, fp64 oracle)",
            "cores": 1, "seconds": round(sec, 2),
            "sample": f"scores and classification of head (0,0), forward of its first {nblk} "
                      f"query blocks, one thread"}


def _timed(fn, warmup, steps, per_step=False):
    """Mean ms per call over `steps` calls after `warmup` (one event pair
    around all of them); with per_step, also the list of per-call times from
    an event at every call boundary."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    mean = evs[0].elapsed_time(evs[-1]) / steps
    if per_step:
        return mean, [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return mean


def sustained_clock(step, max_s=4.0, sync=None):
    """GFX (shader) clock while ``step`` runs back to back.

    amdsmi's GPU metrics table holds per-XCD clocks averaged over a window and
    is refreshed about once a second (its ``system_clock_counter`` moves on at
    each refresh), far longer than the timed steps.  So the step is repeated,
    untimed, until two refreshes whose whole window lies inside the repeated
    run have been read (the first refresh after the start also covers the idle
    time before it).  None where amdsmi is unavailable.  ``sync`` waits for
    the queued steps (torch.cuda.synchronize by default)."""
    if sync is None:
        import torch

        sync = torch.cuda.synchronize
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as exc:
        return {"gfx_mhz": None, "error": str(exc)[:200]}

    def read():
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        clks = m.get("current_gfxclks")
        vals = [float(c) for c in clks if isinstance(c, (int, float)) and 0 < c < 0xFFFF] \
            if isinstance(clks, (list, tuple)) else []
        return m.get("system_clock_counter"), vals, m.get("current_socket_power")

    try:
        prev, _, _ = read()
        refreshes, windows = 0, []
        t0 = time.time()
        while time.time() - t0 < max_s and len(windows) < 2:
            for _ in range(10):
                step()
            sync()
            cnt, vals, power = read()
            if cnt != prev:
                refreshes += 1
                prev = cnt
                if refreshes >= 2 and vals:
                    windows.append((vals, power))
    except Exception as exc:
        return {"gfx_mhz": None, "error": str(exc)[:200]}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
    if not windows:
        return {"gfx_mhz": None, "error": "no metrics refresh inside the repeated run"}
    means = [sum(v) / len(v) for v, _ in windows]
    return {
        "gfx_mhz": round(sum(means) / len(means), 1),
        "gfx_mhz_per_xcd": windows[-1][0],
        "socket_power_w": windows[-1][1],
        "windows": len(windows),
        "source": "amdsmi GPU metrics, current GFX clock averaged over the XCDs, from "
                  "about-1-s refresh windows lying wholly inside an untimed run of the "
                  "same step back to back after the timed steps",
    }


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
    # the same accounting with fp32 states (h d x d, z d per block)
    nbytes32 = 2 * tok + 2 * (bh * t * (d * d + d) * 4) + tok + tok
    return {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "bytes_fp32_states": nbytes32,
            "GB/s_fp32_states": round(nbytes32 / (ms * 1e-3) / 1e9, 1),
            "note": "sla_forward with frac_critical = 0 and the same frac_negligible; states "
                    "are stored in bf16, the fp32 figure counts them as fp32"}


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

    mean, per = _timed(step, 2, 5, per_step=True)
    st = step_stats(per)
    t = wl.num_blocks
    bh = wl.batch * wl.heads
    dense_flops = (4.0 + (10.0 if with_bwd else 0.0)) * 64 * 64 * wl.head_dim * bh * t * t
    tf = dense_flops / (st["median"] * 1e-3) / 1e12
    return {"dense_ms_per_step": st["median"], "dense_step_ms": st, "sla_ms_per_step": round(sla_ms, 4),
            "speedup": round(st["median"] / sla_ms, 2),
            "dense_tflops": round(tf, 1), "dense_frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "note": "frac_critical = 1, frac_negligible = 0 through the same entry points; "
                    "median of 5 steps after 2 warm-up steps; speedup = dense median / SLA "
                    "median step time"}


def sdpa_ratio(wl, q, k, v, do, dev, with_bwd, sla_ms):
    """A dense baseline from outside this library: PyTorch's fused
    scaled-dot-product attention (flash backend, else memory-efficient; never
    the unfused math path) on the same bf16 Q, K, V, forward and, with the
    backward, the gradients of Q, K, V for the same output gradient.  Plain
    softmax attention only (no linear branch, no projection)."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    qq, kk, vv = (x.detach().clone().requires_grad_(with_bwd) for x in (q, k, v))
    scale = wl.head_dim ** -0.5
    err = {}
    for name, backend in (("flash", SDPBackend.FLASH_ATTENTION),
                          ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        def step():
            with sdpa_kernel([backend]):
                out = F.scaled_dot_product_attention(qq, kk, vv, scale=scale)
            if with_bwd:
                qq.grad = kk.grad = vv.grad = None
                out.backward(do)

        try:
            _, per = _timed(step, 2, 5, per_step=True)
        except Exception as e:   # backend not available for this device or shape
            err[name] = str(e).splitlines()[0][:160]
            continue
        st = step_stats(per)
        bh, n = wl.batch * wl.heads, wl.seq_len
        flops = (4.0 + (10.0 if with_bwd else 0.0)) * bh * n * n * wl.head_dim
        tf = flops / (st["median"] * 1e-3) / 1e12
        return {"backend": name, "sdpa_ms_per_step": st["median"], "sdpa_step_ms": st,
                "sla_ms_per_step": round(sla_ms, 4), "speedup": round(st["median"] / sla_ms, 2),
                "sdpa_tflops": round(tf, 1), "sdpa_frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                "skipped_backends": err,
                "note": "torch.nn.functional.scaled_dot_product_attention at the same shape, "
                        "median of 5 steps after 2 warm-up steps; speedup = SDPA median / SLA "
                        "median step time"}
    return {"unavailable": err}


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


def _percentile(sorted_vals, q):
    """Nearest-rank percentile of an ascending list."""
    if not sorted_vals:
        return None
    k = max(0, min(len(sorted_vals) - 1, math.ceil(q / 100.0 * len(sorted_vals)) - 1))
    return sorted_vals[k]


def step_stats(ms_list):
    """median / min / p90 / mean of per-step (or per-launch) times, ms."""
    v = sorted(x for x in ms_list if x is not None)
    if not v:
        return None
    return {"median": round(_percentile(v, 50), 4), "min": round(v[0], 4),
            "p90": round(_percentile(v, 90), 4), "mean": round(sum(v) / len(v), 4), "n": len(v)}


def trace_summary(path, warmup, steps):
    """Per-kernel launch durations of a rocprofv3 --kernel-trace CSV of one run
    of this script.  Every kernel of the hot path is launched the same number
    of times per step, in step order, so the first warmup / (warmup + steps)
    of each kernel's launches are the warm-up steps and are dropped."""
    import csv

    by_name = {}
    with open(path, newline="") as f:
        for rec in csv.DictReader(f):
            name = rec.get("Kernel_Name") or rec.get("KernelName") or rec.get("Name")
            t0 = int(rec.get("Start_Timestamp") or rec.get("BeginNs"))
            t1 = int(rec.get("End_Timestamp") or rec.get("EndNs"))
            by_name.setdefault(name, []).append((t0, (t1 - t0) / 1000.0))
    rows = []
    for name, launches in by_name.items():
        launches.sort()
        total = len(launches)
        per_step = total / float(warmup + steps)
        skip = int(round(warmup * per_step)) if per_step.is_integer() else 0
        us = sorted(d for _, d in launches[skip:])
        rows.append((sum(us), name, total, len(us), _percentile(us, 50), us[0],
                     _percentile(us, 90), sum(us) / len(us)))
    rows.sort(reverse=True)
    busy = sum(r[0] for r in rows)
    out = ["| kernel | launches | timed | median µs | min µs | p90 µs | mean µs | % of timed GPU time |",
           "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for tot, name, total, n, med, mn, p90, mean in rows:
        out.append(f"| `{name}` | {total} | {n} | {med:.1f} | {mn:.1f} | {p90:.1f} | {mean:.1f} | "
                   f"{100.0 * tot / busy:.1f} |")
    out.append("")
    out.append(f"Kernel time over the timed steps: {busy / 1000.0 / steps:.3f} ms per step "
               f"({steps} steps, {warmup} warm-up steps dropped).")
    return "\n".join(out)


# kernels whose roofline reports traffic: tag -> (kernel name stem, sources)
TRAFFIC_KERNELS = {
    "attn_fwd": ("attn_fwd_kernel", ["attn_fwd.hip", "sla_device.h"]),
    "bwd_kv": ("bwd_kv_kernel", ["bwd.hip", "sla_device.h"]),
}
COUNTER_COMMAND = ("rocprofv3 --pmc {c} --output-format csv -d OUT/{t} -o {t} -- "
                   "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-side-runs "
                   "--traffic-probe")


def _counter_rows(path):
    """(dispatch id, kernel name, value) of a rocprofv3 --pmc CSV with one counter."""
    import csv

    out = []
    with open(path, newline="") as f:
        for rec in csv.DictReader(f):
            out.append((int(rec["Dispatch_Id"]), rec["Kernel_Name"], float(rec["Counter_Value"]),
                        int(rec["End_Timestamp"]) - int(rec["Start_Timestamp"])))
    out.sort()
    return out


def counter_summary(fetch_csv, write_csv, grbm_csv, workload, xcc=8, write_json=True):
    """HBM traffic and engine clock per kernel from three rocprofv3 --pmc runs
    of ``bench.py --steps 1 --warmup 1 --traffic-probe`` (FETCH_SIZE;
    WRITE_SIZE; GRBM_COUNT with GRBM_GUI_ACTIVE).

    The run ends with one device copy of 256 MiB (the last dispatch); what the
    counters read for it against the bytes it moves gives the scale factor of
    each counter.  GRBM_COUNT counts engine clocks summed over the ``xcc``
    XCDs; per XCD over the dispatch's duration it gives the clock (biased high
    for short kernels, whose counting window is longer than the kernel).
    Writes profiles/traffic_<tag>_<workload>.json for the kernels in
    TRAFFIC_KERNELS, stamped with the digest of their current sources, and
    returns the markdown table."""
    fetch, write = _counter_rows(fetch_csv), _counter_rows(write_csv)
    grbm = _counter_rows(grbm_csv) if grbm_csv else []
    probe_bytes = 256 << 20
    f_probe, w_probe = fetch[-1], write[-1]
    f_fac = f_probe[2] * 1024.0 / probe_bytes
    w_fac = w_probe[2] * 1024.0 / probe_bytes

    def per_kernel(rows):
        d = {}
        for _, name, val, dur in rows[:-1]:
            if "sla::" in name:          # the library's kernels, not the probe's fill
                d.setdefault(name, []).append((val, dur))
        return d

    fk, wk = per_kernel(fetch), per_kernel(write)
    gk = {}
    for _, name, val, dur in grbm:
        gk.setdefault(name, []).append((val, dur))
    lines = [
        f"Calibration: the copy at the end of each run moves 262144 KiB each way; FETCH_SIZE reads "
        f"{f_probe[2]:.0f} KiB for it (factor {f_fac:.4f}), WRITE_SIZE {w_probe[2]:.0f} KiB "
        f"(factor {w_fac:.4f}).  Bytes below are counter / factor, mean per launch.",
        "",
        "| kernel | launches | read MB | written MB | engine cycles per XCD (M) | duration under counters µs | implied clock MHz |",
        "|---|---:|---:|---:|---:|---:|---:|",
    ]
    summary = {}
    for name, vals in fk.items():
        n = len(vals)
        rd = sum(v for v, _ in vals) / n * 1024.0 / f_fac
        wr = sum(v for v, _ in wk.get(name, [(0.0, 0)])) / max(1, len(wk.get(name, []))) * 1024.0 / w_fac
        g = [x for x in gk.get(name, []) if x[1] > 0]
        # GRBM_COUNT and GRBM_GUI_ACTIVE rows alternate per dispatch: keep one
        # value per dispatch (they agree for a kernel that keeps the GPU busy)
        g = g[::2] if len(g) == 2 * n else g
        cyc = sum(v for v, _ in g) / len(g) / xcc if g else None
        dur = sum(du for _, du in g) / len(g) / 1000.0 if g else None
        mhz = cyc / dur if cyc and dur else None
        stem = name.replace("void ", "").split("(")[0]
        summary[stem] = {"read_bytes": rd, "written_bytes": wr, "cycles_per_xcd": cyc,
                         "duration_us": dur, "mhz": mhz, "launches": n,
                         "fetch_kib": sum(v for v, _ in vals) / n,
                         "write_kib": sum(v for v, _ in wk.get(name, [(0.0, 0)])) / max(1, len(wk.get(name, [])))}
        show_clk = mhz is not None and dur >= 100.0
        lines.append(f"| `{stem}` | {n} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{(cyc / 1e6) if cyc else float('nan'):.3f} | {dur if dur else float('nan'):.1f} | "
                     f"{(f'{mhz:.0f}' if show_clk else '(short)')} |")
    if write_json:
        for tag, (kname, sources) in TRAFFIC_KERNELS.items():
            hit = [v for k, v in summary.items() if kname in k]
            if not hit:
                continue
            r = hit[0]
            rec = {
                "kernel": kname, "workload": workload,
                "source_digest": kernel_sources_digest(sources), "sources": sources,
                "fetch_kib_per_launch": round(r["fetch_kib"], 1),
                "write_kib_per_launch": round(r["write_kib"], 1),
                "copy_probe": {"bytes_read": probe_bytes, "bytes_written": probe_bytes,
                               "fetch_kib": f_probe[2], "write_kib": w_probe[2]},
                "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
                "hbm_bytes_per_launch": int(round(r["read_bytes"] + r["written_bytes"])),
                "engine_cycles_per_xcd": round(r["cycles_per_xcd"]) if r["cycles_per_xcd"] else None,
                "clock_mhz_under_counters": round(r["mhz"], 1) if r["mhz"] else None,
                "commands": [COUNTER_COMMAND.format(c=c, t=c.replace(" ", "_"))
                             for c in ("FETCH_SIZE", "WRITE_SIZE", "GRBM_COUNT GRBM_GUI_ACTIVE")],
            }
            with open(os.path.join(ROOT, "profiles", f"traffic_{tag}_{workload}.json"), "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
    return "\n".join(lines)


SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_ACTIVE_INST_ANY "
    "SQ_INSTS_SALU SQ_ACTIVE_INST_MISC SQ_INSTS_VMEM",
)


def sq_summary(csv_a, csv_b, pairs, simds=1024, engines=32):
    """Per kernel, from two rocprofv3 --pmc runs with the SQ_PASSES counters:
    the matrix-core busy fraction per SIMD (SQ_VALU_MFMA_BUSY_CYCLES over
    ``simds`` SIMDs x the kernel's cycles, the cycles being SQ_BUSY_CYCLES per
    shader engine, ``engines`` of them), the share of wave time spent waiting
    at s_waitcnt (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES), and the instructions per
    critical pair (``pairs`` per launch) issued by all waves."""
    import csv

    data = {}
    for path in (csv_a, csv_b):
        with open(path, newline="") as f:
            for rec in csv.DictReader(f):
                name = rec["Kernel_Name"].replace("void ", "").split("(")[0]
                d = data.setdefault(name, {})
                d.setdefault(rec["Counter_Name"], []).append(float(rec["Counter_Value"]))
                if rec["Counter_Name"] == "SQ_BUSY_CYCLES":
                    d.setdefault("_us", []).append(
                        (int(rec["End_Timestamp"]) - int(rec["Start_Timestamp"])) / 1000.0)

    def mean(d, c):
        v = d.get(c)
        return sum(v) / len(v) if v else float("nan")

    lines = ["| kernel | µs under counters | clock MHz | MFMA busy % | waiting at s_waitcnt % | "
             "MFMA / VALU / LDS / VMEM / SALU instructions per critical pair |",
             "|---|---:|---:|---:|---:|---|"]
    for name, d in data.items():
        if not name.startswith("sla::"):
            continue
        cyc = mean(d, "SQ_BUSY_CYCLES") / engines
        us = mean(d, "_us")
        mfma = mean(d, "SQ_VALU_MFMA_BUSY_CYCLES") / (simds * cyc)
        wait = mean(d, "SQ_WAIT_INST_ANY") / mean(d, "SQ_WAVE_CYCLES")
        mix = " / ".join(f"{mean(d, 'SQ_INSTS_' + k) / pairs:.0f}"
                         for k in ("MFMA", "VALU", "LDS", "VMEM", "SALU"))
        lines.append(f"| `{name}` | {us:.1f} | {cyc / us:.0f} | {100 * mfma:.1f} | {100 * wait:.1f} | {mix} |")
    return "\n".join(lines)


def main():
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.warmup, args.steps))
        return
    if args.sq_summary:
        print(sq_summary(*args.sq_summary, pairs=args.pairs))
        return
    if args.counter_summary:
        print(counter_summary(*args.counter_summary, workload=args.workload))
        return
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
    # timed region: one event at every step boundary (the library runs on
    # torch's current stream), the whole region bracketed by synchronisations
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    bounds[0].record()
    for s in range(args.steps):
        step(ev_sets[s])
        bounds[s + 1].record()
    torch.cuda.synchronize()
    ms = bounds[0].elapsed_time(bounds[-1]) / args.steps
    step_ms = step_stats([bounds[s].elapsed_time(bounds[s + 1]) for s in range(args.steps)])

    # per stage: the median over the timed steps (each stage's events bracket
    # its launches on the stream); min / p90 / mean alongside
    stage_ms, stage_stats = {}, {}
    for si, name in enumerate(B.STAGES):
        if not with_bwd and si >= 5:   # backward stages are not recorded in forward-only runs
            continue
        vals = [hip.elapsed_ms(ev_sets[s][2 * si], ev_sets[s][2 * si + 1]) for s in range(args.steps)]
        st = step_stats(vals)
        if st:
            stage_ms[name] = st["median"]
            stage_stats[name] = st

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
            "frac_of_peak_at_measured_clock": (round(ach / (PEAK_BF16_TFLOPS * mhz / PEAK_CLOCK_MHZ), 4)
                                               if ach and mhz else None),
            "flop_per_launch": flops_k,
            "launch_ms": round(kms, 4) if kms else None,
            "time_basis": "median over the timed steps of the HIP events around the stage's "
                          "single launch (the kernel's median duration in a rocprofv3 kernel "
                          "trace of the same command is the check)",
        }

    # shader clock under this load: the published peaks assume 2.4 GHz
    clock = (sustained_clock(lambda: step(warm_ev)) if not args.no_side_runs
             else {"gfx_mhz": None, "skipped": "--no-side-runs"})
    mhz = clock.get("gfx_mhz")

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
        "step_ms": step_ms,
        "stages_ms": {kk: round(vv, 4) for kk, vv in stage_ms.items()},
        "stages_ms_stats": stage_stats,
        "clock": clock,
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
        rec["vs_dense"] = dense_ratio(wl, q, k, v, w, do, dev, with_bwd, step_ms["median"])
        rec["vs_torch_sdpa"] = sdpa_ratio(wl, q, k, v, do, dev, with_bwd, step_ms["median"])
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

#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE hot path on one MI355X.

Headline (one JSON line on stdout): GMM fwd+bwd TFLOP/s on one expert-parallel
rank's share -- E=32 local experts, hidden 4096, intermediate 1536, 16384
received rows with Zipf(1.2) group sizes and 3 empty experts.  One step is
one pass of the whole hot path:

    moe_permute (top_k=1 local re-routing, histogram)
    -> gmm_fwd_swiglu(W1; writes A and, for the backward, H) -> gmm_fwd(W2)
    -> moe_unpermute
    -> gmm_bwd_swiglu(W2: dW2, and dH = SwiGLU backward of dA, in one launch)
    -> gmm_bwd(W1: dX and dW1 in one launch)

``value`` = algorithmic GEMM FLOPs of the step (real rows only, 6 GEMMs)
divided by the wall time of the whole step, inputs resident in HBM.

Also in the line:
  roofline     -- the dominant kernel (largest share of step time), its
                  algorithmic FLOPs per launch over its mean launch time
                  from HIP events recorded on the launch stream;
  decode       -- the decode-shaped layer forward (T=64, top-8, E=256,
                  hidden 2048, intermediate 512) in HBM GB/s;
  prefill      -- the prefill-shaped layer forward (T=4096, top-8, E=128,
                  hidden 2048, intermediate 512) as a fraction of its
                  attainable roofline max(FLOPs / MFMA peak, bytes / HBM peak),
                  and the backward of the two ends (moe_unpermute_bwd,
                  moe_permute_bwd) on its buffers in HBM GB/s;
  mxfp8        -- the A8W8-FP (MXFP8) forward on the decode and prefill layers
                  and the ep rank: GB/s, TFLOP/s against the fp8 MFMA peak,
                  fraction of the attainable roofline;
  *_ms_events  -- p10 / p50 / p90 of per-step (per-layer) device time from one
                  HIP event pair around each whole step (layer), in a pass of
                  its own; per_call_us comes from another pass with an event
                  pair around every call, and ms_per_step / ms_per_layer from
                  wall time with events around the dominant kernel's launches
                  only (its roofline) or none;
  ceilings     -- hipBLASLt on a dense bf16 product of the ep gate_up shape and
                  a 512 MiB device copy, measured here for context;
  cpu_baseline -- the CPU oracle timed on a bounded sample of the same step.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--prefill-steps", type=int, default=50)
    p.add_argument("--cpu-budget", type=float, default=12.0,
                   help="seconds of oracle work for the CPU baseline (0 = skip)")
    p.add_argument("--skip-decode", action="store_true", help="skip the decode and prefill layer legs")
    p.add_argument("--skip-mx", action="store_true", help="skip the MXFP8 (A8W8-FP) legs")
    p.add_argument("--copy-calibration", action="store_true",
                   help="finish with three 512 MiB device copies (the reference kernel that scales "
                        "the FETCH_SIZE / WRITE_SIZE counters into bytes)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class KernelTimer:
    """Records a pair of HIP events (torch.cuda.Event on the current stream --
    the stream every libmoegmm call is enqueued on) around each call."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []

    def __call__(self, name, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        self.pending.append((name, ev0, ev1))

    def collect(self):
        out = {}
        for name, a, b in self.pending:
            out.setdefault(name, []).append(a.elapsed_time(b))
        self.pending = []
        return out


def step_spans(torch, step, n):
    """ms per step from one HIP event pair around each whole step (no event
    between its calls), over n steps enqueued back to back."""
    ev = []
    for _ in range(n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def percentiles(ms):
    """p10 / p50 / p90 of per-step times in ms."""
    q = np.percentile(np.asarray(ms), [10, 50, 90])
    return dict(p10=round(float(q[0]), 4), p50=round(float(q[1]), 4), p90=round(float(q[2]), 4))


ROOT = os.path.dirname(os.path.abspath(__file__))
def traffic_profile(kernel):
    """The committed HBM-counter summary of `kernel` on the ep step."""
    stem = re.sub(r"[^A-Za-z0-9_]+", "_", kernel).strip("_")
    return os.path.join(ROOT, "profiles", f"{stem}_hbm_traffic_ep_rank.md")


KERNEL_SOURCES = ["grouped_gemm_moe_amd/csrc/gmm.hip", "grouped_gemm_moe_amd/csrc/gmm_engine.h",
                  "grouped_gemm_moe_amd/csrc/common.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if it is missing or was taken on different kernel source."""
    try:
        text = open(traffic_profile(kernel)).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^- (\w+): `([^`]+)`", text, flags=re.M))
    if vals.get("kernel") != kernel or vals.get("source_sha256") != kernel_source_hash():
        return None
    return float(vals["hbm_bytes_per_launch"])


def bf16_dev(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


# ---------------------------------------------------------------------------
# expert-parallel rank share: fwd + bwd
# ---------------------------------------------------------------------------

def ep_gemm_flops(gl, H, I):
    R = int(np.sum(gl))
    fwd1 = 2.0 * R * H * 2 * I
    fwd2 = 2.0 * R * I * H
    # each backward call computes the input and the weight gradient
    return {"gmm_fwd_swiglu": fwd1, "gmm_fwd_down": fwd2,
            "gmm_bwd_swiglu_down": 2 * fwd2, "gmm_bwd_gate_up": 2 * fwd1}


def ep_gemm_bytes(gl, H, I):
    """Algorithmic HBM bytes per call of the step's GEMMs: every operand read
    once (weights only of experts with rows), every output written once (the
    weight gradients of empty experts too: they are written as zeros)."""
    R = int(np.sum(gl))
    E = len(gl)
    act = int(np.sum(np.asarray(gl) > 0))
    w1, w2 = H * 2 * I * 2, I * H * 2
    x, h, a, yp = R * H * 2, R * 2 * I * 2, R * I * 2, R * H * 2
    return {
        "gmm_fwd_swiglu": dict(read=x + act * w1, write=h + a),
        "gmm_fwd_down": dict(read=a + act * w2, write=yp),
        # dW2 = A^T dYp and dH = swiglu_bwd(dYp W2^T, H)
        "gmm_bwd_swiglu_down": dict(read=a + yp + h + act * w2, write=E * w2 + h),
        # dX = dH W1^T and dW1 = X^T dH
        "gmm_bwd_gate_up": dict(read=x + h + act * w1, write=x + E * w1),
    }


# libmoegmm kernel behind each call of the step (kernel symbol -> calls)
EP_KERNELS = {
    "gmm_rows_kernel<2, false>": ["gmm_fwd_swiglu"],
    "gmm_rows_kernel<0, false>": ["gmm_fwd_down"],
    "gmm_bwd_kernel<true>": ["gmm_bwd_swiglu_down"],
    "gmm_bwd_kernel<false>": ["gmm_bwd_gate_up"],
}


def run_ep(torch, dev, args):
    import workloads
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer

    t0 = time.time()
    wl = workloads.ep_slice()
    log(f"ep inputs generated in {time.time() - t0:.1f}s; group_list={wl['group_list'].tolist()}")
    d = wl.dims
    H, I, E, R = d["H"], d["I"], d["E"], d["R"]
    x = bf16_dev(torch, wl["x"], dev)
    dyp = bf16_dev(torch, wl["dyp"], dev)
    w1 = bf16_dev(torch, wl["w1"], dev)
    w2 = bf16_dev(torch, wl["w2"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    layer = MoeLayer(LayerShape(R, 1, E, H, I), dev, with_backward=True)
    timer = KernelTimer(torch)
    g = layer.tokens_per_expert

    # the step's calls, shared with the GPU test of the same composition
    calls = layer.training_step_calls(x, ids, probs, dyp, w1, w2)

    def step(t):
        for name, fn in calls:
            t(name, fn)

    plain = lambda name, fn: fn()  # noqa: E731
    for _ in range(args.warmup):
        step(plain)
    torch.cuda.synchronize()
    # 1. an instrumented pass (an event pair around every call): the per-call
    #    breakdown and which kernel dominates
    timer.collect()
    for _ in range(args.steps):
        step(timer)
    torch.cuda.synchronize()
    per = timer.collect()
    # per-step spans from one event pair around each whole step
    step_ms = step_spans(torch, lambda: step(plain), args.steps)
    flops = ep_gemm_flops(wl["group_list"], H, I)
    total_flops = sum(flops.values())
    mean_ms = {k: float(np.mean(v)) for k, v in per.items()}
    gmm_ms = sum(mean_ms[k] for k in flops)
    kern_ms = {k: sum(mean_ms[c] for c in calls) for k, calls in EP_KERNELS.items()}
    dom = max(kern_ms, key=kern_ms.get)
    dom_calls = EP_KERNELS[dom]
    # 2. the timed region: K steps, events only around the dominant kernel's
    #    launches (its roofline), wall time for the whole step
    only_dom = lambda name, fn: timer(name, fn) if name in dom_calls else fn()  # noqa: E731
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(only_dom)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    dom_per = timer.collect()
    assert int(layer.dev_err.item()) == 0, "device error word set during the bench"
    ms_per_step = wall * 1e3 / args.steps
    dom_flops_per_launch = sum(flops[c] for c in dom_calls) / len(dom_calls)
    dom_ms_per_launch = float(np.mean([v for c in dom_calls for v in dom_per[c]]))
    achieved = dom_flops_per_launch / (dom_ms_per_launch * 1e-3) / 1e12
    traffic = measured_traffic(dom)
    alg = ep_gemm_bytes(wl["group_list"], H, I)
    dom_alg_read = sum(alg[c]["read"] for c in dom_calls) / len(dom_calls)
    dom_alg = dom_alg_read + sum(alg[c]["write"] for c in dom_calls) / len(dom_calls)
    # the same step with the memory-optimised backward (A recomputed from H,
    # gradients written over the forward's dead buffers)
    lm = MoeLayer(LayerShape(R, 1, E, H, I), dev, with_backward=True, low_memory=True)

    def step_lm():
        lm.forward(x, ids, probs, w1, w2, fused=True, keep_h=True)
        lm.backward(dyp, w1, w2)

    for _ in range(3):
        step_lm()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_lm()
    torch.cuda.synchronize()
    lm_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    assert int(lm.dev_err.item()) == 0
    saved = R * (I + 2 * I + H) * 2  # the dA, dH and dX buffers it does without
    del lm
    t_mfma_ms = total_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3  # the step is MFMA-bound
    res = dict(
        ms_per_step=ms_per_step,
        step_ms_events=percentiles(step_ms),
        frac_of_attainable=round(t_mfma_ms / ms_per_step, 4),
        value=total_flops / (ms_per_step * 1e-3) / 1e12,
        gmm_only_tflops=total_flops / (gmm_ms * 1e-3) / 1e12,
        gemm_gflop_per_step=total_flops / 1e9,
        per_call_us={k: round(v * 1e3, 2) for k, v in mean_ms.items()},
        low_memory_backward=dict(ms_per_step=round(lm_ms, 4),
                                 tflops=round(total_flops / (lm_ms * 1e-3) / 1e12, 2),
                                 bytes_saved=saved,
                                 note="A recomputed from H in the backward; dA, dH, dX written over "
                                      "the dead A, H, X_perm buffers; wall time, no events"),
        roofline=dict(bound="mfma", kernel=dom, achieved=round(achieved, 2),
                      peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), traffic=traffic,
                      traffic_unit="bytes per launch (HBM read + write)",
                      algorithmic_bytes=dom_alg, algorithmic_read_bytes=dom_alg_read,
                      traffic_over_algorithmic=round(traffic / dom_alg, 3) if traffic else None,
                      flops_per_launch=dom_flops_per_launch,
                      mean_launch_us=round(dom_ms_per_launch * 1e3, 2)),
    )
    return res, wl


# ---------------------------------------------------------------------------
# decode-shaped layer forward: HBM GB/s
# ---------------------------------------------------------------------------

def decode_bytes(gl, T, K, H, I, fused=True, gathered=False):
    """Algorithmic bytes of one layer forward: weights of experts with rows,
    once; every activation tensor the path materialises written once and read
    once (x_perm unless the gate_up GMM gathers token rows itself, Yp; A
    when the gate_up GMM is fused with SwiGLU; H when it is not, and then A
    written only, by swiglu_gmm_fwd, whose streaming kernel reads H); out
    written; indices."""
    n_active = int(np.sum(np.asarray(gl) > 0))
    S = int(np.sum(gl))
    w = n_active * (H * 2 * I + I * H) * 2
    act = (T * H * 2            # x read (by the permute's gather, or by the gate_up GMM)
           + (0 if gathered else S * H * 2 * 2)  # x_perm written, read
           + (0 if fused else S * 2 * I * 2 * 2)  # h written, read
           + S * I * 2 * (2 if fused else 1)     # a written (and read by the down GMM when fused)
           + S * H * 2 * 2      # yp written, read
           + T * H * 2)         # out written
    idx = T * K * 4 * 3 + T * K * 4 + len(gl) * 8
    return w + act + idx, n_active


def layer_forward(torch, dev, wl, steps, gather=False, routed=False):
    """Time the layer forward on workload `wl` -- permute -> gate_up GMM and
    SwiGLU (fused into one call, no H, except for decode-shaped calls where
    the weight-streaming gate_up + swiglu pair is faster) -> down GMM ->
    unpermute: wall ms per layer, per-call means, and whether it fused.
    gather: the permute computes the maps only and the gate_up GMM reads the
    token rows through sorted_slot (no x_perm).  routed: the whole forward
    as moe_decode_fwd (the routing fused into the gate_up GMM: no permute
    launch)."""
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayer

    d = wl.dims
    T, K, E, H, I = d["T"], d["K"], d["E"], d["H"], d["I"]
    x = bf16_dev(torch, wl["x"], dev)
    w1 = bf16_dev(torch, wl["w1"], dev)
    w2 = bf16_dev(torch, wl["w2"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    layer = MoeLayer(LayerShape(T, K, E, H, I), dev, gather_rows=gather or routed)
    timer = KernelTimer(torch)
    from grouped_gemm_moe_amd import gmm_fwd, moe_unpermute, swiglu_gmm_fwd
    g = layer.tokens_per_expert
    fused = layer.use_fused("auto") and not routed
    sfx = "_gather" if gather else ""

    def step(t):
        if routed:
            t("moe_decode_fwd", lambda: layer.forward_decode(x, ids, probs, w1, w2))
            return
        t("moe_permute_index" if gather else "moe_permute", lambda: layer.permute(x, ids))
        if fused:
            t("gmm_fwd_swiglu" + sfx, lambda: layer.gate_up(w1, True, keep_h=False))
            t("gmm_fwd_down", lambda: gmm_fwd(layer.a, w2, g, out=layer.yp))
        else:
            t("gmm_fwd_gate_up" + sfx, lambda: layer.gate_up(w1, False))
            t("swiglu_gmm_fwd_down", lambda: swiglu_gmm_fwd(layer.h, w2, g, out=(layer.a, layer.yp)))
        t("moe_unpermute", lambda: moe_unpermute(layer.yp, layer.row_id_map, probs, out=layer.out))

    plain = lambda name, fn: fn()  # noqa: E731
    for _ in range(10):
        step(plain)
    torch.cuda.synchronize()
    # wall time without events, then a pass with per-call events
    t0 = time.perf_counter()
    for _ in range(steps):
        step(plain)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    for _ in range(min(50, steps)):
        step(timer)
    torch.cuda.synchronize()
    per = {k: float(np.mean(v)) for k, v in timer.collect().items()}
    spans = percentiles(step_spans(torch, lambda: step(plain), min(50, steps)))
    gl = layer.tokens_per_expert.cpu().numpy()
    return ms, per, gl, (layer, probs, fused, spans)


def end_backward(torch, dev, layer, probs, steps=20):
    """Time the backward of the two ends on a forward's buffers: the
    unpermute backward (dYp and dprobs from a synthetic dout) and the permute
    backward (dx from a synthetic dX_perm), in GB/s of algorithmic bytes."""
    from grouped_gemm_moe_amd import moe_permute_bwd, moe_unpermute_bwd

    s = layer.shape
    T, K, H = s.T, s.top_k, s.H
    R = int(layer.tokens_per_expert.sum().item())
    g = torch.Generator(device=dev).manual_seed(9)
    dout = torch.randn((T, H), generator=g, device=dev).to(torch.bfloat16)
    dxp = torch.randn((s.S, H), generator=g, device=dev).to(torch.bfloat16)
    dyp = torch.empty((s.S, H), dtype=torch.bfloat16, device=dev)
    dp = torch.empty((T, K), dtype=torch.float32, device=dev)
    dx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    calls = {
        "moe_unpermute_bwd": (lambda: moe_unpermute_bwd(dout, layer.yp, layer.row_id_map, probs,
                                                        out=(dyp, dp)),
                              T * H * 2 + 2 * R * H * 2 + 2 * T * K * 4 + s.S * 4),
        "moe_permute_bwd": (lambda: moe_permute_bwd(dxp, layer.row_id_map, T, out=dx),
                            R * H * 2 + T * H * 2 + s.S * 4),
    }
    res = {}
    for name, (fn, nbytes) in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = dict(us=round(us, 2), bytes=nbytes, gb_per_s=round(gbs, 1),
                         frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
    return res


def layer_roofline(gl, T, K, H, I, ms, fused=True, gathered=False):
    """Algorithmic bytes and FLOPs of one layer forward and the fraction of
    the attainable roofline max(FLOPs / MFMA peak, bytes / HBM peak) that the
    measured time reaches."""
    nbytes, n_active = decode_bytes(gl, T, K, H, I, fused, gathered)
    S = int(np.sum(gl))
    flops = 2.0 * S * H * 2 * I + 2.0 * S * I * H
    t_mem = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    roof_ms = max(t_mem, t_mfma) * 1e3
    return dict(bytes_per_layer=nbytes, active_experts=n_active, gflop_per_layer=round(flops / 1e9, 2),
                bound="hbm" if t_mem >= t_mfma else "mfma", roofline_ms=round(roof_ms, 4),
                frac_of_attainable=round(roof_ms / ms, 4))


def run_decode(torch, dev, args):
    """The decode layer forward as the library runs it for decode shapes,
    moe_decode_fwd (the headline: routing fused into the weight-streaming
    gate_up GMM, SwiGLU into the down GMM's row staging, then unpermute),
    with the five-call chain (x_perm materialised, as a training forward
    needs) and the gathered chain beside it, each on the normal and the
    skewed routing."""
    import workloads

    wl = workloads.decode()
    d = wl.dims
    T, K, H, I = d["T"], d["K"], d["H"], d["I"]
    ms, per, gl, (_, _, fused, spans) = layer_forward(torch, dev, wl, args.decode_steps)
    roof = layer_roofline(gl, T, K, H, I, ms, fused)
    n_active = roof["active_experts"]
    gate_up = "gmm_fwd_swiglu" if fused else "gmm_fwd_gate_up"
    down = "gmm_fwd_down" if fused else "swiglu_gmm_fwd_down"
    wbytes = {k: n_active * (H * 2 * I if k == gate_up else I * H) * 2 for k in (gate_up, down)}
    # the same layer with one hot expert (about 50 rows; the others 0-6)
    sk = workloads.decode_skewed()
    ms_s, per_s, gl_s, (_, _, fused_s, _) = layer_forward(torch, dev, sk, args.decode_steps)
    roof_s = layer_roofline(gl_s, T, K, H, I, ms_s, fused_s)
    chain = dict(workload="the same layer as five calls: moe_permute (x_perm materialised) -> gmm_fwd "
                          "(gate_up) -> swiglu_gmm_fwd -> moe_unpermute",
                 ms_per_layer=round(ms, 4), layer_ms_events=spans,
                 gb_per_s=round(roof["bytes_per_layer"] / (ms * 1e-3) / 1e9, 1),
                 bytes_per_layer=roof["bytes_per_layer"], frac_of_attainable=roof["frac_of_attainable"],
                 per_call_us={k: round(v * 1e3, 2) for k, v in per.items()},
                 gmm_weight_stream_gbs={k: round(wbytes[k] / (per[k] * 1e-3) / 1e9, 1) for k in wbytes},
                 skewed=dict(ms_per_layer=round(ms_s, 4),
                             gb_per_s=round(roof_s["bytes_per_layer"] / (ms_s * 1e-3) / 1e9, 1),
                             per_call_us={k: round(v * 1e3, 2) for k, v in per_s.items()}))
    gathered = gathered_layer(torch, dev, wl, args.decode_steps, T, K, H, I)
    routed = routed_layer(torch, dev, wl, args.decode_steps, T, K, H, I)
    routed_s = routed_layer(torch, dev, sk, args.decode_steps, T, K, H, I)
    gbs = routed["gb_per_s"]
    return dict(
        metric="decode MoE layer HBM GB/s",
        workload="decode layer forward: T=64 tokens, top-8 of E=256, hidden 2048, intermediate 512; "
                 "moe_decode_fwd: permute fused into the weight-streaming gate_up GMM -> SwiGLU fused into "
                 "the down GMM -> unpermute",
        value=gbs, unit="GB/s", ms_per_layer=routed["ms_per_layer"], layer_ms_events=routed["layer_ms_events"],
        frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4), bytes_per_layer=routed["bytes_per_layer"],
        active_experts=n_active, frac_of_attainable=routed["frac_of_attainable"],
        per_call_us=routed["per_call_us"],
        skewed=dict(workload="decode layer forward, expert 7 routed 48 more tokens (max rows per expert "
                             f"{int(np.max(gl_s))})",
                    ms_per_layer=routed_s["ms_per_layer"], gb_per_s=routed_s["gb_per_s"]),
        chain=chain,
        gathered=gathered,
    )


def gathered_layer(torch, dev, wl, steps, T, K, H, I):
    """The same layer forward with the dispatch fused into the gate_up GMM
    (moe_permute_index, then the gate_up GMM gathers token rows itself): its
    time, and its fraction of its own roofline, whose bytes no longer hold
    the x_perm write and read."""
    ms, per, gl, (_, _, fused, spans) = layer_forward(torch, dev, wl, steps, gather=True)
    roof = layer_roofline(gl, T, K, H, I, ms, fused, gathered=True)
    return dict(ms_per_layer=round(ms, 4), layer_ms_events=spans,
                gb_per_s=round(roof["bytes_per_layer"] / (ms * 1e-3) / 1e9, 1),
                bytes_per_layer=roof["bytes_per_layer"], roofline_ms=roof["roofline_ms"],
                frac_of_attainable=roof["frac_of_attainable"],
                per_call_us={k: round(v * 1e3, 2) for k, v in per.items()})


def routed_layer(torch, dev, wl, steps, T, K, H, I):
    """The decode layer forward as moe_decode_fwd: the gathered path's
    tensors (same algorithmic bytes) without its permute launch."""
    ms, per, gl, (_, _, _, spans) = layer_forward(torch, dev, wl, steps, routed=True)
    roof = layer_roofline(gl, T, K, H, I, ms, False, gathered=True)
    return dict(ms_per_layer=round(ms, 4), layer_ms_events=spans,
                gb_per_s=round(roof["bytes_per_layer"] / (ms * 1e-3) / 1e9, 1),
                bytes_per_layer=roof["bytes_per_layer"], roofline_ms=roof["roofline_ms"],
                frac_of_attainable=roof["frac_of_attainable"],
                per_call_us={k: round(v * 1e3, 2) for k, v in per.items()})


def run_prefill(torch, dev, args):
    import workloads

    wl = workloads.prefill()
    d = wl.dims
    T, K, H, I = d["T"], d["K"], d["H"], d["I"]
    ms, per, gl, (layer, probs, fused, spans) = layer_forward(torch, dev, wl, args.prefill_steps)
    roof = layer_roofline(gl, T, K, H, I, ms, fused)
    ends = end_backward(torch, dev, layer, probs)
    gbs = roof["bytes_per_layer"] / (ms * 1e-3) / 1e9
    tflops = roof["gflop_per_layer"] * 1e9 / (ms * 1e-3) / 1e12
    return dict(
        metric="prefill MoE layer forward: % of attainable roofline",
        workload="prefill layer forward: T=4096 tokens, top-8 of E=128, hidden 2048, "
                 "intermediate 512; permute -> gate_up GMM fused with SwiGLU -> down -> unpermute",
        value=round(100.0 * roof["frac_of_attainable"], 2), unit="% of attainable roofline",
        ms_per_layer=round(ms, 4), layer_ms_events=spans, gb_per_s=round(gbs, 1), tflops=round(tflops, 2),
        pct_bf16_mfma_peak=round(100.0 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4), **roof,
        per_call_us={k: round(v * 1e3, 2) for k, v in per.items()},
        end_backward=ends,
        gathered=gathered_layer(torch, dev, wl, args.prefill_steps, T, K, H, I),
    )


# ---------------------------------------------------------------------------
# MXFP8 (A8W8-FP) forward: decode and prefill layers, the ep rank's GMMs
# ---------------------------------------------------------------------------

MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, published


def mx_weights(torch, dev, wl):
    """The workload's bf16 weights as MX pairs (MoeLayerMX.prepare_weights:
    transposed once and MX-quantised on the device; not part of a timed
    step)."""
    from grouped_gemm_moe_amd.pipeline import MoeLayerMX

    return MoeLayerMX.prepare_weights(bf16_dev(torch, wl["w1"], dev), bf16_dev(torch, wl["w2"], dev))


def mx_layer_bytes(gl, T, K, H, I, gathered=False):
    """Algorithmic bytes of one A8W8-FP layer forward: MX weights (codes and
    one scale byte per 32) of experts with rows, once; x read; the MX
    activations (xq/xs of every slot row -- or of the T token rows when GMM1
    gathers them --, aq/as) and Yp written once and read once; out written;
    indices."""
    n_active = int(np.sum(np.asarray(gl) > 0))
    S = int(np.sum(gl))
    mx = 1.0 + 1.0 / 32
    w = n_active * (H * 2 * I + I * H) * mx
    xrows = T if gathered else S
    act = (T * H * 2 + xrows * H * mx * 2 + S * I * mx * 2 + S * H * 2 * 2 + T * H * 2)
    idx = T * K * 4 * 3 + T * K * 4 + len(gl) * 8
    return int(w + act + idx), n_active


def mx_layer_forward(torch, dev, wl, steps, gather=False, routed=False):
    """Time permute_mx -> gmm_mx_fwd_swiglu -> gmm_mx_fwd -> unpermute, or
    with gather: mx_quantize of the token rows -> moe_permute_index ->
    gmm_mx_fwd_swiglu_gather -> gmm_mx_fwd -> unpermute, or routed: mx_quantize
    -> moe_decode_fwd_mx (the routing inside GMM1)."""
    from grouped_gemm_moe_amd import (gmm_mx_fwd, gmm_mx_fwd_swiglu, gmm_mx_fwd_swiglu_gather,
                                      moe_permute_index, moe_permute_mx, moe_unpermute, mx_quantize)
    from grouped_gemm_moe_amd.pipeline import LayerShape, MoeLayerMX

    d = wl.dims
    T, K, E, H, I = d["T"], d["K"], d["E"], d["H"], d["I"]
    (w1q, w1s), (w2q, w2s) = mx_weights(torch, dev, wl)
    x = bf16_dev(torch, wl["x"], dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    probs = torch.from_numpy(wl["probs"]).to(dev)
    L = MoeLayerMX(LayerShape(T, K, E, H, I), dev, gather_rows=gather or routed)
    g, err = L.tokens_per_expert, L.dev_err
    timer = KernelTimer(torch)

    def step(t):
        if routed:
            t("moe_decode_fwd_mx", lambda: L.forward_decode(x, ids, probs, (w1q, w1s), (w2q, w2s)))
            return
        if gather:
            t("mx_quantize", lambda: mx_quantize(x, out=(L.xq, L.xs)))
            t("moe_permute_index", lambda: moe_permute_index(ids, E, out=(L.row_id_map, L.sorted_slot, g),
                                                             ws=L.ws_perm, dev_err=err))
            t("gmm_mx_fwd_swiglu", lambda: gmm_mx_fwd_swiglu_gather(L.xq, L.xs, L.sorted_slot, K, w1q, w1s, g,
                                                                    out=(L.aq, L.as_), dev_err=err))
        else:
            t("moe_permute_mx", lambda: moe_permute_mx(x, ids, E, out=(L.xq, L.xs, L.row_id_map,
                                                                      L.sorted_slot, g),
                                                       ws=L.ws_perm, dev_err=err))
            t("gmm_mx_fwd_swiglu", lambda: gmm_mx_fwd_swiglu(L.xq, L.xs, w1q, w1s, g, out=(L.aq, L.as_),
                                                             dev_err=err))
        t("gmm_mx_fwd_down", lambda: gmm_mx_fwd(L.aq, L.as_, w2q, w2s, g, out=L.yp, dev_err=err))
        t("moe_unpermute", lambda: moe_unpermute(L.yp, L.row_id_map, probs, out=L.out, dev_err=err))

    plain = lambda name, fn: fn()  # noqa: E731
    for _ in range(10):
        step(plain)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(plain)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    for _ in range(min(50, steps)):
        step(timer)
    torch.cuda.synchronize()
    per = {k: float(np.mean(v)) for k, v in timer.collect().items()}
    spans = percentiles(step_spans(torch, lambda: step(plain), min(50, steps)))
    assert int(err.item()) == 0, "device error word set during the MX bench"
    return ms, per, g.cpu().numpy(), spans


def run_mx(torch, dev, args):
    """The A8W8-FP forward on the decode and prefill layers and the ep rank."""
    import workloads

    res = {}
    for name, make, steps in (("decode", workloads.decode, args.decode_steps),
                              ("prefill", workloads.prefill, args.prefill_steps),
                              ("ep_forward", workloads.ep_slice, args.prefill_steps)):
        wl = make()
        d = wl.dims
        T, K, H, I = d["T"], d["K"], d["H"], d["I"]
        ms, per, gl, spans = mx_layer_forward(torch, dev, wl, steps)
        nbytes, n_active = mx_layer_bytes(gl, T, K, H, I)
        S = int(np.sum(gl))
        f1, f2 = 2.0 * S * H * 2 * I, 2.0 * S * I * H
        t_mem = nbytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = (f1 + f2) / (MFMA_FP8_PEAK_TFLOPS * 1e12)
        roof_ms = max(t_mem, t_mfma) * 1e3
        g1 = per["gmm_mx_fwd_swiglu"] * 1e-3
        g2 = per["gmm_mx_fwd_down"] * 1e-3
        wbytes1 = n_active * H * 2 * I * (1 + 1 / 32)
        wbytes2 = n_active * I * H * (1 + 1 / 32)
        res[name] = dict(
            ms_per_layer=round(ms, 4), layer_ms_events=spans,
            gb_per_s=round(nbytes / (ms * 1e-3) / 1e9, 1),
            tflops=round((f1 + f2) / (ms * 1e-3) / 1e12, 2), bytes_per_layer=nbytes,
            bound="hbm" if t_mem >= t_mfma else "mfma", roofline_ms=round(roof_ms, 4),
            frac_of_attainable=round(roof_ms / ms, 4), active_experts=n_active,
            gmm_tflops={"gmm_mx_fwd_swiglu": round(f1 / g1 / 1e12, 1),
                        "gmm_mx_fwd_down": round(f2 / g2 / 1e12, 1)},
            gmm_pct_fp8_peak={"gmm_mx_fwd_swiglu": round(100 * f1 / g1 / 1e12 / MFMA_FP8_PEAK_TFLOPS, 2),
                              "gmm_mx_fwd_down": round(100 * f2 / g2 / 1e12 / MFMA_FP8_PEAK_TFLOPS, 2)},
            gmm_weight_stream_gbs={"gmm_mx_fwd_swiglu": round(wbytes1 / g1 / 1e9, 1),
                                   "gmm_mx_fwd_down": round(wbytes2 / g2 / 1e9, 1)},
            per_call_us={k: round(v * 1e3, 2) for k, v in per.items()},
        )
        # the same layer with GMM1 gathering the quantised token rows (no
        # per-slot copy): its time and its fraction of its own roofline
        ms_g, per_g, gl_g, spans_g = mx_layer_forward(torch, dev, wl, steps, gather=True)
        nbytes_g, _ = mx_layer_bytes(gl_g, T, K, H, I, gathered=True)
        roof_g = max(nbytes_g / (HBM_PEAK_GBS * 1e9), t_mfma) * 1e3
        res[name]["gathered"] = dict(ms_per_layer=round(ms_g, 4), layer_ms_events=spans_g,
                                     gb_per_s=round(nbytes_g / (ms_g * 1e-3) / 1e9, 1), bytes_per_layer=nbytes_g,
                                     roofline_ms=round(roof_g, 4), frac_of_attainable=round(roof_g / ms_g, 4),
                                     per_call_us={k: round(v * 1e3, 2) for k, v in per_g.items()})
        if name == "decode":
            # GMM1 routing its own rows (moe_decode_fwd_mx): the gathered tensors, no permute launch
            ms_r, per_r, _, spans_r = mx_layer_forward(torch, dev, wl, steps, routed=True)
            res[name]["routed"] = dict(ms_per_layer=round(ms_r, 4), layer_ms_events=spans_r,
                                       gb_per_s=round(nbytes_g / (ms_r * 1e-3) / 1e9, 1),
                                       frac_of_attainable=round(roof_g / ms_r, 4),
                                       per_call_us={k: round(v * 1e3, 2) for k, v in per_r.items()})
        log(f"mx {name}: {ms:.4f} ms/layer; {res[name]['gb_per_s']} GB/s; {res[name]['tflops']} TFLOP/s; "
            f"per call {res[name]['per_call_us']}; gathered {ms_g:.4f} ms/layer")
        del wl
        torch.cuda.empty_cache()
    res["workload"] = ("A8W8-FP (MXFP8) forward: permute_mx (gather + MX quantisation) -> gate_up GMM "
                       "with SwiGLU and MX requantisation -> down GMM -> unpermute; weights = the bf16 "
                       "workload weights MX-quantised on the device; decode (T=64, top-8, E=256), "
                       "prefill (T=4096, top-8, E=128), the ep rank (16384 rows, E=32, hidden 4096, "
                       "intermediate 1536)")
    res["dtype"] = "fp8 e4m3 x fp8 e4m3 (E8M0 scales), fp32 accumulation"
    return res


# ---------------------------------------------------------------------------
# Achievable ceilings on this GPU, for context (outside every timed step)
# ---------------------------------------------------------------------------

def best_ms(torch, fn, iters=10):
    """Best of 3 event-timed runs of `iters` back-to-back calls, ms per call."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    best = 1e9
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / iters)
    return best


def ceilings(torch, dev):
    """hipBLASLt (torch.matmul) on a dense bf16 product of the ep gate_up
    shape, and a 512 MiB device-to-device copy: what a vendor GEMM and a
    plain copy reach here, next to the published peaks."""
    M, K, N = 16384, 4096, 3072
    a = torch.randn((M, K), device=dev).to(torch.bfloat16)
    b = torch.randn((K, N), device=dev).to(torch.bfloat16)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    mm = best_ms(torch, lambda: torch.matmul(a, b, out=c))
    del a, b, c
    src = torch.empty(256 * 1024 * 1024, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    cp = best_ms(torch, lambda: dst.copy_(src))
    del src, dst
    torch.cuda.empty_cache()
    return dict(hipblaslt_bf16_tflops=round(2.0 * M * K * N / (mm * 1e-3) / 1e12, 1),
                hipblaslt_shape=[M, K, N],
                d2d_copy_gbs=round(2 * 512 * 2 ** 20 / (cp * 1e-3) / 1e9, 1),
                note="copy GB/s counts bytes read + written")


def run_dw_few_tiles(torch, dev):
    """A weight gradient whose tile grid cannot fill the chip: one dense
    expert, dW [2048, 1024] from 32768 rows (32 output tiles), which
    gmm_bwd_weight splits along the rows."""
    import grouped_gemm_moe_amd as moe

    M, K, N = 32768, 2048, 1024
    x = torch.randn((M, K), device=dev).to(torch.bfloat16)
    dy = torch.randn((M, N), device=dev).to(torch.bfloat16)
    g = torch.tensor([M], dtype=torch.int64, device=dev)
    ws = torch.zeros(moe.gmm_workspace_size(1, M, K, N, moe.OP_BWD_WEIGHT), dtype=torch.uint8, device=dev)
    dw = torch.empty((1, K, N), dtype=torch.bfloat16, device=dev)
    ms = best_ms(torch, lambda: moe.gmm_bwd_weight(x, dy, g, out=dw, ws=ws))
    return dict(shape=[M, K, N], us=round(ms * 1e3, 2),
                tflops=round(2.0 * M * K * N / (ms * 1e-3) / 1e12, 1),
                note="dW = x^T dy for one expert; 32 output tiles, the row reduction split in chunks")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample of the ep step
# ---------------------------------------------------------------------------

def cpu_baseline(wl, budget_s):
    import oracle

    # The host cores this process may run on; the BLAS pool is pinned to
    # them, or to the thread limit the environment sets if that is lower
    # (on a shared host OMP_NUM_THREADS states this process's share).
    affinity = len(os.sched_getaffinity(0))
    threads = affinity
    env_limit = os.environ.get("OMP_NUM_THREADS", "")
    if env_limit.isdigit() and 0 < int(env_limit) < threads:
        threads = int(env_limit)
    try:
        from threadpoolctl import threadpool_limits
        pin = threadpool_limits(limits=threads, user_api="blas")
    except Exception:
        pin = None
    gl = wl["group_list"]
    H, I = wl.dims["H"], wl.dims["I"]
    ss, _, _ = oracle.permute_maps(wl["topk_ids"], len(gl))
    off = oracle.expert_offsets(gl)
    flops = 0.0
    rows = 0
    active = [int(e) for e in np.nonzero(gl > 0)[0]]
    passes, done = 0, []  # whole passes over the active experts, then the experts of a partial one
    t0 = time.perf_counter()
    while True:
        done = []
        for e in active:
            n = int(gl[e])
            sl = slice(off[e], off[e + 1])
            xe = oracle.bf16_to_f64(wl["x"][ss[sl]])
            dye = oracle.bf16_to_f64(wl["dyp"][sl])
            w1e = oracle.bf16_to_f64(wl["w1"][e:e + 1])
            w2e = oracle.bf16_to_f64(wl["w2"][e:e + 1])
            h = oracle.round_bf16(oracle.gmm(xe, w1e, [n]))
            a = oracle.round_bf16(oracle.swiglu(h))
            oracle.round_bf16(oracle.gmm(a, w2e, [n]))
            oracle.expert_block_backward(xe, h, a, dye, w1e, w2e, [n])
            flops += 3 * (2.0 * n * H * 2 * I + 2.0 * n * I * H)
            rows += n
            done.append(e)
            if time.perf_counter() - t0 >= budget_s:
                break
        if len(done) == len(active):
            passes, done = passes + 1, []
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    if pin is not None:
        pin.restore_original_limits()
    what = f"{passes} whole pass{'es' if passes != 1 else ''} over the {len(active)} active experts"
    if done:
        what += f" and experts {done} of one more"
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=round(flops / el / 1e12, 5), unit="TFLOP/s", cores=int(threads), kind="oracle",
                affinity_cpus=affinity, cpu_model=model,
                sample=f"oracle (NumPy float64) expert-block fwd+bwd GEMM chain: {what} "
                       f"({rows} rows; {int(gl.sum())} per pass), {flops / 1e9:.1f} GFLOP in {el:.1f} s",
                seconds=round(el, 2))


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import grouped_gemm_moe_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    moe.library()
    dev = torch.device("cuda:0")
    log(f"device: {torch.cuda.get_device_name(0)}")
    ep, wl = run_ep(torch, dev, args)
    log(f"ep: {ep['ms_per_step']:.3f} ms/step, {ep['value']:.1f} TFLOP/s; per call {ep['per_call_us']}")
    log(f"ep, memory-optimised backward: {ep['low_memory_backward']}")
    decode = prefill = None
    if not args.skip_decode:
        decode = run_decode(torch, dev, args)
        log(f"decode: {decode['ms_per_layer']:.4f} ms, {decode['value']:.0f} GB/s; {decode['per_call_us']}")
        log(f"decode, one hot expert: {decode['skewed']}; five-call chain: {decode['chain']}")
        prefill = run_prefill(torch, dev, args)
        log(f"prefill: {prefill['ms_per_layer']:.4f} ms, {prefill['value']:.1f} % of attainable "
            f"({prefill['bound']}-bound); {prefill['per_call_us']}")
    mx = None
    if not args.skip_mx:
        mx = run_mx(torch, dev, args)
    ceil = None
    dw_few = None
    if not args.skip_mx and not args.skip_decode:
        ceil = ceilings(torch, dev)
        log(f"ceilings: {ceil}")
        dw_few = run_dw_few_tiles(torch, dev)
        log(f"dW on few tiles (row reduction split): {dw_few}")
    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(wl, args.cpu_budget)
        cpu["gpu_speedup"] = round(ep["value"] / cpu["value"], 1)
        log(f"cpu baseline: {cpu}")
    line = {
        "metric": "GMM fwd+bwd TFLOP/s & % bf16 MFMA peak; decode MoE layer HBM GB/s",
        "value": round(ep["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ep["ms_per_step"], 4),
        "step_ms_events": ep["step_ms_events"],
        "frac_of_attainable": ep["frac_of_attainable"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "one expert-parallel rank's share, fwd+bwd: E=32 local experts, hidden 4096, "
                        "intermediate 1536, 16384 received rows (top_k=1 local re-routing), Zipf(1.2) "
                        "group sizes with 3 empty experts; permute -> gate_up GMM fused with SwiGLU -> down GMM "
                        "-> unpermute -> expert-block backward (dX and dW of both GMMs)",
            "experts": 32, "hidden": 4096, "intermediate": 1536, "rows": 16384,
            "gemm_gflop_per_step": round(ep["gemm_gflop_per_step"], 1),
        },
        "pct_bf16_mfma_peak": round(100.0 * ep["value"] / MFMA_BF16_PEAK_TFLOPS, 2),
        "gmm_only_tflops": round(ep["gmm_only_tflops"], 2),
        "per_call_us": ep["per_call_us"],
        "low_memory_backward": ep["low_memory_backward"],
        "roofline": ep["roofline"],
        "decode": decode,
        "prefill": prefill,
        "mxfp8": mx,
        "ceilings": ceil,
        "dw_few_tiles": dw_few,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 512 MiB device copies done")


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--sweep A,B] [--no-graph]

A step is one whole layer forward (router, dispatch, expert FFN, combine)
through the C ABI (moe_forward) over one batch of synthetic input that is
already resident in HBM.  The headline workload is the 2048-token prefill
chunk (T=2048, d_model=2048, d_ff=512, E=512, top-10, affine 4-bit g64, fused
gate|up).  Every other workload runs in the same process and is reported
under "sweep": the tiny fp32 layer, the dense bf16 layer at T=512, the decode
layer at T=1 and T=32 and the skewed layer at T=256, each with its own
roofline and oracle timing, plus the backward pass with respect to x
(moe_backward) of the decode and prefill layers.  Weight copies and x copies
rotate from step to step so that the bytes between two reuses of the same
buffer exceed the 256 MB Infinity Cache: every step streams its weights from
HBM.  Each workload's K steps are timed twice, launched eagerly from Python
and as one captured HIP graph of the same K forwards; the faster of the two
is the reported step time ("launch" says which), both are in the line.

Prints ONE JSON line on stdout (everything else goes to stderr).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, TFLOP/s
VALU_F32_PEAK_TFLOPS = 157.3    # MI355X published fp32 vector peak
METRIC = "MoE layer routed rows/s at T=1/32/2048; % of HBM or MFMA roofline"
ROTATE_BYTES = 1 << 30          # reuse distance of weight buffers


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the benchmark needs for raw stream events."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    # Timing-only events: recording one performs no system-scope fence (no
    # L2 write-back and invalidate between the kernels it separates), so the
    # kernels run as they do untimed and the bracket adds little of its own.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def record(self, e, stream: int):
        assert self.lib.hipEventRecord(e, stream) == 0

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


_SLEEP_CYCLES_PER_MS = None


def hold_stream(ms: float):
    """Enqueue a spin kernel of about `ms` milliseconds on torch's current
    stream, so that the host enqueues the launches that follow before the GPU
    reaches them: events recorded between those kernels then time them back to
    back, as a kernel trace does, rather than the host's launch gaps."""
    global _SLEEP_CYCLES_PER_MS
    import torch
    if _SLEEP_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(1 << 22)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = (1 << 22) / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(min(ms, 1000.0) * _SLEEP_CYCLES_PER_MS))


def workload_name(spec, what: str = "forward") -> str:
    w = f"affine {spec.bits}-bit g{spec.group_size}" if spec.quantized else f"dense {spec.act}"
    extra = (", fused gate|up" if spec.gate_up_fused else "") + (
        ", GeGLU (tanh-GELU gate)" if spec.activation == "geglu" else "") + (
        f", per-op {spec.act} GLU rounding" if spec.glu_round else "") + (
        f", {spec.n_shared} shared experts" if spec.n_shared else "") + (
        ", Zipf-skewed router bias" if spec.router_bias == "zipf" else "")
    return (f"{spec.name}: MoE layer {what} T={spec.T} d_model={spec.d_model} d_ff={spec.d_ff} "
            f"E={spec.n_experts} top-{spec.top_k}, {spec.act} activations, {w} experts{extra}")


def data_note(spec) -> str:
    w = (f"quantised to affine {spec.bits}-bit g{spec.group_size}" if spec.quantized
         else f"stored as {spec.act}")
    return f"synthetic (seeded N(0,1/fan_in) weights {w}, N(0,1) {spec.act} x)"


def expert_bytes(spec) -> int:
    """Stored bytes of one expert's gate, up and down weights."""
    n = 3 * spec.d_model * spec.d_ff
    if spec.quantized:
        return n * spec.bits // 8 + (n // spec.group_size) * 4
    return n * (4 if spec.act == "f32" else 2)


def expert_output_bytes(spec) -> float:
    """Bytes per expert-output element between the down projection and the
    combine, in the format moe_forward picks (the library's rule restated):
    fp16 plus one exponent byte per 64 columns on the 16-bit matrix-core
    tiles; fp32 on the vector-unit and decode kernels and when the down
    reduction is split into fp32 partial rows (counted once here)."""
    T, D, F, E, K, S = spec.T, spec.d_model, spec.d_ff, spec.n_experts, spec.top_k, spec.n_shared
    if spec.act == "f32" or D % 64 or F % 64:
        return 4
    N = T * K
    tr = 16 if N <= 8 * E else 64
    if tr == 16 and spec.quantized and N <= E and D <= 2048 and F <= 2048:
        return 4  # decode kernel
    R = N + S * T
    tiles, nbx, nslab = max(min(R, E + S), -(-R // tr)), -(-D // 256), -(-F // 128)
    kz = 1
    while tiles * nbx * kz < 512 and kz < 8 and nslab >= 4 * kz:
        kz *= 2
    return 4 if kz > 1 else 2 + 1 / 64


def accounting(spec, touched: int):
    """Algorithmic bytes and FLOPs of one forward, and per kernel.

    The layer's bytes are the stored weights of the experts the batch touches
    (plus shared experts), the router matrix, x and y.  Per kernel, the
    roofline counts what the step cannot avoid moving: the gate/up launch the
    gate and up weights of the touched experts and x; the down launch the down
    weights; the router launches the router matrix and x.  The intermediates a
    fused implementation need not move (h between the projections, the
    expert outputs between down and combine) are reported beside them, as
    stored by this library, under "intermediate_bytes".
    """
    T, D, F, E, K, S = spec.T, spec.d_model, spec.d_ff, spec.n_experts, spec.top_k, spec.n_shared
    esz = 4 if spec.act == "f32" else 2
    N, R = T * K, T * K + S * T
    eb = expert_bytes(spec)
    w_touched = (touched + S) * eb
    router = D * E * esz
    x_bytes = y_bytes = T * D * esz
    h_bytes = R * F * esz
    ys_bytes = int(R * D * expert_output_bytes(spec))
    gateup = {"bound": "hbm", "bytes": int(w_touched * 2 / 3) + x_bytes, "flops": 2 * R * 2 * D * F,
              "intermediate_bytes": {"h_written": h_bytes}}
    down = {"bound": "hbm", "bytes": int(w_touched / 3), "flops": 2 * R * D * F,
            "intermediate_bytes": {"h_read": h_bytes, "expert_outputs_written": ys_bytes}}
    chunks = -(-D // 64)
    part_bytes = chunks * T * E * 4      # vector-unit router: per-chunk logit partials
    lt_bytes = 2 * T * E * 4             # matrix-core router: two partial logit arrays
    route = {"bound": "hbm", "bytes": router + x_bytes, "flops": 2 * T * D * E,
             "intermediate_bytes": {"router_transposed_written": router, "logit_partials_written": lt_bytes}}
    acc = {
        "layer_bytes": w_touched + router + x_bytes + y_bytes,
        "expert_flops": 2 * R * 3 * D * F,
        "router_flops": 2 * T * D * E,
        # FLOPs of the sparse layer over those of the dense all-experts layer
        "sparse_dense_flop_ratio": (K + S) / (E + S),
        "kernels": {
            # vector-unit router: canonical-order logits (fp32 FMA chains)
            "route_logits": {"bound": "alu", "flops": 2 * T * D * E, "bytes": router + x_bytes,
                             "intermediate_bytes": {"chunk_partials_written": part_bytes}},
            "route_select": {"bound": "hbm", "bytes": N * 8,
                             "intermediate_bytes": {"chunk_partials_read": part_bytes}},
            "route_mfma": route,
            # candidates' exact chains re-read x and router rows; the fp16 staging copy of x is written here
            "route_certify": {"bound": "hbm", "bytes": N * 8,
                              "intermediate_bytes": {"logit_partials_read": lt_bytes, "x_read": x_bytes,
                                                     "x16_written": T * D * 2}},
            "dispatch": {"bound": "hbm", "bytes": N * 4 * 4},
            "route_select_dispatch": {"bound": "hbm", "bytes": N * 8 + N * 4 * 4,
                                      "intermediate_bytes": {"chunk_partials_read": part_bytes}},
            "x_f16": {"bound": "hbm", "bytes": 2 * x_bytes},
            "gateup_gemv": gateup, "down_gemv": down,
            "gateup_mfma": gateup, "down_mfma": down,
            "combine": {"bound": "hbm", "bytes": y_bytes + N * 8,
                        "intermediate_bytes": {"expert_outputs_read": ys_bytes}},
            # one token: selection fused with gate/up, down fused with the combine
            "select_gateup": {**gateup, "bytes": gateup["bytes"] + N * 8,
                              "intermediate_bytes": {"chunk_partials_read": part_bytes, "h_written": R * F * 4}},
            "down_combine": {**down, "bytes": down["bytes"] + y_bytes,
                             "intermediate_bytes": {"h_read": R * F * 4}},
        },
    }
    return acc


_HOST = {}


def host_layer(name):
    """The seeded synthetic layer of a workload (generated once per process)."""
    from sparse_mixture_experts_amd import inputs
    if name not in _HOST:
        t0 = time.time()
        _HOST[name] = inputs.gen_layer(inputs.workload(name))
        log(f"[{name}] generated in {time.time() - t0:.1f}s")
    return _HOST[name]


def run_config(name, steps, warmup, use_graph, hip):
    import torch
    from sparse_mixture_experts_amd import inputs, moe

    spec = inputs.workload(name)
    dev = "cuda:0"
    host = host_layer(name)
    desc = moe.desc_from_spec(spec)
    w0 = moe.DeviceWeights.from_layer(host, dev)
    if spec.quantized:
        # the tile-packed copy of the codes that the grouped kernels read
        # (made once per layer, outside the timed region)
        w0 = w0.with_packed(desc)
    wbytes = w0.nbytes()
    # at least two copies: a step never reads the buffers of the step before
    n_w = max(2, math.ceil(ROTATE_BYTES / max(1, wbytes)))
    weights = [w0] + [w0.clone() for _ in range(n_w - 1)]
    n_x = 8
    xs = [moe.to_device(inputs.gen_x(spec, i), dev) for i in range(n_x)]
    T = spec.T
    out_dt = {"bf16": moe.MOE_DT_BF16, "f16": moe.MOE_DT_F16}.get(spec.act, moe.MOE_DT_F32)
    y = torch.empty((T, spec.d_model), device=dev,
                    dtype={moe.MOE_DT_BF16: torch.bfloat16, moe.MOE_DT_F16: torch.float16}.get(out_dt, torch.float32))
    ws = torch.empty(moe.moe_workspace_size(desc, T), dtype=torch.uint8, device=dev)
    idx = torch.empty((T, spec.top_k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, spec.top_k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        moe.moe_forward(desc, T, xs[i % n_x], weights[i % n_w], y, out_dt, idx, wt, ws, stream)

    # experts touched by each x (for the algorithmic byte count)
    touched = []
    for i in range(n_x):
        step(i)
        torch.cuda.synchronize()
        touched.append(len(np.unique(idx.cpu().numpy())))
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region, eager: K whole forwards launched one by one from Python
    torch.cuda.synchronize()
    ta = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    tb = time.perf_counter()
    eager_ms = (tb - ta) * 1000.0 / steps

    # timed region, graph: the same K forwards (same rotation) captured into
    # one HIP graph and replayed once, so the host's per-call cost (Python,
    # ctypes, launch calls) is out of the measurement
    graph_ms = None
    if use_graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    moe.moe_forward(desc, T, xs[i % n_x], weights[i % n_w], y, out_dt, idx, wt, ws, cap)
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        ta = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        tb = time.perf_counter()
        graph_ms = (tb - ta) * 1000.0 / steps
        del g
    launch = "graph" if graph_ms is not None and graph_ms < eager_ms else "eager"
    ms = graph_ms if launch == "graph" else eager_ms

    # per-kernel durations on the launch stream: each kernel launched with a
    # start and a stop event of its own execution (summed per stage), with the
    # GPU held until the host has enqueued the K steps, so that no kernel
    # waits on the host
    kernel_ms, names = {}, []
    evs = [[hip.event() for _ in range(32)] for _ in range(steps)]
    torch.cuda.synchronize()
    hold_stream(2.0 + 2.0 * steps * eager_ms)
    for i in range(steps):
        names = moe.moe_forward_timed(desc, T, xs[i % n_x], weights[i % n_w], y, out_dt, idx, wt, ws,
                                      evs[i], stream)
    torch.cuda.synchronize()
    assert 0 < len(names) <= 16, names
    for j, nm in enumerate(names):
        kernel_ms[nm] = kernel_ms.get(nm, 0.0) + sum(
            hip.elapsed_ms(evs[i][2 * j], evs[i][2 * j + 1]) for i in range(steps)) / steps
    for row in evs:
        for e in row:
            hip.destroy(e)

    avg_touched = sum(touched[i % n_x] for i in range(steps)) / steps
    acc = accounting(spec, round(avg_touched))
    rows = T * spec.top_k
    res = {
        "name": name, "spec": spec, "ms_per_step": ms, "rows_per_s": rows / (ms / 1e3),
        "tokens_per_s": T / (ms / 1e3), "kernel_ms": kernel_ms, "acc": acc, "touched": avg_touched,
        "weight_copies": n_w, "x_copies": n_x, "launch": launch, "eager_ms": eager_ms, "graph_ms": graph_ms,
    }
    lb = acc["layer_bytes"]
    res["layer_gbs"] = lb / (ms / 1e3) / 1e9
    res["layer_hbm_frac"] = res["layer_gbs"] / HBM_PEAK_GBS
    res["layer_mfma_frac"] = acc["expert_flops"] / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    log(f"[{name}] {ms * 1e3:.1f} us/step, {res['rows_per_s']:.4g} rows/s, layer {res['layer_gbs']:.0f} GB/s "
        f"({100 * res['layer_hbm_frac']:.1f}% HBM), kernels(us): "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in kernel_ms.items()))
    del weights, xs, ws
    torch.cuda.empty_cache()
    return res


def backward_accounting(spec, touched: int):
    """Algorithmic bytes and FLOPs of one backward pass (input gradient).

    Bytes: the touched experts' weights and the router matrix once each, x and
    dy read, dx written.  FLOPs: g and u recomputed (4 R D F), v = Wd^T dy
    (2 R D F), dx rows = Wg^T dg + Wu^T du (4 R D F), router logits recomputed
    (2 T D E) and the router term of dx (2 T D K with renormalisation, else
    2 T D E).
    """
    T, D, F, E, K, S = spec.T, spec.d_model, spec.d_ff, spec.n_experts, spec.top_k, spec.n_shared
    esz = 4 if spec.act == "f32" else 2
    R = T * K + S * T
    w_touched = (touched + S) * expert_bytes(spec)
    nbytes = w_touched + D * E * esz + T * D * esz + 2 * T * D * 4
    flops = 10 * R * D * F + 2 * T * D * E + 2 * T * D * (K if spec.renormalize else E)
    return {"bytes": nbytes, "flops": flops}


def run_backward(name, steps, warmup, hip):
    """K whole backward passes (moe_backward: router and dispatch recomputed,
    then the gradient kernels) with rotating weights, x and dy."""
    import torch
    from sparse_mixture_experts_amd import inputs, moe

    spec = inputs.workload(name)
    dev = "cuda:0"
    host = host_layer(name)
    desc = moe.desc_from_spec(spec)
    w0 = moe.DeviceWeights.from_layer(host, dev)
    if spec.quantized:
        w0 = w0.with_packed(desc)
    n_w = max(2, math.ceil(ROTATE_BYTES / max(1, w0.nbytes())))
    weights = [w0] + [w0.clone() for _ in range(n_w - 1)]
    n_x = 4
    xs = [moe.to_device(inputs.gen_x(spec, i), dev) for i in range(n_x)]
    gen = torch.Generator(device="cpu").manual_seed(1234)
    dys = [torch.randn((spec.T, spec.d_model), generator=gen, dtype=torch.float32).to(dev) for _ in range(n_x)]
    T = spec.T
    dx = torch.empty((T, spec.d_model), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_backward_workspace_size(desc, T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # experts touched by each x (for the algorithmic byte count): one forward each
    fws = torch.empty(moe.moe_workspace_size(desc, T), dtype=torch.uint8, device=dev)
    idx = torch.empty((T, spec.top_k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, spec.top_k), dtype=torch.float32, device=dev)
    y = torch.empty((T, spec.d_model), dtype=torch.float32, device=dev)
    touched = []
    for i in range(n_x):
        moe.moe_forward(desc, T, xs[i], weights[0], y, moe.MOE_DT_F32, idx, wt, fws, stream)
        torch.cuda.synchronize()
        touched.append(len(np.unique(idx.cpu().numpy())))
    del fws, y

    def step(i):
        moe.moe_backward(desc, T, xs[i % n_x], weights[i % n_w], dys[i % n_x], dx, ws, stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    ta = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    tb = time.perf_counter()
    ms = (tb - ta) * 1000.0 / steps
    # GPU time per pass: the same K passes again between two events, with the
    # GPU held until the host has enqueued them
    hold_stream(2.0 + 2.0 * steps * ms)
    hip.record(e0, stream.cuda_stream)
    for i in range(steps):
        step(i)
    hip.record(e1, stream.cuda_stream)
    torch.cuda.synchronize()
    ev_ms = hip.elapsed_ms(e0, e1) / steps
    hip.destroy(e0)
    hip.destroy(e1)
    acc = backward_accounting(spec, round(sum(touched) / n_x))
    t = ev_ms / 1e3
    tflops = acc["flops"] / t / 1e12
    gbs = acc["bytes"] / t / 1e9
    rows = T * spec.top_k
    # 16-bit layers: the contractions run on the matrix cores (fp16 and bf16
    # operands, both 2.5 PFLOP/s dense); fp32 layers on the fp32 vector units.
    # The roofline is whichever of compute and HBM bytes takes longer at peak.
    mc = spec.act != "f32"
    fpeak = MFMA_BF16_PEAK_TFLOPS if mc else VALU_F32_PEAK_TFLOPS
    t_flop, t_hbm = acc["flops"] / (fpeak * 1e12), acc["bytes"] / (HBM_PEAK_GBS * 1e9)
    if t_hbm >= t_flop:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma" if mc else "alu", "achieved": round(tflops, 3), "peak": fpeak, "unit": "TFLOP/s",
                "frac": round(tflops / fpeak, 4)}
    log(f"[bwd:{name}] {ms * 1e3:.1f} us/step (events {ev_ms * 1e3:.1f} us), {tflops:.2f} TFLOP/s "
        f"({100 * tflops / fpeak:.1f}% of {'MFMA' if mc else 'fp32 VALU'}), {gbs:.0f} GB/s "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM)")
    entry = {
        "workload": workload_name(spec, "backward (dx)"), "value": round(rows / (ms / 1e3), 1),
        "unit": "routed rows/s", "tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
        "roofline": {"kernel": "whole backward pass", **roof, "traffic": measured_traffic(f"bwd_{name}", "backward"),
                     "avg_pass_us": round(ev_ms * 1e3, 2), "algorithmic_flops": acc["flops"],
                     "algorithmic_bytes": acc["bytes"], "flop_frac": round(tflops / fpeak, 4),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
    }
    del weights, xs, dys, ws
    torch.cuda.empty_cache()
    return entry


def weights_note(spec) -> str:
    return ("stored codes plus their tile-packed copy (moe_pack_weights, made once per layer outside the "
            "timed region), which the grouped matrix-core kernels read" if spec.quantized
            else f"stored {spec.act} weights")


def path_dtype(spec) -> str:
    """Arithmetic type of the expert contractions (they dominate the step).

    Affine weights are expanded to fp16 and the 16-bit activations are staged
    as fp16 scaled by powers of two, so those products run on fp16 matrix
    cores; dense bf16 / fp16 layers use bf16 / fp16 matrix cores; f32 layers
    use fp32 FMA.  All of them accumulate in fp32.
    """
    if spec.act == "f32":
        return "f32"
    return "fp16" if spec.quantized else ("fp16" if spec.act == "f16" else "bf16")


STAGE_SOURCES = {
    "route_logits": "route.hip", "route_select": "route.hip", "route_mfma": "route_mfma.hip",
    "route_certify": "route_mfma.hip", "route_select_dispatch": "route.hip", "dispatch": "dispatch.hip", "x_f16": "ffn_mfma.hip", "gateup_gemv": "ffn_gemv.hip",
    "down_gemv": "ffn_gemv.hip", "gateup_mfma": "ffn_mfma.hip", "down_mfma": "ffn_mfma.hip",
    "combine": "combine.hip", "select_gateup": "decode_fused.hip", "down_combine": "decode_fused.hip",
    # the whole backward pass: routing and dispatch recomputed, then the gradient kernels
    "backward": ("backward.hip", "backward_mfma.hip", "route.hip", "route_mfma.hip", "dispatch.hip",
                 "ffn_mfma.hip"),
}


def kernel_sources_digest(kernel: str) -> str:
    """SHA-256 over the source of the stage's kernels and every header of the
    library (stamps the traffic counters taken for that stage)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mixture_experts_amd", "csrc")
    headers = sorted(os.path.basename(p) for p in glob.glob(os.path.join(csrc, "*.h")))
    src = STAGE_SOURCES[kernel]
    for f in (list(src) if isinstance(src, tuple) else [src]) + headers:
        with open(os.path.join(ROOT, "sparse_mixture_experts_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(config: str, kernel: str):
    """HBM bytes per launch of `kernel` from the FETCH_SIZE/WRITE_SIZE counter
    summary stored for `config`, each counter scaled by what it reads for a
    copy kernel of known size.  None when no summary exists or the kernel
    sources changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    k = rec.get("kernels", {}).get(kernel)
    if k is None or k.get("sources_sha256") != kernel_sources_digest(kernel):
        return None
    cal = rec["copy_calibration"]
    f_fetch = cal["fetch_kib"] * 1024.0 / cal["bytes"]
    f_write = cal["write_kib"] * 1024.0 / cal["bytes"]
    return int(k["fetch_kib"] * 1024.0 / f_fetch + k["write_kib"] * 1024.0 / f_write)


def calibrate_copy(mib: int):
    """Copy kernel of known size for scaling the traffic counters: 3 launches
    of dst.copy_(src) over `mib` MiB."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def measured_peaks():
    """What this GPU reaches on plain streaming and dense work, measured in the
    same run (context for the published peaks the rooflines use): the
    library's streaming-read kernel over 1 GiB (8192 workgroups of 16-byte
    loads) and over 600 MiB (one launch's size at the prefill gate/up), torch's
    device copy of 1 GiB (read + write bytes), and a bf16 8192^3 matrix
    product (torch.matmul on the vendor GEMM library); each the best of 3
    timed rounds of 5 launches."""
    import torch
    from sparse_mixture_experts_amd import moe
    dev = "cuda:0"
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)

    def best_ms(fn, reps=5, rounds=3):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / reps)
        return best

    blocks = 8192
    words = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    n600 = 600 << 20
    read_ms = best_ms(lambda: moe.moe_stream_read(src, n, words, blocks))
    read600_ms = best_ms(lambda: moe.moe_stream_read(src, n600, words, blocks))
    copy_ms = best_ms(lambda: dst.copy_(src))
    gemm_ms = best_ms(lambda: torch.matmul(a, b))
    out = {"read_GBs": round(n / read_ms / 1e6, 1), "read_600MiB_GBs": round(n600 / read600_ms / 1e6, 1),
           "copy_GBs": round(2 * n / copy_ms / 1e6, 1),
           "bf16_gemm_TFLOPs": round(2 * 8192 ** 3 / gemm_ms / 1e9, 1),
           "how": "moe_stream_read over 1 GiB and over 600 MiB (8192 workgroups, 16-byte loads), torch device "
                  "copy of 1 GiB (read + write bytes), torch.matmul bf16 8192^3; best of 3 rounds of 5 launches"}
    del src, dst, a, b, words
    torch.cuda.empty_cache()
    return out


def roofline(res, peaks=None):
    """Roofline of the step's dominant kernel (the longest average launch):
    algorithmic bytes (or FLOPs for the vector-unit router) per launch over the
    launch's average duration from HIP events on the launch stream."""
    km = res["kernel_ms"]
    dom = max(km, key=km.get)
    traffic = measured_traffic(res["name"], dom)
    kacc = res["acc"]["kernels"].get(dom)
    t = km[dom] / 1e3
    if kacc is None:
        return {"kernel": dom, "bound": None, "achieved": None, "peak": None, "unit": None, "frac": None,
                "traffic": None}
    if kacc["bound"] == "alu":
        a = kacc["flops"] / t / 1e12
        return {"kernel": dom, "bound": "alu", "achieved": round(a, 3), "peak": VALU_F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / VALU_F32_PEAK_TFLOPS, 4), "traffic": traffic,
                "avg_launch_us": round(km[dom] * 1e3, 2), "algorithmic_flops_per_launch": kacc["flops"]}
    a = kacc["bytes"] / t / 1e9
    out = {"kernel": dom, "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic, "avg_launch_us": round(km[dom] * 1e3, 2),
           "algorithmic_bytes_per_launch": kacc["bytes"]}
    if peaks and peaks.get("read_GBs"):
        # the same rate against what a plain streaming read reaches on this GPU
        out["frac_of_measured_read"] = round(a / peaks["read_GBs"], 4)
    if "flops" in kacc:
        out["mfma_frac"] = round(kacc["flops"] / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    if "intermediate_bytes" in kacc:
        out["intermediate_bytes_per_launch"] = kacc["intermediate_bytes"]
    return out


def cpu_baseline(name, n_tokens, threads=None):
    """The oracle, as it stands, on the host cores over a bounded token sample
    (evenly spaced tokens of the workload, each routed over all experts and run
    through its selected experts); threads=None uses every core available to
    the process."""
    import oracle
    from sparse_mixture_experts_amd import inputs

    spec = inputs.workload(name)
    host = host_layer(name)
    d = oracle.Desc(spec.d_model, spec.d_ff, spec.n_experts, spec.top_k, spec.n_shared, spec.act == "bf16",
                    spec.quantized, spec.group_size, spec.gate_up_fused, spec.glu_round,
                    spec.renormalize, spec.bits, int(spec.activation == "geglu"),
                    spec.act == "f16")
    n = min(n_tokens, spec.T)
    toks = np.linspace(0, spec.T - 1, n).astype(np.int32)
    threads = threads or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    _, _, _, used = oracle.forward(d, host["x"], host["w_router"], host["router_bias"], host["experts"],
                                   tokens=toks, n_threads=threads)
    dt = time.perf_counter() - t0
    rows = n * spec.top_k
    return {"value": round(rows / dt, 2), "unit": "routed rows/s", "cores": used, "kind": "oracle",
            "tokens_per_s": round(n / dt, 3),
            "sample": f"{n} of {spec.T} tokens ({rows} routed rows) of {name}, each routed and run through "
                      f"its {spec.top_k} experts; {dt:.2f} s wall on {used} threads"}


# Oracle sample per workload for the sweep's cpu_baseline (tokens), and the
# workloads also timed on one thread (tokens).
CPU_SAMPLE = {"tiny-f32": 16, "dense-bf16-t512": 512, "q4-decode-t1": 1, "q4-decode-t32": 32,
              "q4-skewed-t256": 256, "q4-prefill-t2048": 256}
CPU_ONE_THREAD = {"tiny-f32": 16, "q4-decode-t1": 1, "q4-decode-t32": 8}
DEFAULT_SWEEP = ("tiny-f32,dense-bf16-t512,q4-decode-t1,q4-decode-t32,q4-skewed-t256,"
                 "bwd:q4-decode-t1,bwd:q4-decode-t32,bwd:q4-prefill-t2048")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="q4-prefill-t2048")
    ap.add_argument("--sweep", default=DEFAULT_SWEEP,
                    help="further workloads; a bwd: prefix times the backward pass (moe_backward) instead")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (default: also one HIP graph of the K steps; the faster is reported)")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of the headline workload the oracle runs for cpu_baseline (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device copy of MIB MiB (scale for the HBM traffic counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    from sparse_mixture_experts_amd import moe
    moe.load()
    hip = Hip()
    peaks = measured_peaks()
    log(f"[measured peaks] {peaks}")

    head = run_config(args.config, args.steps, args.warmup, not args.no_graph, hip)
    sweep = []
    for name in [s for s in args.sweep.split(",") if s]:
        if name.startswith("bwd:"):
            sweep.append(run_backward(name[4:], args.steps, args.warmup, hip))
            continue
        r = run_config(name, args.steps, args.warmup, not args.no_graph, hip)
        entry = {
            "workload": workload_name(r["spec"]), "value": round(r["rows_per_s"], 1), "unit": "routed rows/s",
            "tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 5),
            "layer_gbs": round(r["layer_gbs"], 1), "layer_hbm_frac": round(r["layer_hbm_frac"], 4),
            "layer_mfma_frac": round(r["layer_mfma_frac"], 4), "launch": r["launch"],
            "eager_ms_per_step": round(r["eager_ms"], 5),
            "graph_ms_per_step": None if r["graph_ms"] is None else round(r["graph_ms"], 5),
            "sparse_dense_flop_ratio": round(r["acc"]["sparse_dense_flop_ratio"], 5),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in r["kernel_ms"].items()},
            "roofline": roofline(r, peaks)}
        if not args.no_cpu_baseline and name in CPU_SAMPLE:
            entry["cpu_baseline"] = cpu_baseline(name, CPU_SAMPLE[name])
            if name in CPU_ONE_THREAD:
                entry["cpu_baseline_1thread"] = cpu_baseline(name, CPU_ONE_THREAD[name], threads=1)
            log(f"[cpu baseline {name}] {entry['cpu_baseline']}")
        sweep.append(entry)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.config, args.cpu_tokens)
        log(f"[cpu baseline] {cpu}")

    spec = head["spec"]
    line = {
        "metric": METRIC, "value": round(head["rows_per_s"], 1), "unit": "routed rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": path_dtype(spec),
        "data": data_note(spec),
        "config": {"workload": workload_name(spec), "T": spec.T, "d_model": spec.d_model, "d_ff": spec.d_ff,
                   "n_experts": spec.n_experts, "top_k": spec.top_k, "n_shared": spec.n_shared,
                   "routed_rows": spec.T * spec.top_k, "weight_copies_rotated": head["weight_copies"],
                   "weights": weights_note(spec),
                   "launch": head["launch"]},
        "eager_ms_per_step": round(head["eager_ms"], 5),
        "graph_ms_per_step": None if head["graph_ms"] is None else round(head["graph_ms"], 5),
        "tokens_per_s": round(head["tokens_per_s"], 1),
        "layer_roofline": {"algorithmic_bytes": head["acc"]["layer_bytes"], "gbs": round(head["layer_gbs"], 1),
                           "hbm_frac": round(head["layer_hbm_frac"], 4),
                           "expert_flops": head["acc"]["expert_flops"],
                           "mfma_frac": round(head["layer_mfma_frac"], 4),
                           "touched_experts": head["touched"]},
        "sparse_dense_flop_ratio": round(head["acc"]["sparse_dense_flop_ratio"], 5),
        "kernel_us": {k: round(v * 1e3, 2) for k, v in head["kernel_ms"].items()},
        "roofline": roofline(head, peaks),
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

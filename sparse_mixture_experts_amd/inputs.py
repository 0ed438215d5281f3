"""Seeded synthetic inputs for the sparse MoE layer forward.

This module only draws random numbers and stores them in the layer's input
formats (fp32, bf16 or fp16 bits, affine 4- or 8-bit codes with scales and
biases in the 16-bit activation dtype).  It
holds none of the layer's arithmetic; both the GPU tests and the CPU oracle
consume what it returns.

Recipe (the pages fix the shapes, not the draws):
  * NumPy PCG64, one independent stream per part of the layer: x from
    ``[seed, 0, x_index]``, the router from ``[seed, 1]``, expert e (routed
    first, then shared) from ``[seed, 2, e]``; so a layer's weights do not
    depend on T, and the decode layer at T=1 and T=32 shares them.
  * Weights ~ N(0, 1/fan_in) with fan_in = the reduction length (d_model for
    router, gate and up; d_ff for down), drawn in stored (out-major) order:
    gate [d_ff][d_model], up [d_ff][d_model], down [d_model][d_ff].
  * x ~ N(0, 1) except for the tiny fp32 layer, where x ~ N(0, 1/d_model).
  * bf16 storage rounds the fp32 draw to nearest-even (torch's cast); fp16
    storage likewise (NumPy's cast).
  * b-bit affine storage (b = 4 or 8), per group of g (32, 64 or 128)
    consecutive reduction columns of one row: lo = min, hi = max,
    scale = half((hi - lo) / (2^b - 1)), bias = half(lo), half = bf16 or fp16
    (the activation dtype),
    q = clamp(rint((w - bias) / scale), 0, 2^b - 1) (ties to even), q = 0
    where scale == 0.  32/b codes per uint32, code m of a word at bits
    [b*m, b*m + b) holding column (32/b)*word + m.  Codes are stored
    row-major [N][K*b/32]; scales and biases group-major [K/g][N] (the
    scales of one group for consecutive rows are contiguous).
  * Skewed routing: an additive router bias of -2.2 * ln(e + 1) on expert e,
    i.e. twice the log of a Zipf(s = 1.1) weight of rank e + 1 (the Zipf
    normaliser cancels in the softmax).
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    n_shared: int = 0
    act: str = "bf16"            # "f32" | "bf16" | "f16"
    wfmt: str = "dense"          # "dense" | "q4" | "q8" (affine 4- or 8-bit codes)
    group_size: int = 64
    gate_up_fused: bool = False
    glu_round: bool = False
    renormalize: bool = True
    router_bias: str = "none"    # "none" | "zipf"
    x_scale: str = "unit"        # "unit" | "fan_in"
    seed: int = 0
    activation: str = "swiglu"   # "swiglu" | "geglu" (tanh-GELU gate)

    @property
    def quantized(self) -> bool:
        return self.wfmt in ("q4", "q8")

    @property
    def bits(self) -> int:
        return 8 if self.wfmt == "q8" else 4

    @property
    def n_routed_rows(self) -> int:
        return self.T * self.top_k

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)


# The five workloads: shapes, formats and seeds.
CONFIGS = {
    "tiny-f32": LayerSpec("tiny-f32", T=16, d_model=64, d_ff=128, n_experts=8, top_k=2,
                          act="f32", wfmt="dense", x_scale="fan_in", seed=1),
    "dense-bf16-t512": LayerSpec("dense-bf16-t512", T=512, d_model=2048, d_ff=5632, n_experts=8,
                                 top_k=2, act="bf16", wfmt="dense", seed=2),
    "q4-decode-t1": LayerSpec("q4-decode-t1", T=1, d_model=2048, d_ff=768, n_experts=128, top_k=8,
                              wfmt="q4", seed=3),
    "q4-decode-t32": LayerSpec("q4-decode-t32", T=32, d_model=2048, d_ff=768, n_experts=128,
                               top_k=8, wfmt="q4", seed=3),
    "q4-prefill-t2048": LayerSpec("q4-prefill-t2048", T=2048, d_model=2048, d_ff=512, n_experts=512,
                                  top_k=10, wfmt="q4", gate_up_fused=True, glu_round=True,
                                  seed=4),
    "q4-skewed-t256": LayerSpec("q4-skewed-t256", T=256, d_model=2048, d_ff=1408, n_experts=64,
                                top_k=6, n_shared=2, wfmt="q4", router_bias="zipf", seed=5),
}


# The prefill and decode shapes above in the other weight formats and with the
# tanh-GELU GLU (8-bit codes, groups of 32 and 128, fp16 activations):
# measured beside the headline workload and compared with the oracle at full
# size.
VARIANTS = {
    "q8-prefill-t2048": CONFIGS["q4-prefill-t2048"].with_(name="q8-prefill-t2048", wfmt="q8"),
    "q4g32-geglu-prefill-t2048": CONFIGS["q4-prefill-t2048"].with_(name="q4g32-geglu-prefill-t2048",
                                                                   group_size=32, activation="geglu"),
    "q4g128-prefill-t2048": CONFIGS["q4-prefill-t2048"].with_(name="q4g128-prefill-t2048", group_size=128),
    "q8-decode-t1": CONFIGS["q4-decode-t1"].with_(name="q8-decode-t1", wfmt="q8"),
    "q8-decode-t32": CONFIGS["q4-decode-t32"].with_(name="q8-decode-t32", wfmt="q8"),
    # fp16 activations, scales and biases; the per-op GLU rounding is to fp16
    "f16-q4-prefill-t2048": CONFIGS["q4-prefill-t2048"].with_(name="f16-q4-prefill-t2048", act="f16"),
}


def workload(name: str) -> LayerSpec:
    """A named workload: one of CONFIGS or VARIANTS."""
    return CONFIGS[name] if name in CONFIGS else VARIANTS[name]


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(list(key))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even, via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE fp16 bit patterns (uint16), round to nearest even, via NumPy."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_half_bits(a: np.ndarray, half: str) -> np.ndarray:
    """fp32 -> bits of the 16-bit dtype `half` ("bf16" or "f16")."""
    return to_f16_bits(a) if half == "f16" else to_bf16_bits(a)


def half_bits_to_f32(h: np.ndarray, half: str) -> np.ndarray:
    return f16_bits_to_f32(h) if half == "f16" else bf16_bits_to_f32(h)


def quantize_affine(w: np.ndarray, group: int = 64, bits: int = 4, half: str = "bf16"):
    """Encode fp32 rows [N][K] as (uint32 [N][K*bits/32], scales [N][K/g], biases [N][K/g]); scales and
    biases are bits of the 16-bit dtype `half` ("bf16" or "f16")."""
    N, K = w.shape
    per = 32 // bits
    top = float((1 << bits) - 1)
    assert K % group == 0 and group % per == 0
    wg = w.reshape(N, K // group, group).astype(np.float32)
    lo = wg.min(axis=-1)
    hi = wg.max(axis=-1)
    s_bits = to_half_bits((hi - lo) / np.float32(top), half)
    b_bits = to_half_bits(lo, half)
    s = half_bits_to_f32(s_bits, half)[..., None]
    b = half_bits_to_f32(b_bits, half)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((wg - b) / s)
    q = np.where(s == 0, 0.0, np.clip(q, 0, top)).astype(np.uint32).reshape(N, K // per, per)
    words = q[..., 0].copy()
    for m in range(1, per):
        words |= q[..., m] << np.uint32(bits * m)
    return words, s_bits, b_bits


def quantize_q4(w: np.ndarray, group: int = 64):
    """Affine 4-bit encoding of fp32 rows [N][K] (see quantize_affine)."""
    return quantize_affine(w, group, 4)


def gen_x(spec: LayerSpec, x_index: int = 0, T: int | None = None) -> np.ndarray:
    T = spec.T if T is None else T
    std = 1.0 / math.sqrt(spec.d_model) if spec.x_scale == "fan_in" else 1.0
    x = _rng(spec.seed, 0, x_index).standard_normal((T, spec.d_model), dtype=np.float32) * np.float32(std)
    return x if spec.act == "f32" else to_half_bits(x, spec.act)


def gen_router(spec: LayerSpec):
    w = _rng(spec.seed, 1).standard_normal((spec.d_model, spec.n_experts), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(spec.d_model))
    w = w if spec.act == "f32" else to_half_bits(w, spec.act)
    bias = None
    if spec.router_bias == "zipf":
        bias = (-2.2 * np.log(np.arange(1, spec.n_experts + 1, dtype=np.float64))).astype(np.float32)
    return w, bias


def _store(spec: LayerSpec, w: np.ndarray):
    if spec.quantized:
        q, s, b = quantize_affine(w, spec.group_size, spec.bits, spec.act)
        return {"w": q, "scales": np.ascontiguousarray(s.T), "biases": np.ascontiguousarray(b.T)}
    return {"w": w if spec.act == "f32" else to_half_bits(w, spec.act)}


def gen_expert(spec: LayerSpec, e: int) -> dict:
    """Expert e (routed experts first, then shared) in stored form."""
    r = _rng(spec.seed, 2, e)
    D, F = spec.d_model, spec.d_ff
    gate = r.standard_normal((F, D), dtype=np.float32) * np.float32(1.0 / math.sqrt(D))
    up = r.standard_normal((F, D), dtype=np.float32) * np.float32(1.0 / math.sqrt(D))
    down = r.standard_normal((D, F), dtype=np.float32) * np.float32(1.0 / math.sqrt(F))
    out = {"down": _store(spec, down)}
    if spec.gate_up_fused:
        out["gate_up"] = _store(spec, np.concatenate([gate, up], axis=0))
    else:
        out["gate"] = _store(spec, gate)
        out["up"] = _store(spec, up)
    return out


def gen_experts(spec: LayerSpec, workers: int | None = None) -> dict:
    """All experts (routed, then shared) stacked along a leading axis.
    Experts are drawn from independent streams, so they are generated in
    parallel threads with results identical to a sequential loop."""
    n_all = spec.n_experts + spec.n_shared
    first = gen_expert(spec, 0)
    out = {proj: {k: np.empty((n_all,) + v.shape, v.dtype) for k, v in parts.items()}
           for proj, parts in first.items()}

    def fill(e, parts=None):
        parts = parts if parts is not None else gen_expert(spec, e)
        for proj, arrs in parts.items():
            for k, v in arrs.items():
                out[proj][k][e] = v

    fill(0, first)
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(fill, range(1, n_all)))
    return out


def gen_layer(spec: LayerSpec, x_index: int = 0, T: int | None = None) -> dict:
    w_router, bias = gen_router(spec)
    return {"spec": spec, "x": gen_x(spec, x_index, T), "w_router": w_router,
            "router_bias": bias, "experts": gen_experts(spec)}

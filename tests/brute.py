"""NumPy fp64 brute force for small MoE layers (test helper).

An independent restatement of the layer from its definition, used to pin the
CPU oracle: every quantity is computed densely in float64 with NumPy's own
matmul, so it shares no arithmetic path with the oracle's fp32 C loops.
"""
from __future__ import annotations

import numpy as np

from sparse_mixture_experts_amd.inputs import LayerSpec


def bits_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def half_to_f64(spec: LayerSpec, h: np.ndarray) -> np.ndarray:
    """Bits of the layer's 16-bit dtype (bf16, or fp16 for fp16 layers) as float64."""
    return f16_bits_to_f64(h) if spec.act == "f16" else bits_to_f64(h)


def widen(spec: LayerSpec, a: np.ndarray) -> np.ndarray:
    if spec.act == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    return half_to_f64(spec, a)


def unpack_codes(words: np.ndarray, bits: int = 4) -> np.ndarray:
    """uint32 [..., K*b/32] -> codes [..., K] (column (32/b)*w + m is bits [b*m, b*m + b) of word w)."""
    per = 32 // bits
    sh = (np.arange(per, dtype=np.uint32) * bits)
    codes = (words[..., None] >> sh) & np.uint32((1 << bits) - 1)
    return codes.reshape(*words.shape[:-1], words.shape[-1] * per)


def dequant64(spec: LayerSpec, proj: dict) -> np.ndarray:
    if not spec.quantized:
        return widen(spec, proj["w"])
    q = unpack_codes(proj["w"], spec.bits).astype(np.float64)
    g = spec.group_size
    # scales/biases are stored group-major [..., K/g, N]
    s = np.repeat(np.swapaxes(half_to_f64(spec, proj["scales"]), -1, -2), g, axis=-1)
    b = np.repeat(np.swapaxes(half_to_f64(spec, proj["biases"]), -1, -2), g, axis=-1)
    return s * q + b


def weights64(spec: LayerSpec, experts: dict):
    """(gate, up, down) as float64 [n_all][F][D], [n_all][F][D], [n_all][D][F]."""
    F = spec.d_ff
    if spec.gate_up_fused:
        gu = dequant64(spec, experts["gate_up"])
        gate, up = gu[:, :F, :], gu[:, F:, :]
    else:
        gate, up = dequant64(spec, experts["gate"]), dequant64(spec, experts["up"])
    return gate, up, dequant64(spec, experts["down"])


def bf16_round64(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), via float32 first."""
    import torch
    return torch.from_numpy(np.asarray(v, np.float64).astype(np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def f16_round64(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest IEEE binary16 (ties to even), via float32 first."""
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def act_round64(spec: LayerSpec, v: np.ndarray) -> np.ndarray:
    """Per-op rounding of the gated epilogue: to the layer's 16-bit activation dtype."""
    return f16_round64(v) if spec.act == "f16" else bf16_round64(v)


def gelu_tanh64(g: np.ndarray) -> np.ndarray:
    """torch's tanh-approximate GELU in float64 (a library routine, not the oracle's formula)."""
    import torch
    return torch.nn.functional.gelu(torch.from_numpy(np.asarray(g, np.float64)), approximate="tanh").numpy()


def expert_outputs64(spec: LayerSpec, x64: np.ndarray, W) -> np.ndarray:
    """Every expert applied to every token: [T][n_all][D] float64."""
    gate, up, down = W
    g = np.einsum("td,efd->tef", x64, gate)
    u = np.einsum("td,efd->tef", x64, up)
    r = lambda v: act_round64(spec, v)  # noqa: E731
    if spec.activation == "geglu":
        if spec.glu_round:
            g, u = r(g), r(u)
            h = r(r(gelu_tanh64(g)) * u)
        else:
            h = gelu_tanh64(g) * u
    elif spec.glu_round:
        g, u = r(g), r(u)
        s = r(1.0 / (1.0 + np.exp(-g)))
        a = r(g * s)
        h = r(a * u)
    else:
        h = g / (1.0 + np.exp(-g)) * u
    return np.einsum("tef,edf->ted", h, down)


def logits64(spec: LayerSpec, x64: np.ndarray, wr64: np.ndarray, bias) -> np.ndarray:
    l = x64 @ wr64
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def softmax64(l: np.ndarray) -> np.ndarray:
    m = l.max(axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=-1, keepdims=True)


def layer_dense_masked64(spec: LayerSpec, layer: dict, topk_idx: np.ndarray, topk_w: np.ndarray):
    """Dense all-experts output, masked to the given top-k and weighted, plus shared experts."""
    x64 = widen(spec, layer["x"])
    O = expert_outputs64(spec, x64, weights64(spec, layer["experts"]))
    T, E = x64.shape[0], spec.n_experts
    mask = np.zeros((T, E), np.float64)
    np.put_along_axis(mask, topk_idx.astype(np.int64), topk_w.astype(np.float64), axis=1)
    y = np.einsum("te,ted->td", mask, O[:, :E, :])
    if spec.n_shared:
        y = y + O[:, E:, :].sum(axis=1)
    return y


def layer_backward64(spec: LayerSpec, layer: dict, topk_idx: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """dx = dy . dy/dx by torch's autograd in float64 on the dense formulation
    of the layer with the routing held at topk_idx (the unrounded forward)."""
    import torch
    E, K = spec.n_experts, spec.top_k
    x = torch.tensor(widen(spec, layer["x"]), dtype=torch.float64, requires_grad=True)
    wr = torch.tensor(widen(spec, layer["w_router"]), dtype=torch.float64)
    gate, up, down = (torch.tensor(m, dtype=torch.float64) for m in weights64(spec, layer["experts"]))
    logits = x @ wr
    if layer["router_bias"] is not None:
        logits = logits + torch.tensor(np.asarray(layer["router_bias"], np.float64))
    p = torch.softmax(logits, dim=-1)
    idx = torch.tensor(np.asarray(topk_idx, np.int64))
    w = torch.gather(p, 1, idx)
    if spec.renormalize:
        w = w / w.sum(dim=1, keepdim=True)
    act = ((lambda g: torch.nn.functional.gelu(g, approximate="tanh")) if spec.activation == "geglu"
           else torch.nn.functional.silu)
    g = torch.einsum("td,efd->tef", x, gate)
    u = torch.einsum("td,efd->tef", x, up)
    o = torch.einsum("tef,edf->ted", act(g) * u, down)  # every expert on every token
    sel = torch.gather(o[:, :E, :], 1, idx[:, :, None].expand(-1, -1, spec.d_model))
    y = (w[:, :, None] * sel).sum(dim=1) + o[:, E:, :].sum(dim=1)
    (y * torch.tensor(np.asarray(dy, np.float64))).sum().backward()
    return x.grad.numpy()

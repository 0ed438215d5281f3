"""Helpers for the GPU parity tests: upload a generated layer and call the
C-ABI library through the ctypes binding."""
from __future__ import annotations

import math

import numpy as np
import torch

from sparse_mixture_experts_amd import inputs, moe

DEV = "cuda:0"
_TORCH_DT = {moe.MOE_DT_F32: torch.float32, moe.MOE_DT_BF16: torch.bfloat16, moe.MOE_DT_F16: torch.float16}


class GpuLayer:
    """packed: give affine layers the tile-packed copy of their weights, as the
    benchmark does (default), or only the stored layouts (False)."""

    def __init__(self, layer: dict, packed: bool = True):
        self.spec = layer["spec"]
        self.layer = layer
        self.desc = moe.desc_from_spec(self.spec)
        self.x = moe.to_device(layer["x"], DEV)
        self.T = self.x.shape[0]
        self.w = moe.DeviceWeights.from_layer(layer, DEV)
        if packed and self.spec.quantized:
            self.w = self.w.with_packed(self.desc)
            torch.cuda.synchronize()
        self.ws = torch.empty(moe.moe_workspace_size(self.desc, self.T), dtype=torch.uint8, device=DEV)

    @property
    def N(self):
        return self.T * self.spec.top_k

    def route(self):
        idx = torch.empty((self.T, self.spec.top_k), dtype=torch.int32, device=DEV)
        w = torch.empty((self.T, self.spec.top_k), dtype=torch.float32, device=DEV)
        moe.moe_route(self.desc, self.T, self.x, self.w.w_router, self.w.router_bias, idx, w, self.ws)
        torch.cuda.synchronize()
        return idx.cpu().numpy(), w.cpu().numpy()

    def dispatch(self, topk_idx: np.ndarray, tile_rows: int):
        E = self.spec.n_experts
        idx = torch.from_numpy(np.ascontiguousarray(topk_idx, np.int32)).to(DEV)
        T = topk_idx.shape[0]
        N = idx.numel()
        out = {n: torch.full((max(N, 1),), -7, dtype=torch.int32, device=DEV) for n in ("order", "inv_order", "row_map")}
        out["expert_off"] = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
        out["tile_off"] = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
        ws = torch.empty(moe.moe_workspace_size(self.desc, T), dtype=torch.uint8, device=DEV)
        moe.moe_dispatch(self.desc, T, idx, tile_rows, out["order"], out["inv_order"], out["row_map"],
                         out["expert_off"], out["tile_off"], ws)
        torch.cuda.synchronize()
        res = {k: v.cpu().numpy() for k, v in out.items()}
        for k in ("order", "inv_order", "row_map"):
            res[k] = res[k][:N]
        return res

    def expert_ffn(self, row_map: np.ndarray, expert_off: np.ndarray):
        S = self.spec.n_shared
        rows = self.N + S * self.T
        y_sorted = torch.empty((rows, self.spec.d_model), dtype=torch.float32, device=DEV)
        moe.moe_expert_ffn(self.desc, self.T, self.x, torch.from_numpy(row_map).to(DEV),
                           torch.from_numpy(expert_off).to(DEV), self.w, y_sorted, self.ws)
        torch.cuda.synchronize()
        return y_sorted.cpu().numpy()

    def combine(self, y_sorted: np.ndarray, inv_order: np.ndarray, topk_w: np.ndarray, out_dtype=moe.MOE_DT_F32):
        y = torch.empty((self.T, self.spec.d_model), device=DEV,
                        dtype=_TORCH_DT[out_dtype])
        moe.moe_combine(self.desc, self.T, torch.from_numpy(y_sorted).to(DEV), torch.from_numpy(inv_order).to(DEV),
                        torch.from_numpy(np.ascontiguousarray(topk_w)).to(DEV), y, out_dtype)
        torch.cuda.synchronize()
        return y

    def backward(self, dy: np.ndarray) -> np.ndarray:
        """dx (fp32) for the upstream gradient dy [T][d_model] (fp32)."""
        ws = torch.empty(moe.moe_backward_workspace_size(self.desc, self.T), dtype=torch.uint8, device=DEV)
        dyd = torch.from_numpy(np.ascontiguousarray(dy, np.float32)).to(DEV)
        dx = torch.full((self.T, self.spec.d_model), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_backward(self.desc, self.T, self.x, self.w, dyd, dx, ws)
        torch.cuda.synchronize()
        return dx.cpu().numpy()

    def forward(self, out_dtype=moe.MOE_DT_F32, want_routing=True):
        y = torch.empty((self.T, self.spec.d_model), device=DEV,
                        dtype=_TORCH_DT[out_dtype])
        idx = torch.empty((self.T, self.spec.top_k), dtype=torch.int32, device=DEV) if want_routing else None
        w = torch.empty((self.T, self.spec.top_k), dtype=torch.float32, device=DEV) if want_routing else None
        moe.moe_forward(self.desc, self.T, self.x, self.w, y, out_dtype, idx, w, self.ws)
        torch.cuda.synchronize()
        return y, idx, w


def tol_for(spec) -> float:
    """max|y - y_oracle| bound as a fraction of RMS(y_oracle)."""
    return 1e-5 if (spec.act == "f32" and spec.wfmt == "dense") else 2e-2


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    rms = math.sqrt(float(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(y.astype(np.float64) - ref))) / rms


def bf16_rne(a: np.ndarray) -> np.ndarray:
    return inputs.bf16_bits_to_f32(inputs.to_bf16_bits(a))


def f16_rne(a: np.ndarray) -> np.ndarray:
    return inputs.f16_bits_to_f32(inputs.to_f16_bits(a))

"""ctypes binding of the C ABI in include/moe_mi355x.h (libmoe_mi355x.so).

Argument marshalling only: every function below passes device pointers of
torch tensors (or raw integer addresses) and the stream straight to the C
entry point of the same name, raises ``MoeError`` on a negative status and
returns nothing else.  All work happens in the library's HIP kernels; there
is no fallback of any kind, and a missing library raises at load time.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK, MOE_E_INVALID, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP = 0, -1, -2, -3, -4
MOE_DT_F32, MOE_DT_BF16, MOE_DT_F16 = 0, 1, 2
_DT = {"f32": MOE_DT_F32, "bf16": MOE_DT_BF16, "f16": MOE_DT_F16}
MOE_WF_DENSE, MOE_WF_AFFINE_Q4, MOE_WF_AFFINE_Q8 = 0, 1, 2
MOE_ACT_SWIGLU, MOE_ACT_GEGLU = 0, 1
_WFMT = {"dense": MOE_WF_DENSE, "q4": MOE_WF_AFFINE_Q4, "q8": MOE_WF_AFFINE_Q8}
_ACT = {"swiglu": MOE_ACT_SWIGLU, "geglu": MOE_ACT_GEGLU}

EXPORTED = ("moe_workspace_size", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
            "moe_forward", "moe_forward_timed", "moe_backward_workspace_size", "moe_backward",
            "moe_status_string", "moe_forward_noalloc", "moe_packed_bytes", "moe_pack_weights")
MOE_PROJ_GATE, MOE_PROJ_UP, MOE_PROJ_GATE_UP, MOE_PROJ_DOWN = 0, 1, 2, 3
_PROJ = {"gate": MOE_PROJ_GATE, "up": MOE_PROJ_UP, "gate_up": MOE_PROJ_GATE_UP, "down": MOE_PROJ_DOWN}
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024  # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {moe_status_string(status)} ({status})")


class LayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_model", "d_ff", "n_experts", "top_k", "n_shared", "act_dtype", "w_format", "group_size",
        "gate_up_fused", "glu_round", "renormalize", "activation")]


class Proj(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("w_packed", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("gate", Proj),
                ("up", Proj), ("gate_up", Proj), ("down", Proj), ("w_router_packed", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_mixture_experts_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        lib.moe_workspace_size.argtypes = [P(LayerDesc), i32, P(sz)]
        lib.moe_route.argtypes = [P(LayerDesc), i32, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.moe_dispatch.argtypes = [P(LayerDesc), i32, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.moe_expert_ffn.argtypes = [P(LayerDesc), i32, vp, vp, vp, P(Weights), vp, vp, sz, vp]
        lib.moe_combine.argtypes = [P(LayerDesc), i32, vp, vp, vp, vp, i32, vp]
        lib.moe_forward.argtypes = [P(LayerDesc), i32, vp, P(Weights), vp, i32, vp, vp, vp, sz, vp]
        lib.moe_forward_timed.argtypes = [P(LayerDesc), i32, vp, P(Weights), vp, i32, vp, vp, vp, sz, vp,
                                          P(vp), i32, ctypes.c_char_p, sz]
        lib.moe_forward_noalloc.argtypes = [P(LayerDesc), i32, vp, P(Weights), vp, i32, vp, vp, vp]
        lib.moe_backward_workspace_size.argtypes = [P(LayerDesc), i32, P(sz)]
        lib.moe_backward.argtypes = [P(LayerDesc), i32, vp, P(Weights), vp, vp, vp, sz, vp]
        lib.moe_packed_bytes.argtypes = [P(LayerDesc), i32, P(sz)]
        lib.moe_pack_weights.argtypes = [P(LayerDesc), i32, vp, vp, vp, vp, vp]
        lib.moe_stream_read.argtypes = [vp, sz, vp, i32, vp]
        lib.moe_router_packed_bytes.argtypes = [P(LayerDesc), P(sz)]
        lib.moe_pack_router.argtypes = [P(LayerDesc), vp, vp, vp]
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name != "moe_status_string":
                getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def moe_status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def make_desc(d_model, d_ff, n_experts, top_k, n_shared=0, act="bf16", wfmt="dense", group_size=64,
              gate_up_fused=False, glu_round=False, renormalize=True,
              activation="swiglu") -> LayerDesc:
    """act: "f32", "bf16" or "f16"; wfmt: "dense", "q4" or "q8" (affine 4-/8-bit codes); activation:
    "swiglu" or "geglu"."""
    return LayerDesc(d_model, d_ff, n_experts, top_k, n_shared,
                     _DT[act],
                     _WFMT[wfmt], group_size,
                     int(gate_up_fused), int(glu_round), int(renormalize), _ACT[activation])


def desc_from_spec(spec) -> LayerDesc:
    return make_desc(spec.d_model, spec.d_ff, spec.n_experts, spec.top_k, spec.n_shared, spec.act,
                     spec.wfmt, spec.group_size, spec.gate_up_fused, spec.glu_round,
                     spec.renormalize, spec.activation)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise ValueError("tensors passed to the MoE library must be contiguous")
        return t.data_ptr()
    raise TypeError(f"expected a torch tensor, an int address or None, got {type(t)}")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _nbytes(ws):
    if ws is None:
        return 0
    if isinstance(ws, torch.Tensor):
        return ws.numel() * ws.element_size()
    raise TypeError("workspace must be a torch tensor")


def _check(status: int, fn: str):
    if status != MOE_OK:
        raise MoeError(status, fn)


def moe_workspace_size(desc: LayerDesc, T: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(desc), T, ctypes.byref(out)), "moe_workspace_size")
    return out.value


def moe_route(desc, T, x, w_router, router_bias, topk_idx, topk_w, ws, stream=None):
    _check(load().moe_route(ctypes.byref(desc), T, _ptr(x), _ptr(w_router), _ptr(router_bias),
                            _ptr(topk_idx), _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream)), "moe_route")


def moe_dispatch(desc, T, topk_idx, tile_rows, order, inv_order, row_map, expert_off, tile_off, ws,
                 stream=None):
    _check(load().moe_dispatch(ctypes.byref(desc), T, _ptr(topk_idx), tile_rows, _ptr(order),
                               _ptr(inv_order), _ptr(row_map), _ptr(expert_off), _ptr(tile_off),
                               _ptr(ws), _nbytes(ws), _stream(stream)), "moe_dispatch")


def moe_expert_ffn(desc, T, x, row_map, expert_off, weights, y_sorted, ws, stream=None):
    _check(load().moe_expert_ffn(ctypes.byref(desc), T, _ptr(x), _ptr(row_map), _ptr(expert_off),
                                 ctypes.byref(weights.c), _ptr(y_sorted), _ptr(ws), _nbytes(ws),
                                 _stream(stream)), "moe_expert_ffn")


def moe_combine(desc, T, y_sorted, inv_order, topk_w, y, out_dtype, stream=None):
    _check(load().moe_combine(ctypes.byref(desc), T, _ptr(y_sorted), _ptr(inv_order), _ptr(topk_w),
                              _ptr(y), out_dtype, _stream(stream)), "moe_combine")


def moe_forward(desc, T, x, weights, y, out_dtype, topk_idx_out, topk_w_out, ws, stream=None):
    _check(load().moe_forward(ctypes.byref(desc), T, _ptr(x), ctypes.byref(weights.c), _ptr(y), out_dtype,
                              _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), _nbytes(ws),
                              _stream(stream)), "moe_forward")


def moe_forward_noalloc(desc, T, x, weights, y, out_dtype, topk_idx_out, topk_w_out, stream=None):
    _check(load().moe_forward_noalloc(ctypes.byref(desc), T, _ptr(x), ctypes.byref(weights.c), _ptr(y), out_dtype,
                                      _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream)), "moe_forward_noalloc")


def moe_pack_router(desc, w_router, out, stream=None):
    """The prepared router of w_router into out (moe_router_packed_bytes bytes)."""
    _check(load().moe_pack_router(ctypes.byref(desc), _ptr(w_router), _ptr(out), _stream(stream)), "moe_pack_router")


def moe_stream_read(src, nbytes, out, blocks, stream=None):
    """The library's plain streaming read of nbytes of src (a measurement
    kernel outside the layer); out holds blocks * 256 uint32 words."""
    _check(load().moe_stream_read(_ptr(src), nbytes, _ptr(out), blocks, _stream(stream)), "moe_stream_read")


def moe_forward_timed(desc, T, x, weights, y, out_dtype, topk_idx_out, topk_w_out, ws, events, stream=None):
    """moe_forward with kernel i launched between events[2i] and events[2i+1]
    (raw hipEvent_t handles: its start and its end); returns one stage name
    per kernel, in launch order."""
    arr = (ctypes.c_void_p * len(events))(*events)
    names = ctypes.create_string_buffer(512)
    _check(load().moe_forward_timed(ctypes.byref(desc), T, _ptr(x), ctypes.byref(weights.c), _ptr(y), out_dtype,
                                    _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), _nbytes(ws), _stream(stream),
                                    arr, len(events), names, 512), "moe_forward_timed")
    return names.value.decode().split(",") if names.value else []


def moe_backward_workspace_size(desc: LayerDesc, T: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().moe_backward_workspace_size(ctypes.byref(desc), T, ctypes.byref(out)), "moe_backward_workspace_size")
    return out.value


def moe_backward(desc, T, x, weights, dy, dx, ws, stream=None):
    """dx[T][d_model] (fp32) = dy . dy/dx of the layer forward at x (dy fp32)."""
    _check(load().moe_backward(ctypes.byref(desc), T, _ptr(x), ctypes.byref(weights.c), _ptr(dy), _ptr(dx),
                               _ptr(ws), _nbytes(ws), _stream(stream)), "moe_backward")


def moe_packed_bytes(desc: LayerDesc, proj: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().moe_packed_bytes(ctypes.byref(desc), proj, ctypes.byref(out)), "moe_packed_bytes")
    return out.value


def moe_pack_weights(desc, proj: int, w, scales, biases, w_packed, stream=None):
    """Enqueue the tile-packed copy of projection `proj` (codes `w`, `scales`,
    `biases`) into `w_packed` (moe_packed_bytes bytes)."""
    _check(load().moe_pack_weights(ctypes.byref(desc), proj, _ptr(w), _ptr(scales), _ptr(biases), _ptr(w_packed),
                                   _stream(stream)), "moe_pack_weights")


# ---- marshalling helpers ----------------------------------------------------

def to_device(a: np.ndarray, device) -> torch.Tensor:
    """A NumPy array as a device tensor with the matching element size
    (uint16 bits of a 16-bit dtype -> a torch.bfloat16 tensor holding them;
    the library reads them by the layer's dtype; uint32 codes -> torch.int32)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    return torch.from_numpy(a).to(device)


class DeviceWeights:
    """Device copies of a layer's weights plus the C weight table pointing at them."""

    def __init__(self, w_router: torch.Tensor, router_bias, experts: dict, router_packed=None):
        self.w_router, self.router_bias, self.experts = w_router, router_bias, experts
        self.router_packed = router_packed

        def proj(name):
            p = experts.get(name)
            if p is None:
                return Proj(None, None, None)
            return Proj(_ptr(p["w"]), _ptr(p.get("scales")), _ptr(p.get("biases")), _ptr(p.get("w_packed")))

        self.c = Weights(_ptr(w_router), _ptr(router_bias), proj("gate"), proj("up"), proj("gate_up"),
                         proj("down"), _ptr(router_packed))

    @classmethod
    def from_layer(cls, layer: dict, device="cuda") -> "DeviceWeights":
        experts = {name: {k: to_device(v, device) for k, v in p.items()} for name, p in layer["experts"].items()}
        bias = None if layer["router_bias"] is None else to_device(layer["router_bias"], device)
        return cls(to_device(layer["w_router"], device), bias, experts)

    def with_packed(self, desc: LayerDesc, stream=None) -> "DeviceWeights":
        """The same weights plus the tile-packed copy of every affine projection
        (moe_pack_weights), which the grouped kernels then read, and the
        prepared router (moe_pack_router) where the layer can use one."""
        return self.with_packed_experts(desc, stream).with_packed_router(desc, stream)

    def with_packed_router(self, desc: LayerDesc, stream=None) -> "DeviceWeights":
        """The same weights plus the prepared router, or as they are when the
        layer's router takes none."""
        n = ctypes.c_size_t(0)
        if load().moe_router_packed_bytes(ctypes.byref(desc), ctypes.byref(n)) != MOE_OK:
            return self
        packed = torch.empty((n.value,), dtype=torch.uint8, device=self.w_router.device)
        moe_pack_router(desc, self.w_router, packed, stream)
        return DeviceWeights(self.w_router, self.router_bias, self.experts, packed)

    def with_packed_experts(self, desc: LayerDesc, stream=None) -> "DeviceWeights":
        """The same weights plus the tile-packed copy of every affine projection."""
        experts = {}
        for name, p in self.experts.items():
            q = dict(p)
            q.pop("w_packed", None)
            n = moe_packed_bytes(desc, _PROJ[name])
            q["w_packed"] = torch.empty((n,), dtype=torch.uint8, device=p["w"].device)
            moe_pack_weights(desc, _PROJ[name], p["w"], p["scales"], p["biases"], q["w_packed"], stream)
            experts[name] = q
        return DeviceWeights(self.w_router, self.router_bias, experts, self.router_packed)

    def clone(self) -> "DeviceWeights":
        """A byte-identical copy at new device addresses."""
        experts = {n: {k: v.clone() for k, v in p.items()} for n, p in self.experts.items()}
        bias = None if self.router_bias is None else self.router_bias.clone()
        rp = None if self.router_packed is None else self.router_packed.clone()
        return DeviceWeights(self.w_router.clone(), bias, experts, rp)

    def nbytes(self, experts=None) -> int:
        """Bytes held for all weights, or for the listed expert ids only (a
        packed copy counted in proportion)."""
        total = 0
        for p in self.experts.values():
            m = p["w"].shape[0]
            for k, v in p.items():
                size = v.numel() * v.element_size()
                if k == "w_packed":  # one flat buffer for all m matrices
                    total += size if experts is None else size * len(experts) // m
                    continue
                per = size // v.shape[0]
                total += per * (v.shape[0] if experts is None else len(experts))
        return total

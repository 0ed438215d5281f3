"""CPU oracle for the sparse MoE layer forward (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
fp32, explicit dequantisation, no sorting or tiling in the output path) with
ctypes and NumPy arrays.  It never imports the GPU package, and the GPU
package never imports it.

Arrays: activations and dense weights are ``float32`` or ``uint16`` holding
bf16 (or, with ``act_f16``, fp16) bits; affine weights are ``uint32`` words
with 32/b b-bit codes each (code m of a word sits at bits [b*m, b*m+b)),
scales/biases ``uint16`` bits of the 16-bit activation dtype stored
group-major ([..][K/g][N]).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

BUILD_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", "-o", _LIB_PATH, _SRC, "-lm"]


def build() -> str:
    """Compile the oracle library in place (always recompiles)."""
    subprocess.run(BUILD_CMD, check=True, cwd=_HERE)
    return _LIB_PATH


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_model", "d_ff", "n_experts", "top_k", "n_shared", "act_bf16", "w_q4",
        "group_size", "gate_up_fused", "glu_round", "renormalize", "w_bits", "activation", "act_f16")]


class _Proj(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class _Experts(ctypes.Structure):
    _fields_ = [("gate", _Proj), ("up", _Proj), ("gate_up", _Proj), ("down", _Proj)]


_lib = None


def _open(path: str):
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_router_logits.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.oracle_route.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    lib.oracle_dispatch.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp, vp, vp]
    lib.oracle_dequant_row.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    lib.oracle_expert_apply.argtypes = [vp, vp, i32, vp, vp, vp]
    lib.oracle_forward_tokens.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32]
    lib.oracle_backward_tokens.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, i32]
    lib.oracle_last_threads.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _open(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call to another build of moe_oracle.c
    (the tests use this to check that planted mistakes fail the pins)."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


@dataclass(frozen=True)
class Desc:
    """Layer description, mirroring the oracle's C struct."""
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    n_shared: int = 0
    act_bf16: bool = False
    w_q4: bool = False
    group_size: int = 64
    gate_up_fused: bool = False
    glu_round: bool = False
    renormalize: bool = True
    w_bits: int = 4           # affine code width (4 or 8) when w_q4
    activation: int = 0       # 0: SwiGLU, 1: GeGLU (tanh-GELU)
    act_f16: bool = False     # fp16 activations, dense weights and scales/biases (act_bf16 False)

    @property
    def half(self) -> bool:
        return self.act_bf16 or self.act_f16

    def _c(self) -> _Desc:
        return _Desc(self.d_model, self.d_ff, self.n_experts, self.top_k, self.n_shared,
                     int(self.act_bf16), int(self.w_q4), self.group_size,
                     int(self.gate_up_fused), int(self.glu_round), int(self.renormalize),
                     int(self.w_bits), int(self.activation), int(self.act_f16))


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _act(desc: Desc, a):
    a = np.ascontiguousarray(a)
    want = np.uint16 if desc.half else np.float32
    assert a.dtype == want, f"activation array must be {want}, got {a.dtype}"
    return a


def _experts(desc: Desc, w: dict):
    """Build the C struct; returns (struct, keep-alive list)."""
    keep = []

    def proj(name):
        if name not in w or w[name] is None:
            return _Proj(None, None, None)
        p = w[name]
        arrs = [np.ascontiguousarray(p["w"]), p.get("scales"), p.get("biases")]
        arrs = [None if a is None else np.ascontiguousarray(a) for a in arrs]
        if desc.w_q4:
            assert arrs[0].dtype == np.uint32 and arrs[1].dtype == np.uint16 and arrs[2].dtype == np.uint16
        else:
            assert arrs[0].dtype == (np.uint16 if desc.half else np.float32)
        keep.extend(a for a in arrs if a is not None)
        return _Proj(*[_ptr(a) for a in arrs])

    s = _Experts(proj("gate"), proj("up"), proj("gate_up"), proj("down"))
    return s, keep


def bf16_to_f32(h: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(h)))


def f32_to_bf16(f: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(f)))


def f16_to_f32(h: int) -> float:
    return float(_load().oracle_f16_to_f32(int(h)))


def f32_to_f16(f: float) -> int:
    return int(_load().oracle_f32_to_f16(float(f)))


def router_logits(desc: Desc, x, w_router, router_bias=None) -> np.ndarray:
    lib = _load()
    x, w_router = _act(desc, x), _act(desc, w_router)
    T = x.shape[0]
    bias = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    out = np.empty((T, desc.n_experts), np.float32)
    lib.oracle_router_logits(ctypes.byref(desc._c()), T, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(out))
    return out


def route(desc: Desc, x, w_router, router_bias=None):
    lib = _load()
    x, w_router = _act(desc, x), _act(desc, w_router)
    T = x.shape[0]
    bias = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    idx = np.empty((T, desc.top_k), np.int32)
    w = np.empty((T, desc.top_k), np.float32)
    lib.oracle_route(ctypes.byref(desc._c()), T, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(idx), _ptr(w))
    return idx, w


def dispatch(topk_idx, n_experts: int, tile_rows: int) -> dict:
    lib = _load()
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    N = T * k
    out = {n: np.empty(N, np.int32) for n in ("order", "inv_order", "row_map")}
    out["expert_off"] = np.empty(n_experts + 1, np.int32)
    out["tile_off"] = np.empty(n_experts + 1, np.int32)
    lib.oracle_dispatch(T, k, n_experts, _ptr(idx), tile_rows, _ptr(out["order"]), _ptr(out["inv_order"]),
                        _ptr(out["row_map"]), _ptr(out["expert_off"]), _ptr(out["tile_off"]))
    return out


def dequant_row(desc: Desc, proj: dict, e: int, n: int, N: int, K: int) -> np.ndarray:
    lib = _load()
    s, keep = _experts(desc, {"gate": proj})
    out = np.empty(K, np.float32)
    lib.oracle_dequant_row(ctypes.byref(desc._c()), ctypes.byref(s.gate), e, n, N, K, _ptr(out))
    del keep
    return out


def expert_apply(desc: Desc, weights: dict, e: int, x_row):
    lib = _load()
    s, keep = _experts(desc, weights)
    x_row = _act(desc, x_row)
    h = np.empty(desc.d_ff, np.float32)
    out = np.empty(desc.d_model, np.float32)
    lib.oracle_expert_apply(ctypes.byref(desc._c()), ctypes.byref(s), e, _ptr(x_row), _ptr(h), _ptr(out))
    del keep
    return h, out


def forward(desc: Desc, x, w_router, router_bias, weights: dict, tokens=None, n_threads: int = 0):
    """Layer forward for `tokens` (default: all).  Returns (y f32, topk_idx, topk_w, threads_used)."""
    lib = _load()
    x, w_router = _act(desc, x), _act(desc, w_router)
    T = x.shape[0]
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    bias = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    s, keep = _experts(desc, weights)
    n = toks.shape[0]
    y = np.empty((n, desc.d_model), np.float32)
    idx = np.empty((n, desc.top_k), np.int32)
    w = np.empty((n, desc.top_k), np.float32)
    lib.oracle_forward_tokens(ctypes.byref(desc._c()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                              ctypes.byref(s), n, _ptr(toks), _ptr(y), _ptr(idx), _ptr(w), n_threads)
    del keep
    return y, idx, w, int(lib.oracle_last_threads())


def backward(desc: Desc, x, w_router, router_bias, weights: dict, dy, tokens=None, n_threads: int = 0):
    """dx = dy . dy/dx for `tokens` (default: all); dy is fp32 [n_tok][d_model]
    with row r for tokens[r].  Returns (dx f32, threads_used)."""
    lib = _load()
    x, w_router = _act(desc, x), _act(desc, w_router)
    T = x.shape[0]
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    bias = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    n = toks.shape[0]
    assert dy.shape == (n, desc.d_model)
    s, keep = _experts(desc, weights)
    dx = np.empty((n, desc.d_model), np.float32)
    lib.oracle_backward_tokens(ctypes.byref(desc._c()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                               ctypes.byref(s), n, _ptr(toks), _ptr(dy), _ptr(dx), n_threads)
    del keep
    return dx, int(lib.oracle_last_threads())

"""C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side validation rejects bad calls before touching the GPU.

No compute call happens here: every call either fails validation (returns a
negative status, enqueues nothing) or has T == 0 (valid, enqueues nothing).
"""
import ctypes
import glob
import os
import re

import pytest

from sparse_mixture_experts_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 1 << 20  # a fake, 16-byte aligned device address; never dereferenced here


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(moe_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from sparse_mixture_experts_amd import build
        build.build(verbose=False)
    return moe.load()


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert set(moe.EXPORTED) <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def good():
    return moe.make_desc(2048, 768, 128, 8, wfmt="q4")


def weights():
    p = moe.Proj(A, A, A)
    return moe.Weights(A, None, p, p, moe.Proj(None, None, None), p)


def ws_size(d, T):
    return moe.moe_workspace_size(d, T)


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert moe.moe_status_string(s)
    assert "unknown" in moe.moe_status_string(7)


@pytest.mark.parametrize("field,value,status", [
    ("d_model", 0, moe.MOE_E_INVALID), ("d_model", 100, moe.MOE_E_INVALID),
    ("d_ff", 96, moe.MOE_E_INVALID), ("n_experts", 0, moe.MOE_E_INVALID),
    ("n_experts", 1025, moe.MOE_E_INVALID), ("top_k", 0, moe.MOE_E_INVALID),
    ("top_k", 33, moe.MOE_E_INVALID), ("n_shared", -1, moe.MOE_E_INVALID),
    ("n_shared", 9, moe.MOE_E_INVALID), ("act_dtype", 5, moe.MOE_E_INVALID),
    ("w_format", 3, moe.MOE_E_INVALID), ("group_size", 16, moe.MOE_E_UNSUPPORTED),
    ("group_size", 96, moe.MOE_E_UNSUPPORTED), ("group_size", 256, moe.MOE_E_UNSUPPORTED),
    ("act_dtype", moe.MOE_DT_F32, moe.MOE_E_UNSUPPORTED),
    ("renormalize", 2, moe.MOE_E_INVALID), ("gate_up_fused", -1, moe.MOE_E_INVALID),
    ("activation", 2, moe.MOE_E_INVALID), ("activation", -1, moe.MOE_E_INVALID),
])
def test_descriptor_validation(lib, field, value, status):
    d = good()
    setattr(d, field, value)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(d, 4)
    assert ei.value.status == status
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(d, 4, A, A, None, A, A, None, stream=0)
    assert ei.value.status == status


def test_affine_formats_and_groups(lib):
    size = ctypes.c_size_t()
    for wfmt in ("q4", "q8"):
        for g in (32, 64, 128):
            d = moe.make_desc(2048, 768, 128, 8, wfmt=wfmt, group_size=g, activation="geglu")
            assert lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(size)) == moe.MOE_OK
    # the group must divide both reduction lengths
    d = moe.make_desc(2048, 192, 128, 8, wfmt="q8", group_size=128)
    assert lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(size)) == moe.MOE_E_INVALID
    # the affine formats feed 16-bit activations only
    d = moe.make_desc(2048, 768, 128, 8, act="f32", wfmt="q8")
    assert lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(size)) == moe.MOE_E_UNSUPPORTED
    for act in ("bf16", "f16"):
        d = moe.make_desc(2048, 768, 128, 8, act=act, wfmt="q4")
        assert lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(size)) == moe.MOE_OK
    # per-op GLU rounding goes to the 16-bit activation dtype: bf16 or fp16
    for act in ("bf16", "f16"):
        d = moe.make_desc(256, 128, 8, 2, act=act, glu_round=True)
        assert lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(size)) == moe.MOE_OK


def test_backward_validation(lib):
    d = good()
    size = ctypes.c_size_t()
    assert lib.moe_backward_workspace_size(ctypes.byref(d), 4, ctypes.byref(size)) == moe.MOE_OK
    fwd = ctypes.c_size_t()
    lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(fwd))
    assert size.value > fwd.value
    w = weights()
    bad = [(None, A, A), (A, None, A), (A, A, None), (A + 4, A, A)]
    for x, dy, dx in bad:
        assert lib.moe_backward(ctypes.byref(d), 4, x, ctypes.byref(w), dy, dx, A, size.value, None) == \
            moe.MOE_E_INVALID
    assert lib.moe_backward(ctypes.byref(d), 4, A, ctypes.byref(w), A, A, A, size.value - 1, None) == \
        moe.MOE_E_WORKSPACE


def test_top_k_above_experts_and_rounding_needs_16bit(lib):
    d = moe.make_desc(64, 64, 4, 5, act="f32")
    assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(ctypes.c_size_t())) == moe.MOE_E_INVALID
    d = moe.make_desc(64, 64, 4, 2, act="f32", glu_round=True)
    assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(ctypes.c_size_t())) == moe.MOE_E_INVALID


def test_pointer_and_size_validation(lib):
    d = good()
    st = lambda f: pytest.raises(moe.MoeError)  # noqa: E731
    with st(0):
        moe.moe_route(d, -1, A, A, None, A, A, None, stream=0)
    with st(0):
        moe.moe_route(d, 4, None, A, None, A, A, None, stream=0)
    with st(0):
        moe.moe_route(d, 4, A + 4, A, None, A, A, None, stream=0)  # misaligned
    with st(0):
        moe.moe_combine(d, 4, A, A, A, A, 7, stream=0)  # bad out dtype
    with st(0):
        moe.moe_dispatch(d, 4, A, 0, A, A, A, A, A, None, stream=0)  # tile_rows 0


def test_workspace_checks(lib):
    d = good()
    need = ws_size(d, 32)
    assert need >= ws_size(d, 1) > 0
    assert ws_size(d, 0) >= 0
    r = lib.moe_forward(ctypes.byref(d), 32, A, ctypes.byref(weights()), A, 0, None, None, A, need - 1, None)
    assert r == moe.MOE_E_WORKSPACE
    r = lib.moe_expert_ffn(ctypes.byref(d), 32, A, A, A, ctypes.byref(weights()), A, A, 16, None)
    assert r == moe.MOE_E_WORKSPACE
    bad_w = weights()
    bad_w.down = moe.Proj(A, None, A)  # q4 needs scales
    r = lib.moe_forward(ctypes.byref(d), 32, A, ctypes.byref(bad_w), A, 0, None, None, A, need, None)
    assert r == moe.MOE_E_INVALID


def test_zero_tokens_is_a_no_op(lib):
    d = good()
    need = ws_size(d, 0)
    assert lib.moe_route(ctypes.byref(d), 0, A, A, None, A, A, A, need, None) == moe.MOE_OK
    assert lib.moe_dispatch(ctypes.byref(d), 0, A, 64, A, A, A, A, A, A, need, None) == moe.MOE_OK
    assert lib.moe_expert_ffn(ctypes.byref(d), 0, A, A, A, ctypes.byref(weights()), A, A, need, None) == 0
    assert lib.moe_combine(ctypes.byref(d), 0, A, A, A, A, 0, None) == moe.MOE_OK
    assert lib.moe_forward(ctypes.byref(d), 0, A, ctypes.byref(weights()), A, 1, None, None, A, need,
                           None) == moe.MOE_OK


@pytest.mark.parametrize("shape", [
    dict(d_model=2048, d_ff=5632, n_experts=8, top_k=2),                        # dense: split down reductions
    dict(d_model=2048, d_ff=768, n_experts=128, top_k=8, wfmt="q4"),            # decode tiles, then 16-row tiles
    dict(d_model=2048, d_ff=512, n_experts=512, top_k=10, wfmt="q4"),           # prefill shape
    dict(d_model=2048, d_ff=1408, n_experts=64, top_k=6, n_shared=2, wfmt="q4"),
    dict(d_model=256, d_ff=2624, n_experts=4, top_k=2, act="f16"),
    dict(d_model=64, d_ff=128, n_experts=8, top_k=2, act="f32"),
])
def test_workspace_covers_smaller_T(shape):
    """The header promises that the workspace for T tokens also serves every
    smaller T: the size must not decrease as T grows, although the layout of
    the expert outputs changes with T (fp32 rows on decode tiles, fp16 rows
    with exponents on the 64- and 16-row tiles, fp32 partial rows when the
    down reduction is split)."""
    desc = moe.make_desc(**shape)
    prev = 0
    for T in range(0, 2200):
        size = moe.moe_workspace_size(desc, T)
        assert size >= prev, (T, size, prev)
        prev = size


def _packed_size(M, N, K, bits, group):
    """The documented regions, each rounded up to 256 bytes: codes
    [M][N/16][slabs][16][SW] words, fp16 scales [M][N/16][slabs][16][128/group],
    fp16 group terms [M][N/16][16][G rounded up to 32], int32 flags [M]."""
    up = lambda n: (n + 255) // 256 * 256  # noqa: E731
    slabs = -(-K // 128)
    G = K // group
    return (up(M * N * slabs * (128 * bits // 32) * 4) + up(M * N * slabs * (128 // group) * 2)
            + up(M * N * (-(-G // 32) * 32) * 2) + up(M * 4))


def test_packed_bytes_and_validation(lib):
    size = ctypes.c_size_t()
    d = moe.make_desc(2048, 768, 128, 8, n_shared=2, wfmt="q4")
    assert lib.moe_packed_bytes(ctypes.byref(d), moe.MOE_PROJ_GATE, ctypes.byref(size)) == moe.MOE_OK
    assert size.value == _packed_size(130, 768, 2048, 4, 64) == 115016448
    assert lib.moe_packed_bytes(ctypes.byref(d), moe.MOE_PROJ_DOWN, ctypes.byref(size)) == moe.MOE_OK
    assert size.value == _packed_size(130, 2048, 768, 4, 64)
    # 8-bit codes, a reduction of 64 mod 128 padded to a whole slab, fp16
    d8 = moe.make_desc(320, 192, 4, 2, act="f16", wfmt="q8", group_size=32, gate_up_fused=True)
    assert lib.moe_packed_bytes(ctypes.byref(d8), moe.MOE_PROJ_GATE_UP, ctypes.byref(size)) == moe.MOE_OK
    assert size.value == _packed_size(4, 384, 320, 8, 32)
    # a projection the layer does not use, dense weights, bad arguments
    assert lib.moe_packed_bytes(ctypes.byref(d), moe.MOE_PROJ_GATE_UP, ctypes.byref(size)) == moe.MOE_E_INVALID
    assert lib.moe_packed_bytes(ctypes.byref(d), 7, ctypes.byref(size)) == moe.MOE_E_INVALID
    dd = moe.make_desc(2048, 768, 128, 8)
    assert lib.moe_packed_bytes(ctypes.byref(dd), moe.MOE_PROJ_DOWN, ctypes.byref(size)) == moe.MOE_E_UNSUPPORTED
    assert lib.moe_pack_weights(ctypes.byref(d), moe.MOE_PROJ_DOWN, A + 4, A, A, A, None) == moe.MOE_E_INVALID
    assert lib.moe_pack_weights(ctypes.byref(d), moe.MOE_PROJ_DOWN, A, A, A, None, None) == moe.MOE_E_INVALID
    assert lib.moe_pack_weights(ctypes.byref(d), moe.MOE_PROJ_DOWN, A, None, A, A, None) == moe.MOE_E_INVALID
    assert lib.moe_pack_weights(ctypes.byref(d), moe.MOE_PROJ_DOWN, A, A, A + 8, A, None) == moe.MOE_E_INVALID
    # a packed copy on a dense layer, or misaligned, is refused before anything runs
    w = weights()
    w.down = moe.Proj(A, None, None, A)
    need = ws_size(dd, 0)
    assert lib.moe_forward(ctypes.byref(dd), 0, A, ctypes.byref(w), A, 1, None, None, A, need, None) == \
        moe.MOE_E_INVALID
    w = weights()
    w.down = moe.Proj(A, A, A, A + 4)
    assert lib.moe_forward(ctypes.byref(d), 0, A, ctypes.byref(w), A, 1, None, None, A, ws_size(d, 0), None) == \
        moe.MOE_E_INVALID


def test_stream_read_validation(lib):
    # every case is rejected on the host before any launch
    bad = moe.MOE_E_INVALID
    assert lib.moe_stream_read(None, 16, ctypes.c_void_p(64), 1, None) == bad
    assert lib.moe_stream_read(ctypes.c_void_p(64), 16, None, 1, None) == bad
    assert lib.moe_stream_read(ctypes.c_void_p(64), 0, ctypes.c_void_p(64), 1, None) == bad
    assert lib.moe_stream_read(ctypes.c_void_p(64), 24, ctypes.c_void_p(64), 1, None) == bad
    assert lib.moe_stream_read(ctypes.c_void_p(72), 16, ctypes.c_void_p(64), 1, None) == bad
    assert lib.moe_stream_read(ctypes.c_void_p(64), 16, ctypes.c_void_p(64), 0, None) == bad
    assert lib.moe_stream_read(ctypes.c_void_p(64), 16, ctypes.c_void_p(64), 65537, None) == bad


def test_router_packed_bytes_and_validation(lib):
    size = ctypes.c_size_t()
    d = moe.make_desc(2048, 512, 512, 10, wfmt="q4")
    assert lib.moe_router_packed_bytes(ctypes.byref(d), ctypes.byref(size)) == moe.MOE_OK
    wt = 512 * 2048 * 2                                    # [E][d] 16-bit, a multiple of 256 bytes here
    assert size.value == wt + (2048 // 256 + 1) * 512 * 4  # norm partials [d/256][E] and their sums [E]
    d6 = moe.make_desc(320, 128, 6, 2, act="f16")          # 6*320*2 = 3840 bytes (15 * 256), 2 partial rows
    assert lib.moe_router_packed_bytes(ctypes.byref(d6), ctypes.byref(size)) == moe.MOE_OK
    assert size.value == 3840 + 3 * 6 * 4
    d32 = moe.make_desc(64, 128, 8, 2, act="f32")
    assert lib.moe_router_packed_bytes(ctypes.byref(d32), ctypes.byref(size)) == moe.MOE_E_UNSUPPORTED
    assert lib.moe_pack_router(ctypes.byref(d), None, A, None) == moe.MOE_E_INVALID
    assert lib.moe_pack_router(ctypes.byref(d), A, A + 4, None) == moe.MOE_E_INVALID
    # a prepared router where the layer's router takes none, or misaligned
    w = moe.Weights(A, None, moe.Proj(A, None, None), moe.Proj(A, None, None), moe.Proj(None, None, None),
                    moe.Proj(A, None, None), A)
    need = ws_size(d32, 0)
    assert lib.moe_forward(ctypes.byref(d32), 0, A, ctypes.byref(w), A, 0, None, None, A, need, None) == \
        moe.MOE_E_INVALID
    w = weights()
    w.w_router_packed = A + 8
    assert lib.moe_forward(ctypes.byref(d), 0, A, ctypes.byref(w), A, 1, None, None, A, ws_size(d, 0), None) == \
        moe.MOE_E_INVALID
    w.w_router_packed = A
    assert lib.moe_forward(ctypes.byref(d), 0, A, ctypes.byref(w), A, 1, None, None, A, ws_size(d, 0), None) == \
        moe.MOE_OK

"""The tile-packed copy of the affine codes (moe_pack_weights) through the C
ABI: its bytes follow the documented layout, and the forward and backward
that read it give bit for bit the results of the stored layout (the same
bytes in another order), on every kernel family that reads it (64- and
16-row grouped tiles, the resident-h down projection, split down
reductions) and on the paths that keep reading the stored codes (decode
tiles, the one-token kernels)."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_amd import inputs, moe
from sparse_mixture_experts_amd.inputs import LayerSpec
from gpu_util import GpuLayer

pytestmark = pytest.mark.gpu

CASES = {
    # 64-row tiles, separate gate/up, resident down
    "pk-q4": LayerSpec("pk-q4", T=96, d_model=256, d_ff=256, n_experts=4, top_k=2, wfmt="q4", seed=80),
    # fused gate|up with rounding, 16-row tiles, a shared expert
    "pk-q4-fused-tile16": LayerSpec("pk-q4-fused-tile16", T=40, d_model=256, d_ff=128, n_experts=16, top_k=2,
                                    n_shared=1, wfmt="q4", gate_up_fused=True, glu_round=True, seed=81),
    # 8-bit, groups of 32, reductions of 64 mod 128 (d_model 320, d_ff 192)
    "pk-q8-g32-ragged": LayerSpec("pk-q8-g32-ragged", T=80, d_model=320, d_ff=192, n_experts=4, top_k=2,
                                  wfmt="q8", group_size=32, seed=82),
    # a long down reduction over few tiles: the grouped down kernel in parts
    "pk-q4-long-down": LayerSpec("pk-q4-long-down", T=8, d_model=256, d_ff=2048, n_experts=8, top_k=2,
                                 n_shared=1, wfmt="q4", gate_up_fused=True, seed=83),
    # fp16 activations, groups of 128, GeGLU
    "pk-f16-q4-g128-geglu": LayerSpec("pk-f16-q4-g128-geglu", T=64, d_model=256, d_ff=256, n_experts=8, top_k=2,
                                      act="f16", wfmt="q4", group_size=128, activation="geglu", seed=84),
    # decode tiles and the one-token kernels (they read the stored codes)
    "pk-decode": LayerSpec("pk-decode", T=2, d_model=256, d_ff=192, n_experts=64, top_k=4, wfmt="q4", seed=85),
    "pk-one-token": LayerSpec("pk-one-token", T=1, d_model=256, d_ff=192, n_experts=16, top_k=4, wfmt="q8", seed=86),
}
FULL = ["q4-prefill-t2048", "q4-decode-t32", "q4-skewed-t256", "q8-prefill-t2048"]


def _both(spec):
    L = inputs.gen_layer(spec)
    g = GpuLayer(L)
    y0, i0, w0 = g.forward()
    dy = np.random.default_rng(7).standard_normal((g.T, spec.d_model)).astype(np.float32)
    dx0 = g.backward(dy)
    plain = g.w
    g.w = plain.with_packed(g.desc)
    torch.cuda.synchronize()
    y1, i1, w1 = g.forward()
    dx1 = g.backward(dy)
    return L, g, plain, (y0, i0, w0, dx0), (y1, i1, w1, dx1)


def _same(a, b):
    assert np.array_equal(a[1].cpu().numpy(), b[1].cpu().numpy())
    assert np.array_equal(a[2].cpu().numpy().view(np.uint32), b[2].cpu().numpy().view(np.uint32))
    assert np.array_equal(a[0].cpu().numpy().view(np.uint32), b[0].cpu().numpy().view(np.uint32))
    assert np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))


@pytest.mark.parametrize("name", list(CASES))
def test_packed_forward_and_backward_are_bit_identical(name):
    _, _, _, a, b = _both(CASES[name])
    _same(a, b)


@pytest.mark.parametrize("name", FULL)
def test_packed_full_size_bit_identical(name):
    _, _, _, a, b = _both(inputs.workload(name))
    _same(a, b)


@pytest.mark.parametrize("name", ["pk-q4-fused-tile16", "pk-q8-g32-ragged"])
def test_packed_layout(name):
    """packed[m][t][s][r][j] = w[m][16t + r][SW s + j], zero past the row."""
    spec = CASES[name]
    L = inputs.gen_layer(spec)
    g = GpuLayer(L)
    pw = g.w.with_packed(g.desc)
    torch.cuda.synchronize()
    b = spec.bits
    SW = 128 * b // 32
    for proj, p in pw.experts.items():
        w = L["experts"][proj]["w"]                      # [M][N][KW] uint32
        M, N, KW = w.shape
        nslab = -(-KW // SW)
        pad = np.zeros((M, N, nslab * SW), np.uint32)
        pad[:, :, :KW] = w
        want = pad.reshape(M, N // 16, 16, nslab, SW).transpose(0, 1, 3, 2, 4).reshape(M, -1)
        got = p["w_packed"].cpu().numpy().view(np.uint32)
        assert got.shape == want.shape and np.array_equal(got, want), proj

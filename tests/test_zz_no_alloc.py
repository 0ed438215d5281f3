"""moe_forward_noalloc (no workspace argument, library-held device scratch)
against moe_forward on the same inputs, through the C ABI: two calls in a
row, the second with fewer tokens, must give bit-identical routing and
outputs (same kernels, deterministic); layers above the scratch size are
refused on the host with MOE_E_WORKSPACE."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV
from sparse_mixture_experts_amd import inputs, moe
from sparse_mixture_experts_amd.inputs import LayerSpec

pytestmark = pytest.mark.gpu


def _run(desc, T, x, w, spec, noalloc):
    y = torch.full((T, spec.d_model), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((T, spec.top_k), -7, dtype=torch.int32, device=DEV)
    wt = torch.full((T, spec.top_k), float("nan"), dtype=torch.float32, device=DEV)
    if noalloc:
        moe.moe_forward_noalloc(desc, T, x, w, y, moe.MOE_DT_F32, idx, wt)
    else:
        ws = torch.empty(moe.moe_workspace_size(desc, T), dtype=torch.uint8, device=DEV)
        moe.moe_forward(desc, T, x, w, y, moe.MOE_DT_F32, idx, wt, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()


@pytest.mark.parametrize("spec,t_second", [
    (inputs.CONFIGS["q4-decode-t32"], 1),
    (LayerSpec("na-q4-shared-skew", T=130, d_model=256, d_ff=192, n_experts=16, top_k=3, n_shared=2, wfmt="q4",
               router_bias="zipf", seed=25), 40),
    (LayerSpec("na-bf16", T=300, d_model=256, d_ff=320, n_experts=8, top_k=2, seed=22), 7),
])
def test_noalloc_matches_forward(spec, t_second):
    L = inputs.gen_layer(spec)
    print(f"[case] noalloc {spec.name}: T={spec.T} then {t_second}", flush=True)
    desc = moe.desc_from_spec(spec)
    w = moe.DeviceWeights.from_layer(L, DEV)
    x = moe.to_device(L["x"], DEV)
    for T in (spec.T, t_second):
        xs = x[:T].contiguous()
        ref = _run(desc, T, xs, w, spec, noalloc=False)
        got = _run(desc, T, xs, w, spec, noalloc=True)
        assert np.array_equal(got[1], ref[1])
        assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32))
        assert np.array_equal(got[0].view(np.uint32), ref[0].view(np.uint32))
        assert np.all(np.isfinite(got[0]))


def test_noalloc_refuses_layers_above_its_scratch():
    spec = inputs.CONFIGS["q4-prefill-t2048"]
    desc = moe.desc_from_spec(spec)
    assert moe.moe_workspace_size(desc, spec.T) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((spec.T, spec.d_model), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((spec.T, spec.d_model), dtype=torch.float32, device=DEV)
    w = moe.Weights()  # never read: the size check comes first
    st = moe.load().moe_forward_noalloc(ctypes.byref(desc), spec.T, x.data_ptr(), ctypes.byref(w), y.data_ptr(),
                                        moe.MOE_DT_F32, None, None, None)
    assert st == moe.MOE_E_WORKSPACE

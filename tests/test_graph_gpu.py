"""moe_forward captured into a HIP graph: every replay must give the eager
call's results bit for bit (the library only launches kernels, so a graph is
the way a serving loop or the benchmark runs it).  The graph is replayed
several times with other eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

from gpu_util import DEV
from sparse_mixture_experts_amd import inputs, moe
from sparse_mixture_experts_amd.inputs import LayerSpec

pytestmark = pytest.mark.gpu

CASES = [
    inputs.CONFIGS["q4-decode-t1"],   # the one-token kernels
    inputs.CONFIGS["q4-decode-t32"],  # router, dispatch, 16-row tiles, combine
    LayerSpec("g-q4-shared", T=130, d_model=256, d_ff=192, n_experts=16, top_k=3, n_shared=2, wfmt="q4",
              router_bias="zipf", seed=25),  # 64-row tiles with shared experts
    LayerSpec("g-q4-decode", T=3, d_model=512, d_ff=256, n_experts=64, top_k=8, wfmt="q4", seed=26),  # decode tiles
    LayerSpec("g-bf16-long-down", T=64, d_model=256, d_ff=2624, n_experts=4, top_k=2, seed=52),  # split down
]


@pytest.mark.parametrize("spec", CASES, ids=[c.name for c in CASES])
def test_graph_replay_matches_eager(spec):
    print(f"[case] graph {spec.name}: T={spec.T}", flush=True)
    L = inputs.gen_layer(spec)
    desc = moe.desc_from_spec(spec)
    w = moe.DeviceWeights.from_layer(L, DEV)
    x = moe.to_device(L["x"], DEV)
    x2 = moe.to_device(inputs.gen_x(spec, 1), DEV)
    T = spec.T
    ws = torch.empty(moe.moe_workspace_size(desc, T), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty_like(ws)
    y = torch.empty((T, spec.d_model), dtype=torch.float32, device=DEV)
    y2 = torch.empty_like(y)
    idx = torch.empty((T, spec.top_k), dtype=torch.int32, device=DEV)
    wt = torch.empty((T, spec.top_k), dtype=torch.float32, device=DEV)
    moe.moe_forward(desc, T, x, w, y, moe.MOE_DT_F32, idx, wt, ws)
    torch.cuda.synchronize()
    ref = (y.cpu().numpy().copy(), idx.cpu().numpy().copy(), wt.cpu().numpy().copy())

    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            moe.moe_forward(desc, T, x, w, y, moe.MOE_DT_F32, idx, wt, ws, cap)
    torch.cuda.synchronize()
    for r in range(4):
        y.fill_(float("nan"))
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref[1]), f"replay {r}: routing differs"
        assert np.array_equal(wt.cpu().numpy().view(np.uint32), ref[2].view(np.uint32)), f"replay {r}"
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref[0].view(np.uint32)), f"replay {r}: y differs"
        # other eager work between replays (another input, its own workspace)
        moe.moe_forward(desc, T, x2, w, y2, moe.MOE_DT_F32, None, None, ws2)
        torch.cuda.synchronize()

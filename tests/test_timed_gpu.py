"""moe_forward_timed through the C ABI: the same outputs as moe_forward, one
stage name per kernel, and a start/stop event pair of each kernel's own
execution."""
import ctypes

import pytest
import torch

from sparse_mixture_experts_amd import inputs, moe

pytestmark = pytest.mark.gpu


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("name,T", [("q4-decode-t1", 1), ("q4-decode-t32", 32), ("q4-skewed-t256", 64)])
def test_timed_forward_matches_and_times_each_kernel(name, T):
    spec = inputs.workload(name).with_(T=T)
    L = inputs.gen_layer(spec)
    dev = "cuda:0"
    desc = moe.desc_from_spec(spec)
    w = moe.DeviceWeights.from_layer(L, dev)
    x = moe.to_device(L["x"], dev)
    ws = torch.empty(moe.moe_workspace_size(desc, T), dtype=torch.uint8, device=dev)
    y0 = torch.empty((T, spec.d_model), dtype=torch.float32, device=dev)
    y1 = torch.empty_like(y0)
    moe.moe_forward(desc, T, x, w, y0, moe.MOE_DT_F32, None, None, ws)
    hip = _hip()
    evs = []
    for _ in range(32):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    names = moe.moe_forward_timed(desc, T, x, w, y1, moe.MOE_DT_F32, None, None, ws, evs)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert 0 < len(names) <= 16 and all(names), names
    for j in range(len(names)):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * j], evs[2 * j + 1]) == 0
        assert 0.0 < ms.value < 100.0, (names[j], ms.value)
    # fewer events than kernels: the rest launch plainly, names still cover every kernel
    names2 = moe.moe_forward_timed(desc, T, x, w, y1, moe.MOE_DT_F32, None, None, ws, evs[:2])
    torch.cuda.synchronize()
    assert names2 == names and torch.equal(y0, y1)
    for e in evs:
        hip.hipEventDestroy(e)

"""moe_forward_static (the forward for callers that cannot allocate: its scratch is a
static per-device array instead of a bound workspace) against moe_forward, through the C
ABI: two calls in a row on each path, the second with a smaller input, each equal bit for
bit to moe_forward on the same plan and inputs (same kernels), and within the BF16 bars
of the fp64 oracle; a plan beyond the array's size and a training plan are refused; the
device status word of a static call flags invalid routing and is cleared by the next."""
import numpy as np
import pytest

import oracle
from mixture_experts_routed_dispatch_amd import inputs
from tests.gpu_util import BF16, check, dev, device_inputs, np_of, say

pytestmark = pytest.mark.gpu


def _static_then_eager(torch, moe, inp, path):
    t = device_inputs(inp)
    layer = moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, path=path)
    assert moe.moe_workspace_bytes(layer.plan) <= moe.MOE_STATIC_SCRATCH_BYTES
    w = moe.weights(t["w13"].data_ptr(), t["w2"].data_ptr())
    stream = int(torch.cuda.current_stream().cuda_stream)
    y_static = torch.full((inp.T, inp.d), 5.0, dtype=torch.bfloat16, device=dev())
    moe.moe_forward_static(layer.plan, t["x"].data_ptr(), t["ids"].data_ptr(), t["scores"].data_ptr(), w,
                           y_static.data_ptr(), stream)
    st, flags = layer.status()
    assert st == moe.MOE_OK and flags == 0
    y_eager = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    layer.close()
    return y_static, y_eager


@pytest.mark.parametrize("path,big,small", [
    (1, (512, 512, 256, 8, 4), (64, 256, 128, 8, 2)),          # grouped-GEMM path
    (2, (32, 2048, 768, 128, 8), (1, 2048, 768, 128, 8)),      # decode path: 32 tokens, then one
])
def test_forward_static_matches_forward(path, big, small):
    import torch
    from mixture_experts_routed_dispatch_amd import moe
    assert torch.cuda.is_available()
    for shape, seed in ((big, 61), (small, 62)):
        T, d, I, E, k = shape
        say("forward_static path %d T=%d d=%d I=%d E=%d k=%d" % (path, T, d, I, E, k))
        inp = inputs.generate(T, d, I, E, k, "uniform", seed=seed)
        y_static, y_eager = _static_then_eager(torch, moe, inp, path)
        assert torch.equal(y_static.view(torch.int16), y_eager.view(torch.int16))
        ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
        check("y (static scratch)", np_of(y_static), ref, **BF16)


def test_forward_static_refusals_and_status():
    import torch
    from mixture_experts_routed_dispatch_amd import moe
    assert torch.cuda.is_available()
    stream = int(torch.cuda.current_stream().cuda_stream)
    # beyond the array: refused before anything runs
    big = moe.moe_plan(8192, 2048, 768, 16, 8)
    assert moe.moe_workspace_bytes(big) > moe.MOE_STATIC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_static(big, 0, 0, 0, moe.weights(0, 0), 0, stream)
    assert ei.value.status == moe.MOE_ERR_TOO_LARGE
    moe.moe_plan_destroy(big)
    tr = moe.moe_plan(64, 256, 128, 8, 2, training=1)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_static(tr, 0, 0, 0, moe.weights(0, 0), 0, stream)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    moe.moe_plan_destroy(tr)
    # invalid routing on a static call sets the flag; the next static call starts clear
    inp = inputs.generate(48, 256, 128, 8, 2, "uniform", seed=63)
    t = device_inputs(inp)
    plan = moe.moe_plan(inp.T, inp.d, inp.I, inp.E, inp.k, path=moe.MOE_PATH_PREFILL)
    w = moe.weights(t["w13"].data_ptr(), t["w2"].data_ptr())
    y = torch.empty((inp.T, inp.d), dtype=torch.bfloat16, device=dev())
    bad = t["ids"].clone()
    bad[3, 1] = inp.E
    moe.moe_forward_static(plan, t["x"].data_ptr(), bad.data_ptr(), t["scores"].data_ptr(), w, y.data_ptr(), stream)
    st, flags = moe.moe_get_status(plan, clear=False, stream=stream)
    assert st == moe.MOE_ERR_ROUTING and flags & moe.MOE_DEV_ID_OUT_OF_RANGE
    moe.moe_forward_static(plan, t["x"].data_ptr(), t["ids"].data_ptr(), t["scores"].data_ptr(), w, y.data_ptr(),
                           stream)
    st, flags = moe.moe_get_status(plan, clear=False, stream=stream)
    assert st == moe.MOE_OK and flags == 0
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    check("y after a flagged call", np_of(y), ref, **BF16)
    moe.moe_plan_destroy(plan)

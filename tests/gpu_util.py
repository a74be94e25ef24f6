"""Helpers for the GPU tests: moving seeded inputs to the device and error norms."""
import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def bf16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())


def np_of(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def rel(a, b):
    """Norm-wise relative error ||a - b|| / ||b||."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def maxrel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    m = np.abs(b).max()
    return float(np.abs(a - b).max() / m) if m > 0 else float(np.abs(a).max())


def device_inputs(inp):
    import torch
    d = dev()
    out = dict(x=bf16_dev(inp.x), w13=bf16_dev(inp.w13), w2=bf16_dev(inp.w2),
               ids=torch.from_numpy(inp.ids).to(d), scores=torch.from_numpy(inp.scores).to(d))
    if inp.dy is not None:
        out["dy"] = bf16_dev(inp.dy)
    return out


def say(*a):
    print(*a, flush=True)


# Parity bars.  The layer's budget is norm-wise (relative error of the whole tensor
# against the fp64 oracle): 2e-2 for BF16, 6e-2 for MXFP8 against the FP32 oracle.
# Next to it every comparison bounds the largest error against the largest value
# (maxrel = max|got - ref| / max|ref|) and each element:
#     |got - ref| <= elem * (|ref| + rms(ref over the element's slice)),
# so that a defect confined to a few rows or one tile cannot hide inside the norm.
# BF16: a, o and the outputs are rounded to BF16 (relative step 2^-8, so errors of
# about 2^-9 |v| each), which puts the measured norm-wise error near 3e-3 and the
# largest element error of y, dx and dS (max over up to ~10^7 elements) below
# 1.5e-2 of the tensor's rms; `floor` = 5e-3 guards that noise level, elem = 3e-2
# leaves twice the largest expected element error.  Weight gradients are sums over an
# expert's rows, which for an expert with a few rows cancel: an emulation of the
# kernels' BF16 roundings in numpy (a, probs * dy, dh, output) on these test layers
# gives element errors up to 0.048 of the expert's rms, so there the slice is the
# expert and elem = 0.12.  MXFP8 against the oracle that quantizes x and the
# gated-activation output at the same points: a requantized element of `a` lands one
# E4M3 step (up to 12.5 % of it) away from the oracle's when the FP32 and fp64 values
# straddle a rounding boundary; for a large element (5 standard deviations) times a
# large W2 coefficient (3 / sqrt(I)) that moves one output element by about 0.1 of the
# output's rms, so elem = 0.25 and maxrel <= 0.1 (a wrong tile or row piece moves
# elements by about their own magnitude).
BF16 = dict(tol=2e-2, floor=5e-3, elem=3e-2, maxrel_tol=3e-2)
BF16_WGRAD = dict(tol=2e-2, floor=5e-3, elem=0.12, maxrel_tol=3e-2, per_slice=True)
MX = dict(tol=6e-2)
MX_QUANT = dict(tol=1e-2, elem=0.25, maxrel_tol=0.1)


def check(label, got, ref, tol, floor=None, elem=None, maxrel_tol=None, per_slice=False):
    """Assert the bars above for one output tensor; prints the figures.  per_slice: the
    rms of the element bound is taken over each index of the first axis (the expert of a
    weight gradient) instead of the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (label, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), label
    e = rel(got, ref)
    m = maxrel(got, ref)
    worst = 0.0
    if elem is not None and ref.size:
        if per_slice:
            rms = np.sqrt(np.mean(ref.reshape(ref.shape[0], -1) ** 2, axis=1)).reshape((-1,) + (1,) * (ref.ndim - 1))
        else:
            rms = float(np.sqrt(np.mean(ref * ref)))
        excess = np.abs(got - ref) / (elem * (np.abs(ref) + rms) + 1e-300)
        worst = float(excess.max())
    print("  %s: rel %.3e maxrel %.3e worst element %.2f of its bound" % (label, e, m, worst), flush=True)
    assert e <= tol, (label, e, tol)
    if floor is not None:
        assert e <= floor, (label, e, floor)
    if maxrel_tol is not None:
        assert m <= maxrel_tol, (label, m, maxrel_tol)
    if elem is not None and ref.size:
        assert worst <= 1.0, (label, worst, np.unravel_index(int(np.argmax(excess)), ref.shape))
    return e

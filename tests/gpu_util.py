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

"""Pins for the oracle's backward pass (blog post "What it is selling": DGRAD and
WGRAD; nvfp4moe README "Training": input, weight and router gradients).

* Central finite differences of L = <dY, y> in the fp64 oracle along random
  directions for x, W13, W2 and the scores.  Base points and steps are chosen
  so that x +- h v is exact in float32 (BF16 base values, h = 2^-16), so the
  difference quotient sees exactly the intended perturbation.
* The dense case (E = 1, k = 1) against torch float64 autograd.
* Experts that receive no row get a weight gradient of exactly +0.0.
* Token-subset and column-subset evaluations agree with the full ones.
"""
import numpy as np
import pytest
import torch

from mixture_experts_routed_dispatch_amd import inputs

H = 2.0 ** -16


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def small_case(seed, T=12, d=64, I=32, E=5, k=2, routing="uniform"):
    inp = inputs.generate(T=T, d=d, I=I, E=E, k=k, routing=routing, seed=seed, with_dy=True)
    # scores rounded to BF16 values so that s +- h v stays exact in float32
    inp.scores = f32(inputs.to_bf16_bits(inp.scores))
    return inp


def loss(orc, x, ids, s, w13, w2, dy, act=0):
    y = orc.forward_tokens(x, ids, s, w13, w2, act=act)
    return float((y * dy.astype(np.float64)).sum())


def fd(orc, inp, which, v, act=0):
    base = dict(x=f32(inp.x), s=inp.scores, w13=f32(inp.w13), w2=f32(inp.w2))
    dyf = f32(inp.dy)
    vals = []
    for sign in (+1.0, -1.0):
        args = dict(base)
        pert = (base[which].astype(np.float64) + sign * H * v)
        assert np.array_equal(pert.astype(np.float32).astype(np.float64), pert)  # exact in f32
        args[which] = pert.astype(np.float32)
        vals.append(loss(orc, args["x"], inp.ids, args["s"], args["w13"], args["w2"], dyf, act))
    return (vals[0] - vals[1]) / (2 * H)


@pytest.mark.parametrize("seed,act", [(0, 0), (1, 0), (0, 1), (1, 2)])
def test_finite_differences(orc, seed, act):
    inp = small_case(seed)
    rng = np.random.default_rng(100 + seed)
    if act == 2:
        # relu has a kink at 0: no routed gate may cross it under the perturbations, whose
        # effect on a gate is at most h * sum|w| (x moved) or h * sum|x| (W1 moved)
        x64, w64 = f32(inp.x).astype(np.float64), f32(inp.w13).astype(np.float64)
        g = np.einsum("td,eid->tei", x64, w64[:, :inp.I])
        gmin = min(np.abs(g[t, e]).min() for t in range(inp.T) for e in inp.ids[t])
        step = H * max(np.abs(w64[:, :inp.I]).sum(axis=2).max(), np.abs(x64).sum(axis=1).max())
        assert gmin > 2 * step, (gmin, step)
    dx, ds = orc.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy, act=act)
    dw2, dw13 = orc.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy, act=act)
    E, d, I = inp.E, inp.d, inp.I
    dw13_full = dw13.reshape(E, 2 * I, d)          # [E, 2, I, d] with all columns = [E, 2I, d]
    grads = {"x": dx, "s": ds, "w13": dw13_full, "w2": dw2}
    shapes = {"x": inp.x.shape, "s": inp.scores.shape, "w13": inp.w13.shape, "w2": inp.w2.shape}
    for which in ("x", "s", "w13", "w2"):
        v = rng.integers(-1, 2, size=shapes[which]).astype(np.float64)
        num = fd(orc, inp, which, v, act)
        ana = float((grads[which] * v).sum())
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (which, num, ana)


ACT_TORCH = {0: torch.nn.functional.silu,
             1: lambda z: torch.nn.functional.gelu(z, approximate="none"),
             2: torch.nn.functional.relu}


@pytest.mark.parametrize("act", [0, 1, 2])
def test_dense_case_against_torch_autograd(orc, act):
    """E = 1, k = 1: the layer is a dense gated MLP; torch float64 autograd (silu, the
    exact gelu, relu) gives every gradient."""
    inp = small_case(3, T=9, d=64, I=32, E=1, k=1)
    s = np.ones((inp.T, 1), np.float32) * np.float32(0.625)
    xf, w13f, w2f, dyf = f32(inp.x), f32(inp.w13[0]), f32(inp.w2[0]), f32(inp.dy)
    X = torch.tensor(xf, dtype=torch.float64, requires_grad=True)
    W1 = torch.tensor(w13f[:32], dtype=torch.float64, requires_grad=True)
    W3 = torch.tensor(w13f[32:], dtype=torch.float64, requires_grad=True)
    W2 = torch.tensor(w2f, dtype=torch.float64, requires_grad=True)
    S = torch.tensor(s[:, 0].astype(np.float64), requires_grad=True)
    o = (ACT_TORCH[act](X @ W1.T) * (X @ W3.T)) @ W2.T
    y = S[:, None] * o
    (y * torch.tensor(dyf, dtype=torch.float64)).sum().backward()
    dx, ds = orc.backward_tokens(inp.x, inp.ids, s, inp.w13, inp.w2, inp.dy, act=act)
    dw2, dw13 = orc.wgrad_cols(inp.x, inp.ids, s, inp.w13, inp.w2, inp.dy, act=act)
    np.testing.assert_allclose(dx, X.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ds[:, 0], S.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw2[0], W2.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw13[0, 0], W1.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw13[0, 1], W3.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_empty_experts_get_positive_zero(orc):
    inp = small_case(4, T=20, d=64, I=32, E=16, k=2, routing="zipf")
    counts = np.bincount(inp.ids.ravel(), minlength=16)
    assert (counts == 0).sum() >= 8
    dw2, dw13 = orc.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(dw2[e] == 0.0) and not np.any(np.signbit(dw2[e]))
        assert np.all(dw13[e] == 0.0) and not np.any(np.signbit(dw13[e]))
    for e in np.nonzero(counts > 0)[0]:
        assert np.any(dw2[e] != 0.0)


def test_subsets_match_full(orc):
    inp = small_case(5, T=15, d=64, I=32, E=4, k=2)
    dx, ds = orc.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    toks = np.array([14, 3, 3, 0], np.int32)
    dxs, dss = orc.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy, toks=toks)
    np.testing.assert_array_equal(dxs, dx[toks])
    np.testing.assert_array_equal(dss, ds[toks])
    dw2, dw13 = orc.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    cols = np.array([31, 2, 17], np.int32)
    dw2c, dw13c = orc.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy, icols=cols)
    np.testing.assert_array_equal(dw2c, dw2[:, :, cols])
    np.testing.assert_array_equal(dw13c, dw13[:, :, cols, :])


def test_router_gradient_is_unscaled_expert_output(orc):
    # dS[t][j] = <dY[t], o_(t,j)>: with dY = e_n it equals the n-th element of o.
    inp = small_case(6, T=6, d=64, I=32, E=3, k=2)
    _, o = orc.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, want_o=True)
    dy = np.zeros((inp.T, inp.d), np.float32)
    dy[:, 5] = 1.0
    _, ds = orc.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2,
                                inputs.to_bf16_bits(dy))
    np.testing.assert_allclose(ds, o[:, :, 5], rtol=1e-14, atol=1e-15)

"""HIP path against the CPU oracle, through the C ABI (include/moe.h).

* Dispatch (nvfp4moe README "Grouped GEMM", "Training"): bit-exact m_indptr,
  gather, slots and probs on every workload's routing and on adversarial ones;
  the device status word flags invalid routing.
* Forward (blog post "What it is selling"; nvfp4moe README "MoE layer"):
  norm-wise relative error <= 2e-2 (BF16) against the fp64 oracle, BF16 results
  also under the 5e-3 noise floor and every element within 3e-2 (|ref| + rms)
  (tests/gpu_util.py), on small layers that span several tiles with ragged
  tails, and at the full workload sizes (every token of the prefill and decode
  workloads, sampled tokens of the MXFP8 one), with the launch configuration
  the benchmark times.
* Backward (DGRAD, WGRAD, router gradient): the same bars on dx, dscores,
  dW13 and dW2 (also with h recomputed); experts with no row get exactly +0.0.
* Run-to-run bitwise determinism and HIP-graph replay equal to eager calls.
"""
import numpy as np
import pytest

import oracle
from mixture_experts_routed_dispatch_amd import inputs
from tests.gpu_util import BF16, BF16_WGRAD, MX, MX_QUANT, bf16_dev, check, dev, device_inputs, np_of, rel, say

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from mixture_experts_routed_dispatch_amd import moe
    moe.lib()
    oracle.build(force=False)
    return torch


def make_layer(inp, training=False, path=0):
    from mixture_experts_routed_dispatch_amd import moe
    return moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, training=training, path=path)


# ------------------------------------------------------------------ dispatch

def _routing_cases():
    cases = []
    for name in ("tiny", "prefill", "train", "decode1", "decode32", "mxfp8"):
        c = inputs.CONFIGS[name]
        cases.append((name, c["T"], c["E"], c["k"], c["routing"]))
    cases += [("k1", 3000, 16, 1, "uniform"), ("E256k32", 4096, 256, 32, "uniform"),
              ("ragged_chunk", 2049, 7, 3, "uniform"), ("same_experts", 5000, 64, 4, "same"),
              ("descending", 700, 40, 6, "descending"), ("zipf_small", 333, 128, 8, "zipf"),
              ("one_token", 1, 8, 8, "uniform"), ("max_rows", 16384, 256, 8, "uniform")]
    return cases


def _routing(kind, T, E, k, seed):
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        return inputs.uniform_routing(rng, T, E, k)
    if kind == "zipf":
        return inputs.zipf_routing(rng, T, E, k)
    if kind == "same":
        return np.tile(rng.permutation(E)[:k].astype(np.int32), (T, 1))
    if kind == "descending":
        return np.tile(np.arange(E - 1, E - 1 - k, -1, dtype=np.int32), (T, 1))
    raise ValueError(kind)


@pytest.mark.parametrize("name,T,E,k,kind", _routing_cases())
def test_dispatch_bit_exact(torch_cuda, name, T, E, k, kind):
    torch = torch_cuda
    say("dispatch case", name, T, E, k, kind)
    ids = _routing(kind, T, E, k, seed=T + E)
    scores = np.random.default_rng(1).random((T, k)).astype(np.float32)
    from mixture_experts_routed_dispatch_amd import moe
    layer = moe.Layer(T, 64, 64, E, k)
    m_indptr, gather, slots, probs = layer.dispatch(torch.from_numpy(ids).to(dev()),
                                                    torch.from_numpy(scores).to(dev()))
    st, flags = layer.status()
    assert st == moe.MOE_OK and flags == 0
    ref = oracle.dispatch(ids, scores, E)
    assert np.array_equal(m_indptr.cpu().numpy(), ref[0])
    assert np.array_equal(gather.cpu().numpy(), ref[1])
    assert np.array_equal(slots.cpu().numpy(), ref[2])
    assert np.array_equal(probs.cpu().numpy().view(np.uint32), ref[3].view(np.uint32))
    # run-to-run identical
    again = layer.dispatch(torch.from_numpy(ids).to(dev()), torch.from_numpy(scores).to(dev()))
    for a, b in zip((m_indptr, gather, slots, probs), again):
        assert torch.equal(a, b)
    layer.close()


def test_dispatch_flags_invalid_routing(torch_cuda):
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, E, k = 100, 8, 2
    ids = _routing("uniform", T, E, k, 3)
    scores = np.ones((T, k), np.float32)
    layer = moe.Layer(T, 64, 64, E, k)
    bad = ids.copy()
    bad[7, 1] = E            # out of range
    layer.dispatch(torch.from_numpy(bad).to(dev()), torch.from_numpy(scores).to(dev()))
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING and flags & moe.MOE_DEV_ID_OUT_OF_RANGE
    bad = ids.copy()
    bad[9, 1] = bad[9, 0]    # repeated in a row
    layer.dispatch(torch.from_numpy(bad).to(dev()), torch.from_numpy(scores).to(dev()))
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING and flags == moe.MOE_DEV_ID_DUPLICATE
    layer.dispatch(torch.from_numpy(ids).to(dev()), torch.from_numpy(scores).to(dev()))
    st, flags = layer.status()
    assert st == moe.MOE_OK and flags == 0   # the flag was cleared and stays clear
    layer.close()


# ------------------------------------------------------------------ forward

SMALL_SHAPES = [
    # T, d, I, E, k, routing
    (64, 256, 128, 8, 2, "uniform"),       # the tiny workload
    (600, 512, 384, 6, 3, "uniform"),      # ~300 rows/expert: 2 row tiles, ragged tail; 3 W13 tiles
    (257, 320, 192, 5, 2, "uniform"),      # d, I not multiples of the tile: masked tails
    (300, 256, 128, 128, 8, "zipf"),       # skew, 8+ empty experts, many 1-row experts
    (130, 128, 64, 1, 1, "uniform"),       # dense layer (E = 1, k = 1)
    (1, 256, 128, 16, 4, "uniform"),       # one token
    (320, 256, 128, 256, 32, "zipf"),      # the expert and top-k limits (E = 256, k = 32), skewed
]


@pytest.mark.parametrize("T,d,I,E,k,routing", SMALL_SHAPES)
def test_forward_small(torch_cuda, T, d, I, E, k, routing):
    torch = torch_cuda
    say("forward small", T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=11)
    t = device_inputs(inp)
    layer = make_layer(inp, path=1)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    check("y", np_of(y), ref, **BF16)
    layer.close()


def test_forward_zero_scores_give_zero(torch_cuda):
    torch = torch_cuda
    inp = inputs.generate(96, 256, 128, 8, 2, seed=2)
    t = device_inputs(inp)
    layer = make_layer(inp, path=1)
    y = layer.forward(t["x"], t["ids"], torch.zeros_like(t["scores"]), t["w13"], t["w2"])
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy()
    assert np.all(yb == 0)          # +0.0 exactly: sums start at +0 and 0 * o = +-0
    layer.close()


@pytest.mark.parametrize("name,path", [("prefill", 0), ("train", 0), ("decode1", 0), ("decode32", 0),
                                       ("decode1", 1), ("decode32", 1)])
def test_forward_full_size_sampled(torch_cuda, name, path):
    torch = torch_cuda
    say("forward full size", name, "path", path)
    inp = inputs.generate_config(name, seed=0, with_dy=False)
    t = device_inputs(inp)
    layer = make_layer(inp, path=path)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    y2 = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    st, flags = layer.status()
    assert flags == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))      # bitwise deterministic
    # every token: the fp64 oracle takes the 8192 prefill tokens in a few seconds
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    check("y (all %d tokens)" % inp.T, np_of(y), ref, **BF16)
    layer.close()


def _counts_routing(counts, k, seed):
    """ids [T, k] with exactly counts[e] rows per expert (distinct per token), T = sum / k:
    the expert-sorted slot list is cut into k columns T apart (no expert has T rows, so a
    token's experts differ), then tokens and columns are shuffled."""
    counts = np.asarray(counts)
    T = int(counts.sum()) // k
    assert T * k == counts.sum() and counts.max() < T
    flat = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    ids = np.stack([flat[j * T:(j + 1) * T] for j in range(k)], axis=1)
    rng = np.random.default_rng(seed)
    ids = ids[rng.permutation(T)]
    for t in range(T):
        ids[t] = ids[t, rng.permutation(k)]
    return ids


@pytest.mark.parametrize("training", [False, True])
def test_forward_ragged_expert_tails(torch_cuda, training):
    """Experts with a few rows (1 to 60) past four whole 256-row tiles, one with exactly
    1024 rows and one empty: the partly filled last tiles load clamped rows and mask their
    stores.  Every token that has a row in such a tile (plus 32 others) is checked
    against the oracle, in forward and, when training, through dx (which reads the saved
    h of those rows)."""
    import dataclasses
    torch = torch_cuda
    d, I, E, k = 1024, 512, 16, 2
    rng = np.random.default_rng(8)
    counts = 1024 + rng.integers(1, 61, size=E)
    counts[3] = 1024             # an exact multiple of the tile: no partial tile
    counts[7] = 0                # an empty expert
    if counts.sum() % k:
        counts[0] += 1
    say("ragged expert tails: d=%d I=%d E=%d k=%d training=%s counts %s" % (d, I, E, k, training, counts.tolist()))
    ids = _counts_routing(counts, k, seed=9)
    T = ids.shape[0]
    inp = inputs.generate(T, d, I, E, k, "uniform", seed=23, with_dy=training)
    inp = dataclasses.replace(inp, ids=ids)
    t = device_inputs(inp)
    layer = make_layer(inp, training=training, path=1)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    y2 = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    if training:
        dx = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])[0]
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))      # bitwise deterministic
    # tokens of the experts' rows past their last whole tile (rows are in token order)
    toks = set()
    for e in range(E):
        te = np.nonzero((ids == e).any(axis=1))[0]
        toks.update(te[(len(te) // 256) * 256:].tolist())
    toks.update(rng.choice(T, size=32, replace=False).tolist())
    toks = np.array(sorted(toks), np.int32)
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, toks=toks)
    got = np_of(y)[toks]
    check("y (%d tokens)" % len(toks), got, ref, **BF16)
    if training:
        dx_ref, _ = oracle.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy, toks=toks)
        check("dx", np_of(dx)[toks], dx_ref, **BF16)
    layer.close()


# ------------------------------------------------------------------ pre-dispatched rows

@pytest.mark.parametrize("T,d,I,E,k,routing", [(600, 512, 384, 6, 3, "uniform"), (3000, 1024, 512, 16, 4, "uniform"),
                                               (300, 256, 128, 128, 8, "zipf")])
def test_forward_routed_matches_oracle(torch_cuda, T, d, I, E, k, routing):
    """Rows put in expert order by the oracle's own dispatch, with its m_indptr: row
    slots[t][j] of the output is the expert output of (t, j)."""
    torch = torch_cuda
    say("forward routed", T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=31)
    m_indptr, gather, slots, _ = oracle.dispatch(inp.ids, inp.scores, E)
    t = device_inputs(inp)
    x_rows = t["x"][torch.from_numpy(gather.astype(np.int64)).to(dev())].contiguous()
    layer = make_layer(inp, path=1)
    out = layer.forward_routed(x_rows, torch.from_numpy(m_indptr).to(dev()), t["w13"], t["w2"])
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    _, o_ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, want_o=True)
    got = np_of(out)[slots.reshape(-1)].reshape(T, k, d)
    check("o", got, o_ref, **BF16)
    layer.close()


def test_forward_routed_ragged_segments(torch_cuda):
    """Caller-made segments: empty experts (first, middle, last), a segment of one row, and
    fewer rows than T*k; each row is checked as a one-expert token (k = 1, score 1) of the
    oracle, and the rows past m_indptr[E] are left as they were."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, d, I, E, k = 400, 512, 256, 8, 2
    counts = np.array([0, 300, 1, 0, 257, 45, 100, 0])
    m_indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(m_indptr[-1])
    assert n < T * k
    inp = inputs.generate(n, d, I, E, 1, "uniform", seed=32)
    ids = np.repeat(np.arange(E, dtype=np.int32), counts)[:, None]
    ones = np.ones((n, 1), np.float32)
    x_rows = bf16_dev(inp.x)
    w13, w2 = bf16_dev(inp.w13), bf16_dev(inp.w2)
    layer = moe.Layer(T, d, I, E, k, path=moe.MOE_PATH_PREFILL)
    out = torch.full((T * k, d), 3.0, dtype=torch.bfloat16, device=dev())
    layer.forward_routed(x_rows, torch.from_numpy(m_indptr).to(dev()), w13, w2, out=out)
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    _, o_ref = oracle.forward_tokens(inp.x, ids, ones, inp.w13, inp.w2, want_o=True)
    got = np_of(out)
    check("o (ragged segments)", got[:n], o_ref[:, 0], **BF16)
    assert np.all(got[n:] == 3.0)
    layer.close()


def test_forward_routed_mxfp8_ragged_segments(torch_cuda):
    """MXFP8 on caller-made segments (empty experts first, middle and last, a one-row
    segment, fewer rows than T*k, and an x_rows buffer of exactly m_indptr[E] rows): each
    row against the oracle as a one-expert token (k = 1, score 1), on the prepared
    weights, both with FP32 activations and quantizing x and the SwiGLU output as the
    kernels do; rows past m_indptr[E] stay as they were."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, d, I, E, k = 400, 512, 256, 8, 2
    counts = np.array([0, 300, 1, 0, 257, 45, 100, 0])
    m_indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(m_indptr[-1])
    assert n < T * k
    inp = inputs.generate(n, d, I, E, 1, "uniform", seed=33)
    ids = np.repeat(np.arange(E, dtype=np.int32), counts)[:, None]
    ones = np.ones((n, 1), np.float32)
    layer = moe.Layer(T, d, I, E, k, precision=moe.MOE_MXFP8_E4M3, path=moe.MOE_PATH_PREFILL)
    w13q, w13s, w2q, w2s = layer.prepare_weights(bf16_dev(inp.w13), bf16_dev(inp.w2))
    out = torch.full((T * k, d), 3.0, dtype=torch.bfloat16, device=dev())
    layer.forward_routed(bf16_dev(inp.x), torch.from_numpy(m_indptr).to(dev()), w13q, w2q, w13s, w2s, out=out)
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    got = np_of(out)
    w13f, w2f = _prepared_f32(inp.w13), _prepared_f32(inp.w2)
    ref = oracle.forward_tokens(inp.x, ids, ones, w13f, w2f)
    ref_q = oracle.forward_tokens_mx(inp.x, ids, ones, w13f, w2f)
    check("o vs fp32 oracle", got[:n], ref, **MX)
    check("o vs quantizing oracle", got[:n], ref_q, **MX_QUANT)
    assert np.all(got[n:] == 3.0)
    layer.close()


def test_forward_routed_mxfp8_matches_oracle(torch_cuda):
    """MXFP8: rows put in expert order by the oracle's dispatch give, row for row, the
    expert outputs of the token-routed forward's quantizing oracle, and the status stays
    clear."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, d, I, E, k = 600, 512, 384, 6, 3
    inp = inputs.generate(T, d, I, E, k, "uniform", seed=34)
    m_indptr, gather, slots, _ = oracle.dispatch(inp.ids, inp.scores, E)
    t = device_inputs(inp)
    x_rows = t["x"][torch.from_numpy(gather.astype(np.int64)).to(dev())].contiguous()
    layer = moe.Layer(T, d, I, E, k, precision=moe.MOE_MXFP8_E4M3, path=moe.MOE_PATH_PREFILL)
    w13q, w13s, w2q, w2s = layer.prepare_weights(t["w13"], t["w2"])
    out = layer.forward_routed(x_rows, torch.from_numpy(m_indptr).to(dev()), w13q, w2q, w13s, w2s)
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    w13f, w2f = _prepared_f32(inp.w13), _prepared_f32(inp.w2)
    ids_rows = np.zeros((T * k, 1), np.int32)
    for e in range(E):
        ids_rows[m_indptr[e]:m_indptr[e + 1], 0] = e
    x_bits = inp.x[gather]
    ref_q = oracle.forward_tokens_mx(x_bits, ids_rows, np.ones((T * k, 1), np.float32), w13f, w2f)
    check("o vs quantizing oracle", np_of(out), ref_q, **MX_QUANT)
    layer.close()


def test_forward_routed_rejects_bad_indptr(torch_cuda):
    """A decreasing m_indptr, or one whose total passes T*k, sets MOE_DEV_BAD_INDPTR and
    leaves the output untouched (every expert taken as empty)."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, d, I, E, k = 256, 256, 128, 4, 2
    layer = moe.Layer(T, d, I, E, k, path=moe.MOE_PATH_PREFILL)
    g = torch.Generator(device="cpu").manual_seed(3)
    x_rows = (torch.randn((T * k, d), generator=g) * 0.5).to(torch.bfloat16).to(dev())
    w13 = (torch.randn((E, 2 * I, d), generator=g) / 16).to(torch.bfloat16).to(dev())
    w2 = (torch.randn((E, d, I), generator=g) / 11).to(torch.bfloat16).to(dev())
    for bad in ([0, 100, 50, 300, 400], [0, 100, 200, 300, T * k + 1], [5, 100, 200, 300, 400]):
        out = torch.full((T * k, d), 7.0, dtype=torch.bfloat16, device=dev())
        layer.forward_routed(x_rows, torch.tensor(bad, dtype=torch.int32, device=dev()), w13, w2, out=out)
        st, flags = layer.status(clear=True)
        assert st == moe.MOE_ERR_ROUTING and flags == moe.MOE_DEV_BAD_INDPTR, bad
        assert bool(torch.all(out == 7.0)), bad
    layer.close()


def test_graph_replay_matches_eager(torch_cuda):
    torch = torch_cuda
    inp = inputs.generate(512, 512, 256, 8, 4, seed=4)
    t = device_inputs(inp)
    layer = make_layer(inp, path=1)
    y_eager = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    y_out = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"], y=y_out)   # warm
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"], y=y_out)
    for rep in range(4):
        y_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_out.view(torch.int16), y_eager.view(torch.int16)), rep
        # eager work between replays
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
        torch.cuda.synchronize()
    layer.close()


def test_mxfp8_graph_replay_matches_eager(torch_cuda):
    """The MXFP8 forward (dispatch, x conversion and its routed scale copy, both FP8
    products, combine) captured in one HIP graph: every replay, with eager calls of the
    same plan between replays, equals the eager result bit for bit."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    inp = inputs.generate(512, 512, 256, 8, 4, seed=8)
    t = device_inputs(inp)
    layer = moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, precision=moe.MOE_MXFP8_E4M3, path=1)
    w13q, w13s, w2q, w2s = layer.prepare_weights(t["w13"], t["w2"])
    fwd = lambda y=None: layer.forward(t["x"], t["ids"], t["scores"], w13q, w2q, w13s, w2s, y=y)
    y_eager = fwd()
    torch.cuda.synchronize()
    y_out = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd(y_out)                                   # warm
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fwd(y_out)
    for rep in range(4):
        y_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_out.view(torch.int16), y_eager.view(torch.int16)), rep
        fwd()                                        # eager work between replays
        torch.cuda.synchronize()
    assert layer.status()[1] == 0
    layer.close()


@pytest.mark.parametrize("acc,rec", [(False, False), (True, True)])
def test_training_graph_replay_matches_eager(torch_cuda, acc, rec):
    """Forward + backward of a training plan captured in one HIP graph: every replay (the
    gradient buffers reset first, eager work of the same plan between replays) gives the
    eager results bit for bit; with wgrad_accumulate and recompute_h as well."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, d, I, E, k = 400, 512, 384, 6, 3
    inp = inputs.generate(T, d, I, E, k, "uniform", seed=61, with_dy=True)
    t = device_inputs(inp)
    layer = moe.Layer(T, d, I, E, k, training=True, wgrad_accumulate=acc, recompute_h=rec)
    g0 = torch.Generator(device="cpu").manual_seed(11)
    dw13_0 = (torch.randn((E, 2 * I, d), generator=g0) * 0.05).to(torch.bfloat16).to(dev())
    dw2_0 = (torch.randn((E, d, I), generator=g0) * 0.05).to(torch.bfloat16).to(dev())
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev())
    dx = torch.empty_like(y)
    ds = torch.empty((T, k), dtype=torch.float32, device=dev())
    dw13, dw2 = dw13_0.clone(), dw2_0.clone()

    def step():
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"], y=y)
        layer.backward(t["dy"], t["x"], t["w13"], t["w2"], dx=dx, dw13=dw13, dw2=dw2, dscores=ds)

    step()
    torch.cuda.synchronize()
    ref = [v.clone() for v in (y, dx, dw13, dw2, ds)]
    gr = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                             # warm on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        dw13.copy_(dw13_0)
        dw2.copy_(dw2_0)
        for v in (y, dx, ds):
            v.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "dx", "dw13", "dw2", "ds"), (y, dx, dw13, dw2, ds), ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (rep, name)
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])   # eager work between replays
        torch.cuda.synchronize()
    assert layer.status()[1] == 0
    layer.close()


def test_routed_graph_replay_matches_eager(torch_cuda):
    """moe_forward_routed captured in a HIP graph replays to the eager result."""
    torch = torch_cuda
    T, d, I, E, k = 600, 512, 384, 6, 3
    inp = inputs.generate(T, d, I, E, k, "uniform", seed=63)
    m_indptr, gather, _, _ = oracle.dispatch(inp.ids, inp.scores, E)
    t = device_inputs(inp)
    x_rows = t["x"][torch.from_numpy(gather.astype(np.int64)).to(dev())].contiguous()
    mi = torch.from_numpy(m_indptr).to(dev())
    layer = make_layer(inp, path=1)
    ref = layer.forward_routed(x_rows, mi, t["w13"], t["w2"]).clone()
    out = torch.empty_like(ref)
    gr = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward_routed(x_rows, mi, t["w13"], t["w2"], out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        layer.forward_routed(x_rows, mi, t["w13"], t["w2"], out=out)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
        torch.cuda.synchronize()
    layer.close()


# ------------------------------------------------------------------ decode path

DECODE_SHAPES = [
    # T, d, I, E, k, routing
    (1, 256, 128, 8, 2, "uniform"),
    (7, 512, 384, 16, 4, "uniform"),
    (3, 256, 128, 8, 8, "uniform"),        # every token picks every expert: 3 rows each
    (20, 256, 192, 4, 4, "uniform"),       # 20 rows per expert: two 16-row groups
    (64, 128, 64, 1, 1, "uniform"),        # dense layer through the decode kernels, 64 rows
    (8, 320, 192, 64, 32, "uniform"),      # k = 32
    (30, 256, 128, 128, 8, "zipf"),        # skewed, some experts with many rows, most empty
    (256, 128, 64, 200, 1, "uniform"),     # T*k at the decode limit
    (32, 1024, 512, 64, 8, "uniform"),     # enough items for one wave per item (no K split)
    (64, 256, 2048, 8, 4, "uniform"),      # W13 items >= 8 per CU (pipelined W13), 32 rows per expert
    (48, 512, 2048, 16, 4, "zipf"),        # the same, skewed: row groups of 16 past the first
    (64, 2048, 256, 24, 4, "zipf"),        # one wave per W2 item, skewed: row groups past 16
    (1, 512, 256, 16, 4, "uniform"),       # one token: W13 split four ways over K, then W2 + combine
    (1, 1024, 640, 64, 6, "uniform"),      # one token, k = 6: three expert pairs in the W2 launch
    (1, 512, 192, 32, 5, "uniform"),       # one token, odd k: the last expert pair half empty
    (1, 4096, 512, 16, 4, "uniform"),      # one token, d = 4096: 512 blocks of 8 outputs in the W2 launch
]


@pytest.mark.parametrize("T,d,I,E,k,routing", DECODE_SHAPES)
def test_decode_small(torch_cuda, T, d, I, E, k, routing):
    torch = torch_cuda
    say("decode small", T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=17)
    t = device_inputs(inp)
    layer = make_layer(inp, path=2)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    y2 = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    st, flags = layer.status()
    assert flags == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))      # counters reset between calls
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    check("y", np_of(y), ref, **BF16)
    layer.close()


def test_decode_zero_scores_and_rerouting(torch_cuda):
    torch = torch_cuda
    inp = inputs.generate(16, 256, 128, 32, 4, seed=21)
    t = device_inputs(inp)
    layer = make_layer(inp, path=2)
    y0 = layer.forward(t["x"], t["ids"], torch.zeros_like(t["scores"]), t["w13"], t["w2"])
    torch.cuda.synchronize()
    assert np.all(y0.view(torch.int16).cpu().numpy() == 0)
    # a different routing in between must not disturb the next call
    other = inputs.uniform_routing(np.random.default_rng(99), inp.T, inp.E, inp.k)
    layer.forward(t["x"], torch.from_numpy(other).to(dev()), t["scores"], t["w13"], t["w2"])
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    check("y", np_of(y), ref, **BF16)
    layer.close()


@pytest.mark.parametrize("T,d,I,E,k", [(4, 512, 256, 16, 4), (1, 512, 256, 16, 4), (32, 1024, 512, 64, 8)])
def test_decode_graph_replay_matches_eager(torch_cuda, T, d, I, E, k):
    """Replays of a captured decode call equal the eager result: T = 4 (W2 split over K
    per item) and T = 32 (one wave per W2 item), three launches with the combine; T = 1,
    W13, then W2 with the combine."""
    torch = torch_cuda
    inp = inputs.generate(T, d, I, E, k, seed=23)
    t = device_inputs(inp)
    layer = make_layer(inp, path=2)
    y_eager = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    y_out = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"], y=y_out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"], y=y_out)
    for rep in range(4):
        y_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_out.view(torch.int16), y_eager.view(torch.int16)), rep
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
        torch.cuda.synchronize()
    layer.close()


def test_decode_flags_invalid_routing(torch_cuda):
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    inp = inputs.generate(4, 256, 128, 8, 2, seed=5)
    t = device_inputs(inp)
    layer = make_layer(inp, path=2)
    bad = inp.ids.copy()
    bad[1, 1] = bad[1, 0]
    layer.forward(t["x"], torch.from_numpy(bad).to(dev()), t["scores"], t["w13"], t["w2"])
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING and flags == moe.MOE_DEV_ID_DUPLICATE
    bad = inp.ids.copy()
    bad[2, 0] = -3
    layer.forward(t["x"], torch.from_numpy(bad).to(dev()), t["scores"], t["w13"], t["w2"])
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING and flags & moe.MOE_DEV_ID_OUT_OF_RANGE
    layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    st, flags = layer.status()
    assert st == moe.MOE_OK and flags == 0
    layer.close()


def test_decode_one_token_flags_and_recovery(torch_cuda):
    """One token with invalid routing (a repeated id, an id past E): each flag is raised
    alone, and the next valid calls match the oracle."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    inp = inputs.generate(1, 512, 256, 16, 4, seed=37)
    t = device_inputs(inp)
    layer = make_layer(inp, path=2)
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    bad = inp.ids.copy()
    bad[0, 2] = bad[0, 1]
    layer.forward(t["x"], torch.from_numpy(bad).to(dev()), t["scores"], t["w13"], t["w2"])
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING and flags == moe.MOE_DEV_ID_DUPLICATE
    bad = inp.ids.copy()
    bad[0, 3] = inp.E + 5
    layer.forward(t["x"], torch.from_numpy(bad).to(dev()), t["scores"], t["w13"], t["w2"])
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING and flags == moe.MOE_DEV_ID_OUT_OF_RANGE
    for _ in range(3):
        y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
        torch.cuda.synchronize()
        st, flags = layer.status()
        assert st == moe.MOE_OK and flags == 0
        check("y", np_of(y), ref, **BF16)
    layer.close()


# ------------------------------------------------------------------ mega (fused) decode

@pytest.mark.parametrize("T,d,I,E,k,routing", DECODE_SHAPES)
def test_mega_decode_small(torch_cuda, T, d, I, E, k, routing):
    """The fused decode (plan option mega: W13, activation and W2 chunked over I in one
    launch with FP32 partial outputs, then the combine launch) against the oracle, and
    bitwise repeatable."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    say("mega decode small", T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=17)
    t = device_inputs(inp)
    layer = moe.Layer(T, d, I, E, k, path=moe.MOE_PATH_DECODE, mega=True)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    y2 = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    st, flags = layer.status()
    assert flags == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    check("y (mega)", np_of(y), ref, **BF16)
    layer.close()


@pytest.mark.parametrize("name", ["decode1", "decode32"])
def test_mega_decode_full_size(torch_cuda, name):
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    say("mega decode full size", name)
    inp = inputs.generate_config(name, seed=0, with_dy=False)
    t = device_inputs(inp)
    layer = moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, mega=True)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    check("y (mega, all %d tokens)" % inp.T, np_of(y), ref, **BF16)
    layer.close()


@pytest.mark.parametrize("act,name", [(1, "geglu"), (2, "reglu")])
def test_mega_decode_gated_activations(torch_cuda, act, name):
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, d, I, E, k = 7, 512, 384, 16, 4
    say("mega decode", name, T, d, I, E, k)
    inp = inputs.generate(T, d, I, E, k, "uniform", seed=51)
    t = device_inputs(inp)
    layer = moe.Layer(T, d, I, E, k, mega=True, activation=act)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, act=act)
    check("y (mega, %s)" % name, np_of(y), ref, **BF16)
    layer.close()


def test_mega_decode_graph_replay_and_flags(torch_cuda):
    """Captured in a HIP graph, every replay equals the eager result bit for bit; invalid
    routing is flagged, and the next valid call equals the first."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    inp = inputs.generate(32, 512, 256, 64, 8, seed=23)
    t = device_inputs(inp)
    layer = moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, mega=True)
    y_eager = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    y_out = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"], y=y_out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"], y=y_out)
    for rep in range(4):
        y_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_out.view(torch.int16), y_eager.view(torch.int16)), rep
        layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
        torch.cuda.synchronize()
    assert layer.status()[1] == 0
    bad = inp.ids.copy()
    bad[3, 2] = bad[3, 0]
    bad[5, 1] = inp.E + 4
    layer.forward(t["x"], torch.from_numpy(bad).to(dev()), t["scores"], t["w13"], t["w2"])
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING
    assert flags & moe.MOE_DEV_ID_DUPLICATE and flags & moe.MOE_DEV_ID_OUT_OF_RANGE
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16))
    layer.close()


@pytest.mark.parametrize("mode", ["bf16", "mxfp8", "bf16-train", "mxfp8-train"])
def test_forward_flags_invalid_routing(torch_cuda, mode):
    """A grouped-GEMM call (forward, or forward + backward) whose routing holds
    out-of-range ids flags them and stays in bounds: the dispatch leaves the routed rows
    past the valid count unwritten (the workspace is filled with 0xFF bytes first, so
    their indices read as -1), and the next call with valid routing matches a fresh
    layer bit for bit."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    mx, train = mode.startswith("mxfp8"), mode.endswith("-train")
    inp = inputs.generate(300, 256, 128, 8, 2, "uniform", seed=23, with_dy=train)
    t = device_inputs(inp)
    prec = moe.MOE_MXFP8_E4M3 if mx else moe.MOE_BF16

    def run(layer, ids):
        if mx:
            w13q, w13s, w2q, w2s = layer.prepare_weights(t["w13"], t["w2"])
            y = layer.forward(t["x"], ids, t["scores"], w13q, w2q, w13s, w2s)
            if not train:
                return [y]
            w13t, w13ts, w2t, w2ts = layer.prepare_weights_backward(t["w13"], t["w2"])
            return [y] + list(layer.backward(t["dy"], t["x"], w13q, w2q, w13t=w13t, w13t_scale=w13ts,
                                             w2t=w2t, w2t_scale=w2ts))
        y = layer.forward(t["x"], ids, t["scores"], t["w13"], t["w2"])
        if not train:
            return [y]
        return [y] + list(layer.backward(t["dy"], t["x"], t["w13"], t["w2"]))

    def bits(v):
        return v.view(torch.int32) if v.dtype == torch.float32 else v.view(torch.int16)

    layer = moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, precision=prec, training=train, path=1)
    layer.workspace.fill_(0xFF)
    torch.cuda.synchronize()
    layer.status(clear=True)            # the fill set every status bit too
    bad = inp.ids.copy()
    bad[5, 0] = inp.E
    bad[17, 1] = -2
    run(layer, torch.from_numpy(bad).to(dev()))
    torch.cuda.synchronize()
    st, flags = layer.status(clear=True)
    assert st == moe.MOE_ERR_ROUTING and flags & moe.MOE_DEV_ID_OUT_OF_RANGE
    out = [v.clone() for v in run(layer, t["ids"])]
    torch.cuda.synchronize()
    st, flags = layer.status()
    assert st == moe.MOE_OK and flags == 0
    layer.close()
    fresh = moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, precision=prec, training=train, path=1)
    ref = run(fresh, t["ids"])
    torch.cuda.synchronize()
    for a, b in zip(out, ref):
        assert torch.equal(bits(a), bits(b))
    fresh.close()


# ------------------------------------------------------------------ backward

BWD_SHAPES = [
    (64, 256, 128, 8, 2, "uniform"),
    (400, 512, 384, 6, 3, "uniform"),
    (257, 320, 192, 5, 2, "uniform"),
    (300, 256, 128, 128, 8, "zipf"),
    (130, 128, 64, 1, 1, "uniform"),
    (320, 256, 128, 256, 32, "zipf"),       # E = 256, k = 32, skewed (empty and one-row experts)
]


@pytest.mark.parametrize("T,d,I,E,k,routing", BWD_SHAPES)
def test_backward_small(torch_cuda, T, d, I, E, k, routing):
    torch = torch_cuda
    say("backward small", T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=13, with_dy=True)
    t = device_inputs(inp)
    layer = make_layer(inp, training=True)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    dx, dw13, dw2, ds = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    y_ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    dx_ref, ds_ref = oracle.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    dw2_ref, dw13_ref = oracle.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    dw13_ref = dw13_ref.reshape(E, 2 * I, d)
    for name, got, ref in (("y", np_of(y), y_ref), ("dx", np_of(dx), dx_ref), ("ds", np_of(ds), ds_ref),
                           ("dw2", np_of(dw2), dw2_ref), ("dw13", np_of(dw13), dw13_ref)):
        check(name, got, ref, **(BF16_WGRAD if name.startswith("dw") else BF16))
    counts = np.bincount(inp.ids.ravel(), minlength=E)
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(dw2[e].view(torch.int16).cpu().numpy() == 0)
        assert np.all(dw13[e].view(torch.int16).cpu().numpy() == 0)
    layer.close()


@pytest.mark.parametrize("T,d,I,E,k,hot", [(13000, 320, 192, 3, 1, 12500), (7000, 256, 128, 4, 2, 6600)])
def test_backward_split_weight_gradient_tiles(torch_cuda, T, d, I, E, k, hot):
    """An expert with more than 192 stages of 32 routed rows (12500 rows: 3 pieces, 6600
    rows: 2 pieces) has its weight-gradient tiles cut along K into pieces whose FP32
    partial sums are added up in piece order after the product; the result must match
    the oracle and repeat bitwise."""
    import dataclasses
    torch = torch_cuda
    say("backward split tiles", T, d, I, E, k, hot)
    inp = inputs.generate(T, d, I, E, k, "uniform", seed=21, with_dy=True)
    rng = np.random.default_rng(5)
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        if t < hot:
            ids[t] = np.concatenate([[0], 1 + rng.permutation(E - 1)[:k - 1]])
        else:
            ids[t] = 1 + rng.permutation(E - 1)[:k]
    inp = dataclasses.replace(inp, ids=ids)
    t = device_inputs(inp)
    layer = make_layer(inp, training=True)
    layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    dx, dw13, dw2, ds = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])
    _, dw13b, dw2b, _ = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    assert torch.equal(dw13.view(torch.int16), dw13b.view(torch.int16))
    assert torch.equal(dw2.view(torch.int16), dw2b.view(torch.int16))
    dw2_ref, dw13_ref = oracle.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    dw13_ref = dw13_ref.reshape(E, 2 * I, d)
    check("dw2", np_of(dw2), dw2_ref, **BF16_WGRAD)
    check("dw13", np_of(dw13), dw13_ref, **BF16_WGRAD)
    layer.close()


@pytest.mark.parametrize("T,d,I,E,k,routing,hot", [(400, 512, 384, 6, 3, "uniform", 0),
                                                    (300, 256, 128, 128, 8, "zipf", 0),
                                                    (7000, 256, 128, 4, 2, "uniform", 6600)])
def test_backward_accumulates_weight_gradients(torch_cuda, T, d, I, E, k, routing, hot):
    """wgrad_accumulate: dW13 and dW2 start from random values and come back as those
    values plus the gradient (experts with no row bitwise unchanged); the hot case has an
    expert of 6600 rows, whose tiles are cut into pieces and summed by the fixup kernel."""
    import dataclasses
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    say("backward accumulate", T, d, I, E, k, routing, hot)
    inp = inputs.generate(T, d, I, E, k, routing, seed=41, with_dy=True)
    if hot:
        rng = np.random.default_rng(6)
        ids = np.empty((T, k), np.int32)
        for t in range(T):
            ids[t] = (np.concatenate([[0], 1 + rng.permutation(E - 1)[:k - 1]]) if t < hot
                      else 1 + rng.permutation(E - 1)[:k])
        inp = dataclasses.replace(inp, ids=ids)
    t = device_inputs(inp)
    layer = moe.Layer(T, d, I, E, k, training=True, wgrad_accumulate=True)
    g = torch.Generator(device="cpu").manual_seed(7)
    dw13_0 = (torch.randn((E, 2 * I, d), generator=g) * 0.05).to(torch.bfloat16).to(dev())
    dw2_0 = (torch.randn((E, d, I), generator=g) * 0.05).to(torch.bfloat16).to(dev())
    dw13, dw2 = dw13_0.clone(), dw2_0.clone()
    layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    layer.backward(t["dy"], t["x"], t["w13"], t["w2"], dw13=dw13, dw2=dw2)
    torch.cuda.synchronize()
    dw2_ref, dw13_ref = oracle.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    dw13_ref = dw13_ref.reshape(E, 2 * I, d) + np_of(dw13_0)
    dw2_ref = dw2_ref + np_of(dw2_0)
    check("dw13", np_of(dw13), dw13_ref, **BF16_WGRAD)
    check("dw2", np_of(dw2), dw2_ref, **BF16_WGRAD)
    counts = np.bincount(inp.ids.ravel(), minlength=E)
    for e in np.nonzero(counts == 0)[0]:
        assert torch.equal(dw13[e].view(torch.int16), dw13_0[e].view(torch.int16))
        assert torch.equal(dw2[e].view(torch.int16), dw2_0[e].view(torch.int16))
    layer.close()


@pytest.mark.parametrize("T,d,I,E,k,routing", [(400, 512, 384, 6, 3, "uniform"),     # h in the dX region
                                               (300, 128, 256, 8, 2, "uniform"),     # 2I > 3d: own region
                                               (300, 256, 128, 128, 8, "zipf")])
def test_backward_recompute_h_matches_saved(torch_cuda, T, d, I, E, k, routing):
    """recompute_h: the forward keeps no h and the backward recomputes it with the same
    kernel from the same x and W13.  Every gradient is checked against the oracle, and
    equals, bit for bit, that of a plan that saved h."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    say("backward recompute h", T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=43, with_dy=True)
    t = device_inputs(inp)
    outs = []
    for rec in (True, False):
        layer = moe.Layer(T, d, I, E, k, training=True, recompute_h=rec)
        y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
        dx, dw13, dw2, ds = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])
        torch.cuda.synchronize()
        assert layer.status()[1] == 0
        outs.append([v.clone() for v in (y, dx, dw13, dw2, ds)])
        layer.close()
    y_ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    dx_ref, ds_ref = oracle.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    dw2_ref, dw13_ref = oracle.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy)
    refs = (y_ref, dx_ref, dw13_ref.reshape(E, 2 * I, d), dw2_ref, ds_ref)
    for name, got, ref in zip(("y", "dx", "dw13", "dw2", "ds"), outs[0], refs):
        check(name + " (recomputed h)", np_of(got), ref, **(BF16_WGRAD if name.startswith("dw") else BF16))
    for name, a, b in zip(("y", "dx", "dw13", "dw2", "ds"), outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), name


def test_no_tokens(torch_cuda):
    """T = 0: the forward writes nothing and succeeds; the backward gives all-zero weight
    gradients (every expert is empty)."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    say("no tokens: T=0 d=256 I=128 E=8 k=2")
    d, I, E, k = 256, 128, 8, 2
    layer = moe.Layer(0, d, I, E, k, training=True)
    x = torch.empty((0, d), dtype=torch.bfloat16, device=dev())
    ids = torch.empty((0, k), dtype=torch.int32, device=dev())
    scores = torch.empty((0, k), dtype=torch.float32, device=dev())
    w13 = torch.randn((E, 2 * I, d), device=dev()).to(torch.bfloat16)
    w2 = torch.randn((E, d, I), device=dev()).to(torch.bfloat16)
    y = layer.forward(x, ids, scores, w13, w2)
    dw13 = torch.full((E, 2 * I, d), 7.0, dtype=torch.bfloat16, device=dev())
    dw2 = torch.full((E, d, I), 7.0, dtype=torch.bfloat16, device=dev())
    dx, dw13, dw2, ds = layer.backward(x, x, w13, w2, dw13=dw13, dw2=dw2)
    torch.cuda.synchronize()
    assert y.shape == (0, d) and dx.shape == (0, d) and ds.shape == (0, k)
    assert not torch.any(dw13.view(torch.int16) != 0)
    assert not torch.any(dw2.view(torch.int16) != 0)
    layer.close()


def test_backward_full_size_sampled(torch_cuda):
    torch = torch_cuda
    say("backward full size: train workload")
    inp = inputs.generate_config("train", seed=0, with_dy=True)
    t = device_inputs(inp)
    layer = make_layer(inp, training=True)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    dx, dw13, dw2, ds = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])
    dx2, dw13b, dw2b, ds2 = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    for a, b in ((dx, dx2), (dw13, dw13b), (dw2, dw2b), (ds, ds2)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    # 1024 tokens (every expert's first and last routed token among them) for dx and dS,
    # 64 of the 768 intermediate columns (the first and last of each 256-wide tile among
    # them) for dW13 and dW2, every expert
    rng = np.random.default_rng(7)
    toks = set(rng.choice(inp.T, size=1024, replace=False).tolist())
    for e in range(inp.E):
        te = np.nonzero((inp.ids == e).any(axis=1))[0]
        if len(te):
            toks.update((int(te[0]), int(te[-1])))
    toks = np.array(sorted(toks), np.int32)
    dx_ref, ds_ref = oracle.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy,
                                            toks=toks)
    check("dx (%d tokens)" % len(toks), np_of(dx)[toks], dx_ref, **BF16)
    check("ds", np_of(ds)[toks], ds_ref, **BF16)
    cols = set(rng.choice(inp.I, size=58, replace=False).tolist()) | {0, 255, 256, 511, 512, inp.I - 1}
    cols = np.array(sorted(cols), np.int32)
    dw2_ref, dw13_ref = oracle.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy,
                                          icols=cols)
    dw2_np = np_of(dw2)[:, :, cols]
    dw13_np = np.stack([np_of(dw13[:, cols, :]), np_of(dw13[:, inp.I + cols, :])], axis=1)
    check("dw2 (%d columns)" % len(cols), dw2_np, dw2_ref, **BF16_WGRAD)
    check("dw13", dw13_np, dw13_ref, **BF16_WGRAD)
    counts = np.bincount(inp.ids.ravel(), minlength=inp.E)
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) >= 8
    for e in empty:
        assert not torch.any(dw2[e].view(torch.int16) != 0)
        assert not torch.any(dw13[e].view(torch.int16) != 0)
    layer.close()


# ------------------------------------------------------------------ MXFP8 conversion

def test_quantize_bit_exact(torch_cuda):
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    rng = np.random.default_rng(0)
    rows, K = 300, 256
    v = (rng.standard_normal((rows, K)) * np.exp(rng.normal(0, 4, (rows, 1)))).astype(np.float32)
    v[0] = 0.0
    v[1, :32] = -0.0
    v[2] = 448.0 * np.sign(rng.standard_normal(K))
    v[3] = 1e-40                                         # float32 subnormal: bf16 subnormal after rounding
    v[4] = 3.0e38
    bits = inputs.to_bf16_bits(v)
    bits[5] = rng.integers(0, 65536, K).astype(np.uint16)   # arbitrary bit patterns ...
    finite = np.isfinite((bits[5].astype(np.uint32) << 16).view(np.float32))
    bits[5][~finite] = 0                                     # ... except Inf / NaN
    src = bf16_dev(bits)
    codes = torch.empty((rows, K), dtype=torch.uint8, device=dev())
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev())
    moe.moe_quantize_mxfp8(src.data_ptr(), rows, K, codes.data_ptr(), scales.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(bits)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_every_bf16_value(torch_cuda):
    """Every finite BF16 value through the device E4M3/E8M0 conversion at 18 block scales:
    the values, sorted by magnitude, fill blocks 31 at a time behind an anchor element of
    2^j times the group's largest magnitude (j = 0..17), so each value is converted at
    scaled magnitudes from the top of the E4M3 range down through its subnormal steps
    to zero.  Codes and scale bytes must equal the oracle's bit for bit."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    allbits = np.arange(65536, dtype=np.uint32)
    vals = (allbits << 16).view(np.float32)
    fin = allbits[np.isfinite(vals)].astype(np.uint16)
    fin = fin[np.argsort(np.abs((fin.astype(np.uint32) << 16).view(np.float32)), kind="stable")]
    groups = -(-fin.size // 31)
    fin = np.concatenate([fin, np.zeros(groups * 31 - fin.size, np.uint16)]).reshape(groups, 31)
    gmax = np.abs((fin.astype(np.uint32) << 16).view(np.float32)).max(axis=1)
    blocks = []
    for j in range(18):
        anchor = gmax.astype(np.float64) * 2.0 ** j
        ok = anchor < 3.0e38
        a_bits = inputs.to_bf16_bits(anchor[ok].astype(np.float32))
        assert np.array_equal((a_bits.astype(np.uint32) << 16).view(np.float32), anchor[ok])   # exact
        blocks.append(np.concatenate([a_bits[:, None], fin[ok]], axis=1))
    blocks = np.concatenate(blocks)
    pad = -len(blocks) % 8
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.uint16)])
    bits = np.ascontiguousarray(blocks.reshape(-1, 256))
    rows, K = bits.shape
    say("quantize every finite bf16 value: %d blocks" % (rows * K // 32))
    src = bf16_dev(bits)
    codes = torch.empty((rows, K), dtype=torch.uint8, device=dev())
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev())
    moe.moe_quantize_mxfp8(src.data_ptr(), rows, K, codes.data_ptr(), scales.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(bits)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_prepare_weights_bit_exact(torch_cuda):
    torch = torch_cuda
    inp = inputs.generate(16, 256, 128, 4, 2, seed=3)
    t = device_inputs(inp)
    layer = make_layer(inp)
    w13_q, w13_s, w2_q, w2_s = layer.prepare_weights(t["w13"], t["w2"])
    torch.cuda.synchronize()
    r13 = oracle.mx_quantize(inp.w13)
    r2 = oracle.mx_quantize(inp.w2)

    def row_major(s_bm, shape):
        # block-major [K/128, N, 4] -> [N, K/32], N = all rows of the weight
        g, n, _ = s_bm.shape
        return s_bm.transpose(1, 0, 2).reshape(n, 4 * g).reshape(shape)

    assert np.array_equal(w13_q.cpu().numpy(), r13[0])
    assert np.array_equal(row_major(w13_s.cpu().numpy(), r13[1].shape), r13[1])
    assert np.array_equal(w2_q.cpu().numpy(), r2[0])
    assert np.array_equal(row_major(w2_s.cpu().numpy(), r2[1].shape), r2[1])
    layer.close()


# ------------------------------------------------------------------ MXFP8 forward


MX_SHAPES = [
    # T, d, I, E, k, routing
    (64, 256, 128, 8, 2, "uniform"),
    (300, 512, 256, 6, 3, "uniform"),      # ragged row tiles
    (257, 256, 384, 5, 2, "uniform"),      # three W13 column tiles
    (200, 256, 128, 64, 8, "zipf"),        # skew and empty experts
    (130, 256, 128, 1, 1, "uniform"),      # dense layer
    (100, 2304, 128, 4, 2, "uniform"),     # 18 scale words per row: a partial second group chunk
    (320, 256, 128, 256, 32, "zipf"),      # the expert and top-k limits (E = 256, k = 32), skewed
]


def _mx_run(torch, inp, t):
    from mixture_experts_routed_dispatch_amd import moe
    layer = moe.Layer(inp.T, inp.d, inp.I, inp.E, inp.k, precision=moe.MOE_MXFP8_E4M3)
    w13q, w13s, w2q, w2s = layer.prepare_weights(t["w13"], t["w2"])
    y = layer.forward(t["x"], t["ids"], t["scores"], w13q, w2q, w13s, w2s)
    y2 = layer.forward(t["x"], t["ids"], t["scores"], w13q, w2q, w13s, w2s)
    torch.cuda.synchronize()
    st, flags = layer.status()
    assert flags == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))      # bitwise deterministic
    layer.close()
    return y


def _prepared_f32(w):
    return oracle.mx_dequantize(*oracle.mx_quantize(w))


@pytest.mark.parametrize("T,d,I,E,k,routing", MX_SHAPES)
def test_mxfp8_forward_small(torch_cuda, T, d, I, E, k, routing):
    torch = torch_cuda
    say("mxfp8 forward small", T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=19)
    t = device_inputs(inp)
    y = np_of(_mx_run(torch, inp, t))
    w13f, w2f = _prepared_f32(inp.w13), _prepared_f32(inp.w2)
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, w13f, w2f)
    ref_q = oracle.forward_tokens_mx(inp.x, inp.ids, inp.scores, w13f, w2f)
    check("y vs fp32 oracle", y, ref, **MX)
    check("y vs quantizing oracle", y, ref_q, **MX_QUANT)


def test_mxfp8_forward_full_size_sampled(torch_cuda):
    torch = torch_cuda
    say("mxfp8 forward full size: T=16384 d=4096 I=2048 E=64 k=8")
    inp = inputs.generate_config("mxfp8", seed=0)
    t = device_inputs(inp)
    y = np_of(_mx_run(torch, inp, t))
    del t
    torch.cuda.empty_cache()
    rng = np.random.default_rng(9)
    toks = np.sort(rng.choice(inp.T, size=256, replace=False)).astype(np.int32)
    toks[0] = 0
    toks[-1] = inp.T - 1
    w13f, w2f = _prepared_f32(inp.w13), _prepared_f32(inp.w2)
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, w13f, w2f, toks=toks)
    ref_q = oracle.forward_tokens_mx(inp.x, inp.ids, inp.scores, w13f, w2f, toks=toks)
    check("y vs fp32 oracle", y[toks], ref, **MX)
    check("y vs quantizing oracle", y[toks], ref_q, **MX_QUANT)


# ------------------------------------------------------------------ GeGLU / ReGLU

ACTS = [(1, "geglu"), (2, "reglu")]


@pytest.mark.parametrize("act,name", ACTS)
@pytest.mark.parametrize("T,d,I,E,k,routing,path", [(600, 512, 384, 6, 3, "uniform", 1),
                                                    (257, 320, 192, 5, 2, "uniform", 1),
                                                    (1, 256, 128, 16, 4, "uniform", 2),
                                                    (7, 512, 384, 16, 4, "uniform", 2)])
def test_forward_gated_activations(torch_cuda, act, name, T, d, I, E, k, routing, path):
    """GeGLU (exact GELU) and ReGLU W13 epilogues on the grouped-GEMM path (1) and the
    decode path (2, one and seven tokens) against the oracle with the same activation."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    say("forward", name, T, d, I, E, k, routing, "path", path)
    inp = inputs.generate(T, d, I, E, k, routing, seed=51)
    t = device_inputs(inp)
    layer = moe.Layer(T, d, I, E, k, path=path, activation=act)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, act=act)
    check("y", np_of(y), ref, **BF16)
    layer.close()


@pytest.mark.parametrize("act,name", ACTS)
@pytest.mark.parametrize("T,d,I,E,k,routing", [(400, 512, 384, 6, 3, "uniform"), (300, 256, 128, 128, 8, "zipf")])
def test_backward_gated_activations(torch_cuda, act, name, T, d, I, E, k, routing):
    """The backward of GeGLU / ReGLU (f'(g) in the W2 DGRAD epilogue, f(g) in du and in
    the saved a) against the oracle's gradients with the same activation."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    say("backward", name, T, d, I, E, k, routing)
    inp = inputs.generate(T, d, I, E, k, routing, seed=53, with_dy=True)
    t = device_inputs(inp)
    layer = moe.Layer(T, d, I, E, k, training=True, activation=act)
    y = layer.forward(t["x"], t["ids"], t["scores"], t["w13"], t["w2"])
    dx, dw13, dw2, ds = layer.backward(t["dy"], t["x"], t["w13"], t["w2"])
    torch.cuda.synchronize()
    y_ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, act=act)
    dx_ref, ds_ref = oracle.backward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy, act=act)
    dw2_ref, dw13_ref = oracle.wgrad_cols(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dy, act=act)
    for name, got, ref in (("y", np_of(y), y_ref), ("dx", np_of(dx), dx_ref), ("ds", np_of(ds), ds_ref),
                           ("dw2", np_of(dw2), dw2_ref), ("dw13", np_of(dw13), dw13_ref.reshape(E, 2 * I, d))):
        check(name, got, ref, **(BF16_WGRAD if name.startswith("dw") else BF16))
    layer.close()


@pytest.mark.parametrize("act,name", ACTS)
def test_mxfp8_forward_gated_activations(torch_cuda, act, name):
    """The MXFP8 W13 epilogue with GeGLU / ReGLU before the E4M3 re-quantization."""
    torch = torch_cuda
    from mixture_experts_routed_dispatch_amd import moe
    T, d, I, E, k = 300, 512, 256, 6, 3
    say("mxfp8 forward", name, T, d, I, E, k)
    inp = inputs.generate(T, d, I, E, k, "uniform", seed=57)
    t = device_inputs(inp)
    layer = moe.Layer(T, d, I, E, k, precision=moe.MOE_MXFP8_E4M3, activation=act)
    w13q, w13s, w2q, w2s = layer.prepare_weights(t["w13"], t["w2"])
    y = np_of(layer.forward(t["x"], t["ids"], t["scores"], w13q, w2q, w13s, w2s))
    torch.cuda.synchronize()
    assert layer.status()[1] == 0
    w13f, w2f = _prepared_f32(inp.w13), _prepared_f32(inp.w2)
    ref = oracle.forward_tokens(inp.x, inp.ids, inp.scores, w13f, w2f, act=act)
    ref_q = oracle.forward_tokens_mx(inp.x, inp.ids, inp.scores, w13f, w2f, act=act)
    check("y vs fp32 oracle", y, ref, **MX)
    check("y vs quantizing oracle", y, ref_q, **MX_QUANT)
    layer.close()

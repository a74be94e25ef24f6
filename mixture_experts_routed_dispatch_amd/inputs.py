"""Seeded synthetic inputs for the routed expert layer.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle; it holds none of the layer's arithmetic (no dispatch, GEMM, SwiGLU or
combine), only the random draws and the BF16 rounding of the drawn values.

Workloads follow the shapes the pages use: the nvfp4moe README's inference
example (d=2048, I=768, E=16, k=8, 8192 tokens, section "MoE layer") and
training example (T=8192, E=128, k=8, section "Training"), its "skewed
routing, and empty experts" (section "Supported kernel surface") and
"batch-one decode" (section "MoE layer"), and the blog post's MXFP8 E4M3
mode ("What it is selling").  The pages name no dataset.

Recipe (numpy PCG64, one generator per call, fixed draw order):
  x ~ N(0, 1); W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/I), each drawn in float32 and
  rounded to BF16 (nearest even); routing; score logits ~ N(0, 1) with
  scores = softmax over the k picks (float32); optional dY ~ N(0, 1) BF16.
  Uniform routing: the k smallest of argsort(uniform(T, E)) per token.
  Zipf routing: a seeded permutation gives expert e the rank pi(e) in 1..E,
  weight rank^-s (s = 1.2) for the E - n_empty best ranks and 0 for the
  n_empty worst (forced empty), and ids are the top-k of log(weight) +
  Gumbel noise, i.e. sampling without replacement proportional to weight.
"""
from __future__ import annotations

import dataclasses

import numpy as np

CONFIGS = {
    # name: (T, d, I, E, k, routing)
    "tiny": dict(T=64, d=256, I=128, E=8, k=2, routing="uniform"),
    "prefill": dict(T=8192, d=2048, I=768, E=16, k=8, routing="uniform"),
    "train": dict(T=8192, d=2048, I=768, E=128, k=8, routing="zipf"),
    "decode1": dict(T=1, d=2048, I=768, E=128, k=8, routing="uniform"),
    "decode32": dict(T=32, d=2048, I=768, E=128, k=8, routing="uniform"),
    "mxfp8": dict(T=16384, d=4096, I=2048, E=64, k=8, routing="uniform"),
}


@dataclasses.dataclass
class MoEInputs:
    T: int
    d: int
    I: int
    E: int
    k: int
    x: np.ndarray        # uint16 BF16 bits [T, d]
    w13: np.ndarray      # uint16 BF16 bits [E, 2I, d]: rows [0, I) gate (W1), [I, 2I) up (W3)
    w2: np.ndarray       # uint16 BF16 bits [E, d, I]
    ids: np.ndarray      # int32 [T, k], distinct per row
    scores: np.ndarray   # float32 [T, k]
    dy: np.ndarray | None = None  # uint16 BF16 bits [T, d]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return to_bf16_bits(v)


def uniform_routing(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    return np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :k].astype(np.int32)


def zipf_routing(rng: np.random.Generator, T: int, E: int, k: int, s: float = 1.2,
                 n_empty: int = 8) -> np.ndarray:
    if k > E - n_empty:
        raise ValueError("top-k larger than the number of experts that may receive rows")
    rank = rng.permutation(E) + 1                      # rank of expert e, 1..E
    w = np.where(rank <= E - n_empty, rank.astype(np.float64) ** (-s), 0.0)
    with np.errstate(divide="ignore"):
        logw = np.log(w)
    keys = logw[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def softmax_scores(rng: np.random.Generator, T: int, k: int) -> np.ndarray:
    logits = rng.standard_normal((T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def generate(T: int, d: int, I: int, E: int, k: int, routing: str = "uniform", seed: int = 0,
             with_dy: bool = False, zipf_s: float = 1.2, n_empty: int = 8) -> MoEInputs:
    rng = np.random.default_rng(seed)
    x = _normal_bf16(rng, (T, d), 1.0)
    w13 = np.empty((E, 2 * I, d), np.uint16)
    w2 = np.empty((E, d, I), np.uint16)
    for e in range(E):                               # W1 for all experts, then W3, then W2
        w13[e, :I] = _normal_bf16(rng, (I, d), d ** -0.5)
    for e in range(E):
        w13[e, I:] = _normal_bf16(rng, (I, d), d ** -0.5)
    for e in range(E):
        w2[e] = _normal_bf16(rng, (d, I), I ** -0.5)
    if routing == "uniform":
        ids = uniform_routing(rng, T, E, k)
    elif routing == "zipf":
        ids = zipf_routing(rng, T, E, k, zipf_s, n_empty)
    else:
        raise ValueError("unknown routing %r" % routing)
    scores = softmax_scores(rng, T, k)
    dy = _normal_bf16(rng, (T, d), 1.0) if with_dy else None
    return MoEInputs(T, d, I, E, k, x, w13, w2, ids, scores, dy)


def generate_config(name: str, seed: int = 0, with_dy: bool | None = None) -> MoEInputs:
    c = dict(CONFIGS[name])
    if with_dy is None:
        with_dy = name == "train"
    return generate(c["T"], c["d"], c["I"], c["E"], c["k"], c["routing"], seed, with_dy)


def disjoint_routings(E: int, k: int, count: int, seed: int = 0) -> np.ndarray:
    """`count` single-token routings [count, k] whose expert sets are pairwise disjoint
    while count*k <= E (a seeded partition of the experts; used to keep each decode
    call on weights the previous calls did not touch)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(E).astype(np.int32)
    out = np.empty((count, k), np.int32)
    for c in range(count):
        idx = [(c * k + j) % E for j in range(k)]
        out[c] = perm[idx]
    return out

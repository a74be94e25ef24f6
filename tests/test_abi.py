"""The C-ABI library (include/moe.h): it loads without a GPU, exports every
declared entry point, and rejects bad calls on the host before touching the
device (the plan's limits follow the nvfp4moe README, "Limits"; the refusal
of unsupported modes at creation follows the blog post, "What it is
selling")."""
import ctypes
import os
import re

import pytest

from mixture_experts_routed_dispatch_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from mixture_experts_routed_dispatch_amd import build
        build.build()
    return moe.lib()


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert set(syms) == set(moe.EXPORTS)
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert len(moe.status_string(st)) >= 2 and moe.status_string(st) != "unknown status"
    assert moe.status_string(-99) == "unknown status"


@pytest.mark.parametrize("cfg,expect", [
    (dict(T=64, d=256, I=128, E=8, k=2), moe.MOE_OK),
    (dict(T=0, d=256, I=128, E=8, k=2), moe.MOE_OK),                 # empty batch is valid
    (dict(T=-1, d=256, I=128, E=8, k=2), moe.MOE_ERR_INVALID_ARG),
    (dict(T=8, d=0, I=128, E=8, k=2), moe.MOE_ERR_INVALID_ARG),
    (dict(T=8, d=256, I=128, E=8, k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(T=8, d=250, I=128, E=8, k=2), moe.MOE_ERR_UNSUPPORTED),    # K not a multiple of 64
    (dict(T=8, d=256, I=100, E=8, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=8, d=256, I=128, E=257, k=2), moe.MOE_ERR_UNSUPPORTED),  # > 256 experts
    (dict(T=8, d=256, I=128, E=4, k=5), moe.MOE_ERR_UNSUPPORTED),    # k > E
    (dict(T=16385, d=256, I=128, E=64, k=8), moe.MOE_ERR_UNSUPPORTED),  # > 131072 rows
    (dict(T=16384, d=256, I=128, E=64, k=8), moe.MOE_OK),            # exactly at the limit
    (dict(T=8, d=256, I=128, E=8, k=2, precision=7), moe.MOE_ERR_INVALID_ARG),
    (dict(T=8, d=256, I=128, E=8, k=2, training=2), moe.MOE_ERR_INVALID_ARG),
    (dict(T=8, d=256, I=128, E=8, k=2, path=9), moe.MOE_ERR_INVALID_ARG),
    (dict(T=8, d=256, I=128, E=8, k=2, precision=1, training=1), moe.MOE_OK),   # MXFP8 training
    (dict(T=16384, d=4096, I=2048, E=64, k=8, precision=1, training=1, recompute_h=1), moe.MOE_OK),
    (dict(T=8, d=256, I=128, E=8, k=2, precision=1, path=2), moe.MOE_ERR_UNSUPPORTED),  # no MXFP8 decode
    (dict(T=8, d=256, I=128, E=8, k=2, precision=1), moe.MOE_OK),            # MXFP8 forward
    (dict(T=16384, d=4096, I=2048, E=64, k=8, precision=1), moe.MOE_OK),     # the MXFP8 workload
    (dict(T=8, d=192, I=128, E=8, k=2, precision=1), moe.MOE_ERR_UNSUPPORTED),  # d % 256
    (dict(T=8, d=256, I=192, E=8, k=2, precision=1), moe.MOE_ERR_UNSUPPORTED),  # I % 128
    (dict(T=8, d=32768, I=16384, E=8, k=2), moe.MOE_ERR_UNSUPPORTED),      # 32-bit offsets
    (dict(T=32, d=2048, I=768, E=128, k=8, path=2), moe.MOE_OK),      # decode: T*k <= 256
    (dict(T=33, d=2048, I=768, E=128, k=8, path=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=1, d=256, I=128, E=8, k=2, path=2, training=1), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=0, d=256, I=128, E=8, k=2, path=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=64, d=256, I=128, E=8, k=2, training=1, wgrad_accumulate=1), moe.MOE_OK),
    (dict(T=64, d=256, I=128, E=8, k=2, wgrad_accumulate=1), moe.MOE_ERR_UNSUPPORTED),  # no backward
    (dict(T=64, d=256, I=128, E=8, k=2, training=1, wgrad_accumulate=2), moe.MOE_ERR_INVALID_ARG),
    (dict(T=64, d=256, I=128, E=8, k=2, training=1, recompute_h=1), moe.MOE_OK),
    (dict(T=64, d=256, I=128, E=8, k=2, recompute_h=1), moe.MOE_ERR_UNSUPPORTED),     # nothing to recompute
    (dict(T=64, d=256, I=128, E=8, k=2, training=1, recompute_h=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(T=64, d=256, I=128, E=8, k=2, activation=1), moe.MOE_OK),
    (dict(T=8, d=256, I=128, E=8, k=2, precision=1, activation=2), moe.MOE_OK),
    (dict(T=64, d=256, I=128, E=8, k=2, activation=3), moe.MOE_ERR_INVALID_ARG),
    (dict(T=1, d=2048, I=768, E=128, k=8, mega=1), moe.MOE_OK),              # fused decode
    (dict(T=32, d=2048, I=768, E=128, k=8, path=2, mega=1), moe.MOE_OK),
    (dict(T=64, d=256, I=128, E=8, k=8, mega=1), moe.MOE_ERR_UNSUPPORTED),    # not a decode plan
    (dict(T=8, d=256, I=128, E=8, k=2, path=1, mega=1), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=8, d=256, I=128, E=8, k=2, training=1, mega=1), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=8, d=256, I=128, E=8, k=2, mega=2), moe.MOE_ERR_INVALID_ARG),
])
def test_plan_validation(L, cfg, expect):
    c = moe.MoeConfig(cfg["T"], cfg["d"], cfg["I"], cfg["E"], cfg["k"], cfg.get("precision", 0),
                      cfg.get("training", 0), cfg.get("path", 0), cfg.get("wgrad_accumulate", 0),
                      cfg.get("recompute_h", 0), cfg.get("activation", 0), cfg.get("mega", 0))
    h = ctypes.c_void_p()
    st = L.moe_plan(ctypes.byref(c), ctypes.byref(h))
    assert st == expect
    if st == moe.MOE_OK:
        assert h.value
        assert L.moe_workspace_bytes(h) > 0
        L.moe_plan_destroy(h)
    else:
        assert not h.value


def test_null_arguments_and_unbound_workspace(L):
    assert L.moe_plan(None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_bytes(None) == 0
    assert L.moe_plan_destroy(None) == moe.MOE_OK
    plan = moe.moe_plan(64, 256, 128, 8, 2, training=1)
    w = moe.weights(0x1000, 0x2000)
    # no workspace bound yet: rejected before any launch
    assert L.moe_forward(plan, 0x1000, 0x1000, 0x1000, ctypes.byref(w), 0x1000, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(plan, 0x10, 0x10, 0x10, 0x10, 0x10, 0x10, None) == moe.MOE_ERR_WORKSPACE
    # NULL tensors
    assert L.moe_forward(plan, None, 0x1000, 0x1000, ctypes.byref(w), 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_forward(plan, 0x1000, 0x1000, 0x1000, None, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    wn = moe.weights(0, 0x2000)
    assert L.moe_forward(plan, 0x1000, 0x1000, 0x1000, ctypes.byref(wn), 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    # bind rejects misaligned or short buffers without touching the device
    assert L.moe_bind_workspace(plan, 0x1001, 1 << 30) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_bind_workspace(plan, 0x1000, 16) == moe.MOE_ERR_WORKSPACE
    assert L.moe_bind_workspace(plan, None, 1 << 30) == moe.MOE_ERR_INVALID_ARG
    # backward: workspace checked after arguments
    assert L.moe_backward(plan, 0x10, 0x10, ctypes.byref(w), 0x10, 0x10, 0x10, 0x10, None) == moe.MOE_ERR_WORKSPACE
    f = ctypes.c_int32()
    assert L.moe_get_status(plan, ctypes.byref(f), 0, None) == moe.MOE_ERR_WORKSPACE
    moe.moe_plan_destroy(plan)


def test_backward_on_inference_plan_is_a_state_error(L):
    plan = moe.moe_plan(64, 256, 128, 8, 2, training=0)
    w = moe.weights(0x1000, 0x2000)
    assert L.moe_backward(plan, 0x10, 0x10, ctypes.byref(w), 0x10, 0x10, 0x10, 0x10, None) == moe.MOE_ERR_STATE
    moe.moe_plan_destroy(plan)


def test_quantize_argument_checks(L):
    assert L.moe_quantize_mxfp8(0x10, 4, 48, 0x10, 0x10, None) == moe.MOE_ERR_INVALID_ARG  # K % 32
    assert L.moe_quantize_mxfp8(None, 4, 64, 0x10, 0x10, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_mxfp8(0x10, -1, 64, 0x10, 0x10, None) == moe.MOE_ERR_INVALID_ARG


def test_workspace_grows_with_training_state(L):
    a = moe.moe_plan(8192, 2048, 768, 16, 8, training=0)
    b = moe.moe_plan(8192, 2048, 768, 16, 8, training=1)
    R = 8192 * 8
    assert moe.moe_workspace_bytes(a) >= R * (768 + 2048) * 2
    assert moe.moe_workspace_bytes(b) >= moe.moe_workspace_bytes(a) + R * (4 * 768 + 2048) * 2
    moe.moe_plan_destroy(a)
    moe.moe_plan_destroy(b)


def test_oracle_and_library_share_nothing():
    """The oracle package and the HIP library do not import or include each other."""
    pkg = os.path.join(ROOT, "mixture_experts_routed_dispatch_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    src = f.read()
                assert "import oracle" not in src and "from oracle" not in src, fn
                assert "moe_oracle" not in src and "liborc" not in src, fn
    with open(os.path.join(ROOT, "oracle", "moe_oracle.c")) as f:
        src = f.read()
    assert "#include \"" not in src
    with open(os.path.join(ROOT, "oracle", "__init__.py")) as f:
        src = f.read()
    assert "mixture_experts_routed_dispatch_amd" not in src


def test_plan_explain_mxfp8_regions(L):
    """An MXFP8 plan's report lists the conversion regions with the sizes the layouts
    fix: codes of x [T, d], its scales [T, d/32], their routed block-major copy
    [d/128, R, 4], codes of a [R, I] and their scales; the BF16 `a` region is absent."""
    T, d, I, E, k = 16384, 4096, 2048, 64, 8
    plan = moe.moe_plan(T, d, I, E, k, precision=moe.MOE_MXFP8_E4M3)
    try:
        R = T * k
        text = moe.moe_plan_explain(plan)
        sizes = {}
        for line in text.splitlines():
            f = line.split()
            if line.startswith("  ") and len(f) >= 3 and f[1].isdigit():
                sizes[f[0]] = int(f[1])
        assert sizes["xq"] == T * d and sizes["xs"] == T * d // 32
        assert sizes["xs_routed"] == R * d // 32
        assert sizes["aq"] == R * I and sizes["as"] == R * I // 32
        assert sizes["o"] == 2 * R * d and "a" not in sizes
        assert sum(sizes.values()) <= moe.moe_workspace_bytes(plan)
    finally:
        moe.moe_plan_destroy(plan)


def test_plan_explain_mxfp8_training(L):
    """An MXFP8 training plan keeps a in BF16 for dW2 and holds the backward's quantized
    operands: dO along d (codes + scales, R d 33/32 bytes), (dg, du) along 2I, and the
    token-layout weight-gradient operands over T*k + 128 E rows (P: max(I, d) features,
    Q: max(d, 2I)); recomputing h puts it in the token-layout region, R * 2I * 2 bytes less."""
    T, d, I, E, k = 16384, 4096, 2048, 64, 8
    keep = moe.moe_plan(T, d, I, E, k, precision=moe.MOE_MXFP8_E4M3, training=1)
    rec = moe.moe_plan(T, d, I, E, k, precision=moe.MOE_MXFP8_E4M3, training=1, recompute_h=1)
    try:
        R, ntok = T * k, T * k + 128 * E

        def sizes(plan):
            out = {}
            for line in moe.moe_plan_explain(plan).splitlines():
                f = line.split()
                if line.startswith("  ") and len(f) >= 3 and f[1].isdigit():
                    out[f[0]] = int(f[1])
            return out
        sk, sr = sizes(keep), sizes(rec)
        assert sk["a"] == 2 * R * I and sk["h"] == 2 * R * 2 * I
        assert sk["dOq"] == R * d * 33 // 32 and sk["dhq"] == R * 2 * I * 33 // 32
        assert sk["tokP"] == max(I, d) * ntok * 33 // 32 and sk["tokQ"] == max(d, 2 * I) * ntok * 33 // 32
        assert "h" not in sr and "xg" not in sk and "dys" not in sk
        assert moe.moe_workspace_bytes(keep) - moe.moe_workspace_bytes(rec) == 2 * R * 2 * I
        assert "first h, recomputed" in moe.moe_plan_explain(rec)
    finally:
        moe.moe_plan_destroy(keep)
        moe.moe_plan_destroy(rec)


def test_plan_explain_and_recompute_workspace(L):
    """The report names every region with its bytes and the total the plan asks for; a
    training plan that recomputes h needs R * 2I * 2 bytes less (h takes the place of the
    backward's dX / weight-gradient operands), which the report says."""
    T, d, I, E, k = 8192, 2048, 768, 128, 8
    keep = moe.moe_plan(T, d, I, E, k, training=1)
    rec = moe.moe_plan(T, d, I, E, k, training=1, recompute_h=1)
    inf = moe.moe_plan(T, d, I, E, k, training=0)
    try:
        R = T * k
        assert moe.moe_workspace_bytes(keep) - moe.moe_workspace_bytes(rec) == 2 * R * 2 * I
        for plan in (keep, rec, inf):
            text = moe.moe_plan_explain(plan)
            assert ("workspace %d bytes" % moe.moe_workspace_bytes(plan)) in text
            for name in ("m_indptr", "gather", "slots", "probs", "o"):
                assert "\n  %s " % name in text
            assert "limits: T*k <= 131072" in text
            assert len(text) == int(L.moe_plan_explain(ctypes.c_void_p(plan), None, 0))
        t_keep, t_rec = moe.moe_plan_explain(keep), moe.moe_plan_explain(rec)
        assert "h saved by the forward" in t_keep and "\n  h " in t_keep
        assert "h recomputed in the backward, in the dX / WGRAD-operand region" in t_rec
        assert "\n  h " not in t_rec
        # saved bytes: the dispatch, a and o (and h unless recomputed)
        saved = lambda t: int(t.split("kept from the training forward for the backward: ")[1].split(" ")[0])
        assert saved(t_keep) - saved(t_rec) == 2 * R * 2 * I
        assert saved(moe.moe_plan_explain(inf)) == 0
        # truncation: at most len - 1 characters and a NUL
        buf = ctypes.create_string_buffer(20)
        n = L.moe_plan_explain(ctypes.c_void_p(keep), buf, 20)
        assert n == len(t_keep) and buf.value.decode() == t_keep[:19]
        assert L.moe_plan_explain(None, None, 0) == 0
    finally:
        for plan in (keep, rec, inf):
            moe.moe_plan_destroy(plan)

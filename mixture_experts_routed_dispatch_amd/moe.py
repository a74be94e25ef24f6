"""Python binding of libmoe (include/moe.h): argument marshalling only.

Each function has the name of the C entry point it calls and takes plain
integers for device pointers and streams.  Every step of the layer runs in
the HIP kernels of libmoe; there is no other implementation to fall back to,
so a missing library raises instead of computing anything.

`Layer` is a convenience owner of one plan plus a workspace tensor allocated
with torch (PyTorch supplies device memory and streams, nothing else).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_STATE = -4
MOE_ERR_HIP = -5
MOE_ERR_ROUTING = -6
MOE_ERR_TOO_LARGE = -7
MOE_STATIC_SCRATCH_BYTES = 32 << 20

MOE_BF16 = 0
MOE_MXFP8_E4M3 = 1

MOE_PATH_AUTO = 0
MOE_PATH_PREFILL = 1
MOE_PATH_DECODE = 2

MOE_DEV_ID_OUT_OF_RANGE = 1
MOE_DEV_ID_DUPLICATE = 2
MOE_DEV_BAD_INDPTR = 4
MOE_ACT_SWIGLU, MOE_ACT_GEGLU, MOE_ACT_REGLU = 0, 1, 2

# every symbol include/moe.h declares
EXPORTS = ("moe_plan", "moe_workspace_bytes", "moe_bind_workspace", "moe_plan_destroy",
           "moe_dispatch", "moe_quantize_mxfp8", "moe_prepare_weights", "moe_prepare_weights_backward",
           "moe_forward", "moe_forward_static",
           "moe_forward_routed",
           "moe_backward", "moe_get_status", "moe_status_string", "moe_profile", "moe_plan_explain",
           "moe_profile_read")

STAGES = ("dispatch", "quant_x", "w13", "w2", "combine", "score_grad", "dgrad_w2", "wgrad_w2",
          "dgrad_w13", "wgrad_w13", "dx_combine", "decode_w13", "decode_w2", "wgrad_rows", "recompute_h",
          "mega", "quant_do", "act_bwd", "quant_t")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, status_string(status), status))


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("training", ctypes.c_int32), ("path", ctypes.c_int32),
                ("wgrad_accumulate", ctypes.c_int32), ("recompute_h", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("mega", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("w13t", ctypes.c_void_p), ("w13t_scale", ctypes.c_void_p),
                ("w2t", ctypes.c_void_p), ("w2t_scale", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (run __graft_entry__.build()); "
                               "there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.moe_plan.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(vp)]
        L.moe_plan.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [vp]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_plan_explain.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
        L.moe_plan_explain.restype = ctypes.c_size_t
        L.moe_bind_workspace.argtypes = [vp, vp, ctypes.c_size_t]
        L.moe_bind_workspace.restype = ctypes.c_int
        L.moe_plan_destroy.argtypes = [vp]
        L.moe_plan_destroy.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [vp] * 8
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_quantize_mxfp8.argtypes = [vp, i64, i32, vp, vp, vp]
        L.moe_quantize_mxfp8.restype = ctypes.c_int
        L.moe_prepare_weights.argtypes = [vp] * 8
        L.moe_prepare_weights_backward.argtypes = [vp] * 8
        L.moe_prepare_weights_backward.restype = ctypes.c_int
        L.moe_prepare_weights.restype = ctypes.c_int
        L.moe_forward.argtypes = [vp, vp, vp, vp, ctypes.POINTER(MoeWeights), vp, vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_static.argtypes = [vp, vp, vp, vp, ctypes.POINTER(MoeWeights), vp, vp]
        L.moe_forward_static.restype = ctypes.c_int
        L.moe_forward_routed.argtypes = [vp, vp, vp, ctypes.POINTER(MoeWeights), vp, vp]
        L.moe_forward_routed.restype = ctypes.c_int
        L.moe_backward.argtypes = [vp, vp, vp, ctypes.POINTER(MoeWeights), vp, vp, vp, vp, vp]
        L.moe_backward.restype = ctypes.c_int
        L.moe_get_status.argtypes = [vp, ctypes.POINTER(i32), i32, vp]
        L.moe_get_status.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_profile.argtypes = [vp, i32]
        L.moe_profile.restype = ctypes.c_int
        L.moe_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32), i32]
        L.moe_profile_read.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().moe_status_string(int(status)).decode()
    except Exception:  # library not loadable: describe the code ourselves
        return "status %d" % status


def _ok(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def moe_plan(T, d, I, E, k, precision=MOE_BF16, training=0, path=MOE_PATH_AUTO,
             wgrad_accumulate=0, recompute_h=0, activation=MOE_ACT_SWIGLU, mega=0) -> int:
    cfg = MoeConfig(T, d, I, E, k, precision, training, path, wgrad_accumulate, recompute_h, activation, mega)
    h = ctypes.c_void_p()
    _ok(lib().moe_plan(ctypes.byref(cfg), ctypes.byref(h)), "moe_plan")
    return h.value


def moe_workspace_bytes(plan: int) -> int:
    return int(lib().moe_workspace_bytes(plan))


def moe_plan_explain(plan: int) -> str:
    n = int(lib().moe_plan_explain(plan, None, 0))
    buf = ctypes.create_string_buffer(n + 1)
    lib().moe_plan_explain(plan, buf, n + 1)
    return buf.value.decode()


def moe_bind_workspace(plan: int, ptr: int, nbytes: int):
    _ok(lib().moe_bind_workspace(plan, ptr, nbytes), "moe_bind_workspace")


def moe_plan_destroy(plan: int):
    _ok(lib().moe_plan_destroy(plan), "moe_plan_destroy")


def moe_dispatch(plan, ids, scores, m_indptr, gather, slots, probs, stream=0):
    _ok(lib().moe_dispatch(plan, ids, scores, m_indptr, gather, slots, probs, stream), "moe_dispatch")


def moe_quantize_mxfp8(v, rows, K, codes, scales, stream=0):
    _ok(lib().moe_quantize_mxfp8(v, rows, K, codes, scales, stream), "moe_quantize_mxfp8")


def moe_prepare_weights(plan, w13, w2, w13_q, w13_s, w2_q, w2_s, stream=0):
    _ok(lib().moe_prepare_weights(plan, w13, w2, w13_q, w13_s, w2_q, w2_s, stream),
        "moe_prepare_weights")


def moe_prepare_weights_backward(plan, w13, w2, w13t_q, w13t_s, w2t_q, w2t_s, stream=0):
    _ok(lib().moe_prepare_weights_backward(plan, w13, w2, w13t_q, w13t_s, w2t_q, w2t_s, stream),
        "moe_prepare_weights_backward")


def weights(w13, w2, w13_scale=0, w2_scale=0, w13t=0, w13t_scale=0, w2t=0, w2t_scale=0) -> MoeWeights:
    return MoeWeights(w13, w2, w13_scale or None, w2_scale or None, w13t or None, w13t_scale or None,
                      w2t or None, w2t_scale or None)


def moe_forward(plan, x, ids, scores, w: MoeWeights, y, stream=0):
    _ok(lib().moe_forward(plan, x, ids, scores, ctypes.byref(w), y, stream), "moe_forward")


def moe_forward_static(plan, x, ids, scores, w: MoeWeights, y, stream=0):
    _ok(lib().moe_forward_static(plan, x, ids, scores, ctypes.byref(w), y, stream), "moe_forward_static")


def moe_forward_routed(plan, x_rows, m_indptr, w: MoeWeights, out, stream=0):
    _ok(lib().moe_forward_routed(plan, x_rows, m_indptr, ctypes.byref(w), out, stream),
        "moe_forward_routed")


def moe_backward(plan, dy, x, w: MoeWeights, dx, dw13, dw2, dscores, stream=0):
    _ok(lib().moe_backward(plan, dy, x, ctypes.byref(w), dx, dw13, dw2, dscores, stream),
        "moe_backward")


def moe_get_status(plan, clear=True, stream=0):
    """Returns (status, device_flags); synchronises the stream."""
    flags = ctypes.c_int32(0)
    st = lib().moe_get_status(plan, ctypes.byref(flags), 1 if clear else 0, stream)
    if st not in (MOE_OK, MOE_ERR_ROUTING):
        raise MoeError(st, "moe_get_status")
    return st, flags.value


def moe_profile(plan, enable: bool):
    _ok(lib().moe_profile(plan, 1 if enable else 0), "moe_profile")


def moe_profile_read(plan) -> dict:
    """{stage name: (total ms, launches)} for the stages recorded since the last read."""
    n = len(STAGES)
    ms = (ctypes.c_float * n)()
    cnt = (ctypes.c_int32 * n)()
    _ok(lib().moe_profile_read(plan, ms, cnt, n), "moe_profile_read")
    return {STAGES[i]: (float(ms[i]), int(cnt[i])) for i in range(n) if cnt[i] > 0}


# ---------------------------------------------------------------- torch plumbing

def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class Layer:
    """One plan plus its torch-allocated workspace; all compute goes through libmoe."""

    def __init__(self, T, d, I, E, k, precision=MOE_BF16, training=False, path=MOE_PATH_AUTO,
                 device="cuda", wgrad_accumulate=False, recompute_h=False, activation=MOE_ACT_SWIGLU,
                 mega=False):
        import torch
        self.T, self.d, self.I, self.E, self.k = T, d, I, E, k
        self.precision = precision
        self.plan = moe_plan(T, d, I, E, k, precision, int(bool(training)), path,
                             int(bool(wgrad_accumulate)), int(bool(recompute_h)), int(activation),
                             int(bool(mega)))
        nbytes = moe_workspace_bytes(self.plan)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        moe_bind_workspace(self.plan, _ptr(self.workspace), self.workspace.numel())

    def explain(self) -> str:
        return moe_plan_explain(self.plan)

    def close(self):
        if self.plan:
            moe_plan_destroy(self.plan)
            self.plan = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def dispatch(self, ids, scores, stream=None):
        import torch
        dev = ids.device
        R = self.T * self.k
        m_indptr = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        gather = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
        slots = torch.empty((self.T, self.k), dtype=torch.int32, device=dev)
        probs = torch.empty(max(R, 1), dtype=torch.float32, device=dev)
        moe_dispatch(self.plan, _ptr(ids), _ptr(scores), _ptr(m_indptr), _ptr(gather),
                     _ptr(slots), _ptr(probs), _stream(stream))
        return m_indptr, gather[:R], slots, probs[:R]

    def forward(self, x, ids, scores, w13, w2, w13_scale=None, w2_scale=None, y=None, stream=None):
        import torch
        if y is None:
            y = torch.empty((self.T, self.d), dtype=torch.bfloat16, device=x.device)
        w = weights(_ptr(w13), _ptr(w2), _ptr(w13_scale), _ptr(w2_scale))
        moe_forward(self.plan, _ptr(x), _ptr(ids), _ptr(scores), w, _ptr(y), _stream(stream))
        return y

    def forward_routed(self, x_rows, m_indptr, w13, w2, w13_scale=None, w2_scale=None, out=None,
                       stream=None):
        """Expert outputs of rows already in expert order (int32 m_indptr [E+1] on the
        device); out BF16 [T*k, d], of which rows m_indptr[E].. are not written.  MXFP8
        plans take the prepared weights and their scales."""
        import torch
        if out is None:
            out = torch.empty((self.T * self.k, self.d), dtype=torch.bfloat16, device=x_rows.device)
        w = weights(_ptr(w13), _ptr(w2), _ptr(w13_scale), _ptr(w2_scale))
        moe_forward_routed(self.plan, _ptr(x_rows), _ptr(m_indptr), w, _ptr(out), _stream(stream))
        return out

    def backward(self, dy, x, w13, w2, dx=None, dw13=None, dw2=None, dscores=None, stream=None,
                 w13_scale=None, w13t=None, w13t_scale=None, w2t=None, w2t_scale=None):
        """BF16 plans take the BF16 weights; MXFP8 plans the tensors of
        prepare_weights_backward (w13t, w13t_scale, w2t, w2t_scale) and, with
        recompute_h, the forward's prepared w13 and w13_scale (w2 unused)."""
        import torch
        dev = dy.device
        if dx is None:
            dx = torch.empty((self.T, self.d), dtype=torch.bfloat16, device=dev)
        if dw13 is None:
            dw13 = torch.empty((self.E, 2 * self.I, self.d), dtype=torch.bfloat16, device=dev)
        if dw2 is None:
            dw2 = torch.empty((self.E, self.d, self.I), dtype=torch.bfloat16, device=dev)
        if dscores is None:
            dscores = torch.empty((self.T, self.k), dtype=torch.float32, device=dev)
        w = weights(_ptr(w13), _ptr(w2), _ptr(w13_scale), 0, _ptr(w13t), _ptr(w13t_scale), _ptr(w2t),
                    _ptr(w2t_scale))
        moe_backward(self.plan, _ptr(dy), _ptr(x), w, _ptr(dx), _ptr(dw13), _ptr(dw2), _ptr(dscores),
                     _stream(stream))
        return dx, dw13, dw2, dscores

    def prepare_weights(self, w13, w2, stream=None):
        import torch
        dev = w13.device
        E, I, d = self.E, self.I, self.d
        w13_q = torch.empty((E, 2 * I, d), dtype=torch.uint8, device=dev)
        # scales block-major: [K/128, rows, 4] (see moe_prepare_weights in include/moe.h)
        w13_s = torch.empty((d // 128, E * 2 * I, 4), dtype=torch.uint8, device=dev)
        w2_q = torch.empty((E, d, I), dtype=torch.uint8, device=dev)
        w2_s = torch.empty((I // 128, E * d, 4), dtype=torch.uint8, device=dev)
        moe_prepare_weights(self.plan, _ptr(w13), _ptr(w2), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q),
                            _ptr(w2_s), _stream(stream))
        return w13_q, w13_s, w2_q, w2_s

    def prepare_weights_backward(self, w13, w2, stream=None):
        """(w13t, w13t_scale, w2t, w2t_scale) for the MXFP8 backward: W13_e^T [d, 2I] and
        W2_e^T [I, d] quantized along their last dimension, scales block-major."""
        import torch
        dev = w13.device
        E, I, d = self.E, self.I, self.d
        w13t = torch.empty((E, d, 2 * I), dtype=torch.uint8, device=dev)
        w13t_s = torch.empty((2 * I // 128, E * d, 4), dtype=torch.uint8, device=dev)
        w2t = torch.empty((E, I, d), dtype=torch.uint8, device=dev)
        w2t_s = torch.empty((d // 128, E * I, 4), dtype=torch.uint8, device=dev)
        moe_prepare_weights_backward(self.plan, _ptr(w13), _ptr(w2), _ptr(w13t), _ptr(w13t_s), _ptr(w2t),
                                     _ptr(w2t_s), _stream(stream))
        return w13t, w13t_s, w2t, w2t_s

    def status(self, clear=True, stream=None):
        return moe_get_status(self.plan, clear, _stream(stream))

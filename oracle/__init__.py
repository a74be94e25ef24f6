"""CPU oracle for the routed Mixture-of-Experts expert layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The product path (the HIP library and its
Python binding) never imports, links or runs anything here, and nothing here
imports the product package.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64).  This module only
compiles it with gcc, widens BF16 bit patterns to their exact float32 values,
and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_lib = None

ORC_OK, ORC_ERR_RANGE, ORC_ERR_DUPLICATE, ORC_ERR_ALLOC = 0, 1, 2, 3


class RoutingError(ValueError):
    """The routing violates the layer's precondition (id out of range or repeated in a row)."""


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liborc.so`` with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i32, f64p = ctypes.c_int, ctypes.POINTER(ctypes.c_double)
        vp = ctypes.c_void_p
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_check_routing.argtypes = [i32, i32, i32, vp]
        lib.orc_dispatch.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp]
        lib.orc_forward_tokens.argtypes = [i32] * 5 + [vp] * 5 + [i32, vp, vp, vp, vp, i32]
        lib.orc_backward_tokens.argtypes = [i32] * 5 + [vp] * 6 + [i32, vp, vp, vp, i32]
        lib.orc_wgrad_cols.argtypes = [i32] * 5 + [vp] * 6 + [i32, vp, vp, vp, i32]
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_decode.restype = ctypes.c_double
        lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_mx_scale_byte.argtypes = [f64p, i32]
        lib.orc_mx_scale_byte.restype = ctypes.c_uint8
        lib.orc_mx_quantize.argtypes = [ctypes.c_int64, i32, vp, vp, vp]
        lib.orc_mx_dequantize.argtypes = [ctypes.c_int64, i32, vp, vp, vp]
        lib.orc_forward_tokens_mx.argtypes = [i32] * 5 + [vp] * 5 + [i32, vp, vp, i32]
        lib.orc_train_mx.argtypes = [i32] * 5 + [vp] * 6 + [i32] + [i32] + [vp] * 4 + [i32] + [vp] * 3
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of BF16 bit patterns (uint16)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return widen_bf16(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc: int):
    if rc == ORC_ERR_RANGE:
        raise RoutingError("expert id out of range")
    if rc == ORC_ERR_DUPLICATE:
        raise RoutingError("expert id repeated within a token row")
    if rc == ORC_ERR_ALLOC:
        raise MemoryError("oracle allocation failed")
    if rc != ORC_OK:
        raise RuntimeError("oracle error %d" % rc)


def num_threads() -> int:
    return int(_L().orc_num_threads())


def check_routing(ids: np.ndarray, E: int) -> int:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    return _L().orc_check_routing(T, E, k, _p(ids))


def dispatch(ids: np.ndarray, scores: np.ndarray, E: int):
    """Stable expert-major dispatch -> (m_indptr[E+1], gather[R], slots[T,k], probs[R])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    T, k = ids.shape
    m_indptr = np.zeros(E + 1, np.int32)
    gather = np.zeros(T * k, np.int32)
    slots = np.zeros((T, k), np.int32)
    probs = np.zeros(T * k, np.float32)
    _check(_L().orc_dispatch(T, E, k, _p(ids), _p(scores), _p(m_indptr), _p(gather),
                             _p(slots), _p(probs)))
    return m_indptr, gather, slots, probs


def _shapes(x, w13, w2, ids):
    T, d = x.shape
    E, twoI, d2 = w13.shape
    I = twoI // 2
    assert d2 == d and w2.shape == (E, d, I) and ids.shape[0] == T
    return T, d, I, E, ids.shape[1]


ACT_SWIGLU, ACT_GEGLU, ACT_REGLU = 0, 1, 2


def forward_tokens(x, ids, scores, w13, w2, toks=None, want_o=False, want_a=False, act=ACT_SWIGLU):
    """y for the listed tokens ([ntok, d] float64); optionally o [ntok,k,d] and a [ntok,k,I].
    act: the gated activation (0 SwiGLU, 1 GeGLU with the exact GELU, 2 ReGLU)."""
    xf, w13f, w2f = _f32(x), _f32(w13), _f32(w2)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    T, d, I, E, k = _shapes(xf, w13f, w2f, ids)
    toks = np.arange(T, dtype=np.int32) if toks is None else np.ascontiguousarray(toks, np.int32)
    n = len(toks)
    y = np.zeros((n, d), np.float64)
    o = np.zeros((n, k, d), np.float64) if want_o else None
    a = np.zeros((n, k, I), np.float64) if want_a else None
    _check(_L().orc_forward_tokens(T, d, I, E, k, _p(xf), _p(ids), _p(scores), _p(w13f), _p(w2f),
                                   n, _p(toks), _p(y), _p(o) if o is not None else None,
                                   _p(a) if a is not None else None, int(act)))
    out = [y]
    if want_o:
        out.append(o)
    if want_a:
        out.append(a)
    return out[0] if len(out) == 1 else tuple(out)


def backward_tokens(x, ids, scores, w13, w2, dy, toks=None, act=ACT_SWIGLU):
    """(dX [ntok, d], dS [ntok, k]) in float64 for the listed tokens."""
    xf, w13f, w2f, dyf = _f32(x), _f32(w13), _f32(w2), _f32(dy)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    T, d, I, E, k = _shapes(xf, w13f, w2f, ids)
    toks = np.arange(T, dtype=np.int32) if toks is None else np.ascontiguousarray(toks, np.int32)
    n = len(toks)
    dx = np.zeros((n, d), np.float64)
    ds = np.zeros((n, k), np.float64)
    _check(_L().orc_backward_tokens(T, d, I, E, k, _p(xf), _p(ids), _p(scores), _p(w13f), _p(w2f),
                                    _p(dyf), n, _p(toks), _p(dx), _p(ds), int(act)))
    return dx, ds


def wgrad_cols(x, ids, scores, w13, w2, dy, icols=None, act=ACT_SWIGLU):
    """Weight gradients on intermediate columns icols (all by default).

    Returns (dW2[:, :, icols] as [E, d, ni], dW13 rows (icols, I+icols) as [E, 2, ni, d]).
    """
    xf, w13f, w2f, dyf = _f32(x), _f32(w13), _f32(w2), _f32(dy)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    T, d, I, E, k = _shapes(xf, w13f, w2f, ids)
    icols = np.arange(I, dtype=np.int32) if icols is None else np.ascontiguousarray(icols, np.int32)
    ni = len(icols)
    dw2 = np.zeros((E, d, ni), np.float64)
    dw13 = np.zeros((E, 2, ni, d), np.float64)
    _check(_L().orc_wgrad_cols(T, d, I, E, k, _p(xf), _p(ids), _p(scores), _p(w13f), _p(w2f),
                               _p(dyf), ni, _p(icols), _p(dw2), _p(dw13), int(act)))
    return dw2, dw13


def e4m3_decode(code: int) -> float:
    return _L().orc_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return int(_L().orc_e4m3_encode(float(v)))


def mx_scale_byte(block) -> int:
    b = np.ascontiguousarray(block, dtype=np.float64)
    return int(_L().orc_mx_scale_byte(b.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), len(b)))


def mx_quantize(v) -> tuple:
    """Rows of length K (multiple of 32) -> (E4M3 codes uint8 same shape, E8M0 scales [.., K/32])."""
    vf = _f32(v)
    K = vf.shape[-1]
    assert K % 32 == 0
    rows = vf.size // K
    codes = np.zeros(vf.shape, np.uint8)
    scales = np.zeros(vf.shape[:-1] + (K // 32,), np.uint8)
    _L().orc_mx_quantize(rows, K, _p(vf), _p(codes), _p(scales))
    return codes, scales


def mx_dequantize(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    K = codes.shape[-1]
    rows = codes.size // K
    out = np.zeros(codes.shape, np.float32)
    _L().orc_mx_dequantize(rows, K, _p(codes), _p(scales), _p(out))
    return out


def forward_tokens_mx(x, ids, scores, w13, w2, toks=None, act=ACT_SWIGLU):
    """y with x and the gated-activation output passed through MX block-32 quantize/dequantize."""
    xf, w13f, w2f = _f32(x), _f32(w13), _f32(w2)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    T, d, I, E, k = _shapes(xf, w13f, w2f, ids)
    toks = np.arange(T, dtype=np.int32) if toks is None else np.ascontiguousarray(toks, np.int32)
    n = len(toks)
    y = np.zeros((n, d), np.float64)
    _check(_L().orc_forward_tokens_mx(T, d, I, E, k, _p(xf), _p(ids), _p(scores), _p(w13f),
                                      _p(w2f), n, _p(toks), _p(y), int(act)))
    return y


def train_mx(x, ids, scores, w13, w2, dy, act=ACT_SWIGLU, toks=None, icols=None):
    """One MXFP8 training step from BF16 master weights: every expert product takes MX images
    of both operands along its own reduction dimension, WGRAD operands blocked along each
    expert's routed rows.  Returns (y, dx, ds, dw13, dw2) in float64 for the tokens `toks`
    (default all) and the intermediate indices `icols` (default all: dw13 [E, 2I, d],
    dw2 [E, d, I]; else dw13 [E, 2, ni, d] gate and up rows of icols, dw2 [E, d, ni])."""
    xf, w13f, w2f, dyf = _f32(x), _f32(w13), _f32(w2), _f32(dy)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    T, d, I, E, k = _shapes(xf, w13f, w2f, ids)
    full_cols = icols is None
    toks = np.arange(T, dtype=np.int32) if toks is None else np.ascontiguousarray(toks, np.int32)
    icols = np.arange(I, dtype=np.int32) if full_cols else np.ascontiguousarray(icols, np.int32)
    n, ni = len(toks), len(icols)
    y = np.zeros((n, d), np.float64)
    dx = np.zeros((n, d), np.float64)
    ds = np.zeros((n, k), np.float64)
    dw13 = np.zeros((E, 2, ni, d), np.float64)
    dw2 = np.zeros((E, d, ni), np.float64)
    _check(_L().orc_train_mx(T, d, I, E, k, _p(xf), _p(ids), _p(scores), _p(w13f), _p(w2f), _p(dyf),
                             int(act), n, _p(toks), _p(y), _p(dx), _p(ds), ni, _p(icols), _p(dw13),
                             _p(dw2)))
    if full_cols:
        dw13 = dw13.reshape(E, 2 * I, d)
    return y, dx, ds, dw13, dw2

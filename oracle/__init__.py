"""ctypes view of the CPU oracle (qgemv_oracle.c).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg use it to produce expected values; the HIP library and its
binding never import it.  Every function takes and returns numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

Q8_0 = 1
Q4_0 = 2
Q4_K = 3
QK = 32
QK_K = 256
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 144}
BLOCK_WEIGHTS = {Q8_0: 32, Q4_0: 32, Q4_K: 256}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        L = C.CDLL(_build.LIB)
        p = C.c_void_p
        i64 = C.c_int64
        ci = C.c_int
        L.orc_f16_to_f32.restype = C.c_float
        L.orc_f16_to_f32.argtypes = [C.c_uint16]
        L.orc_f32_to_f16.restype = C.c_uint16
        L.orc_f32_to_f16.argtypes = [C.c_float, C.POINTER(C.c_int)]
        L.orc_f32_to_f16_array.argtypes = [p, p, i64, C.POINTER(C.c_int)]
        L.orc_f16_to_f32_array.argtypes = [p, p, i64]
        for f in ("orc_quantize_q8_0", "orc_quantize_q4_0", "orc_quantize_q4_k"):
            getattr(L, f).restype = ci
            getattr(L, f).argtypes = [p, i64, i64, p]
        L.orc_dequantize.restype = ci
        L.orc_dequantize.argtypes = [ci, p, i64, i64, p]
        L.orc_quantize_acts.restype = ci
        L.orc_quantize_acts.argtypes = [p, ci, i64, p, p, p]
        L.orc_blockdots.restype = ci
        L.orc_blockdots.argtypes = [ci, p, i64, i64, p, ci, p]
        L.orc_gemv_q.restype = ci
        L.orc_gemv_q.argtypes = [ci, p, i64, i64, p, ci, p, ci]
        L.orc_gemv_q_rows.restype = ci
        L.orc_gemv_q_rows.argtypes = [ci, p, i64, i64, p, ci, p, i64, p, ci]
        L.orc_gemv_f16.restype = ci
        L.orc_gemv_f16.argtypes = [p, i64, i64, p, ci, p, ci]
        L.orc_gemv_f16_rows.restype = ci
        L.orc_gemv_f16_rows.argtypes = [p, i64, i64, p, ci, p, i64, p, ci]
        L.orc_gemv_q8_0_grouped.restype = ci
        L.orc_gemv_q8_0_grouped.argtypes = [p, i64, i64, i64, p, ci, p, p, ci, p]
        L.orc_route_topk.restype = ci
        L.orc_route_topk.argtypes = [p, ci, i64, ci, p, p]
        L.orc_swiglu.argtypes = [p, p, i64, p]
        L.orc_add_rmsnorm.argtypes = [p, p, p, C.c_double, ci, i64, p, p]
        L.orc_e4m3_encode_array.argtypes = [p, p, i64]
        L.orc_e4m3_decode.restype = C.c_double
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_quantize_fp8_weights.restype = ci
        L.orc_quantize_fp8_weights.argtypes = [p, i64, i64, p, p]
        L.orc_quantize_fp8_acts.restype = ci
        L.orc_quantize_fp8_acts.argtypes = [p, ci, i64, p, p]
        L.orc_gemv_fp8.restype = ci
        L.orc_gemv_fp8.argtypes = [p, p, i64, i64, p, ci, p, i64, p, ci]
        L.orc_moe_step.restype = ci
        L.orc_moe_step.argtypes = [p, ci, i64, p, i64, ci, p, p, p, i64, p, p, p, p, p, p, p]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ fp16 ---
def f32_to_f16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    ov = C.c_int(0)
    lib().orc_f32_to_f16_array(_ptr(x), _ptr(out), x.size, C.byref(ov))
    return out, bool(ov.value)


def f16_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


# --------------------------------------------------------------- weights ---
def quantize_weights(fmt, w):
    """fp32 [n][k] -> canonical blocks, uint8 [n][k/32][block bytes] (Q4_K: [n][k/256][144])."""
    w = _c(w, np.float32)
    n, k = w.shape
    out = np.zeros((n, k // BLOCK_WEIGHTS[fmt], BLOCK_BYTES[fmt]), np.uint8)
    f = {Q8_0: lib().orc_quantize_q8_0, Q4_0: lib().orc_quantize_q4_0, Q4_K: lib().orc_quantize_q4_k}[fmt]
    rc = f(_ptr(w), n, k, _ptr(out))
    if rc == -1:
        raise ValueError(f"k must be a multiple of {BLOCK_WEIGHTS[fmt]}")
    if rc == -2:
        raise OverflowError("a block scale overflowed fp16")
    return out


def dequantize(fmt, blocks, n, k):
    blocks = _c(blocks, np.uint8)
    out = np.empty((n, k), np.float64)
    assert lib().orc_dequantize(fmt, _ptr(blocks), n, k, _ptr(out)) == 0
    return out


# ----------------------------------------------------------- activations ---
def quantize_acts(x):
    x = _c(x, np.float32)
    rows, k = x.shape
    qx = np.empty((rows, k), np.int8)
    dx = np.empty((rows, k // QK), np.float32)
    sx = np.empty((rows, k // QK), np.int32)
    assert lib().orc_quantize_acts(_ptr(x), rows, k, _ptr(qx), _ptr(dx), _ptr(sx)) == 0
    return qx, dx, sx


def blockdots(fmt, blocks, n, k, qx):
    blocks = _c(blocks, np.uint8)
    qx = _c(qx, np.int8)
    rows = qx.shape[0]
    out = np.empty((rows, n, k // QK), np.int32)
    assert lib().orc_blockdots(fmt, _ptr(blocks), n, k, _ptr(qx), rows, _ptr(out)) == 0
    return out


# ------------------------------------------------------------------ GEMV ---
def gemv_q(fmt, blocks, n, k, x, threads=1):
    blocks = _c(blocks, np.uint8)
    x = _c(x, np.float32)
    rows = x.shape[0]
    y = np.empty((rows, n), np.float32)
    assert lib().orc_gemv_q(fmt, _ptr(blocks), n, k, _ptr(x), rows, _ptr(y), threads) == 0
    return y


def gemv_q_rows(fmt, blocks, n, k, x, sel, threads=1):
    blocks = _c(blocks, np.uint8)
    x = _c(x, np.float32)
    sel = _c(sel, np.int64)
    rows = x.shape[0]
    y = np.empty((rows, sel.size), np.float32)
    assert lib().orc_gemv_q_rows(fmt, _ptr(blocks), n, k, _ptr(x), rows, _ptr(sel), sel.size, _ptr(y),
                                 threads) == 0
    return y


def gemv_f16(w16, x, threads=1):
    w16 = _c(w16, np.uint16)
    x = _c(x, np.float32)
    n, k = w16.shape
    rows = x.shape[0]
    y = np.empty((rows, n), np.float32)
    assert lib().orc_gemv_f16(_ptr(w16), n, k, _ptr(x), rows, _ptr(y), threads) == 0
    return y


def gemv_f16_rows(w16, x, sel, threads=1):
    w16 = _c(w16, np.uint16)
    x = _c(x, np.float32)
    sel = _c(sel, np.int64)
    n, k = w16.shape
    rows = x.shape[0]
    y = np.empty((rows, sel.size), np.float32)
    assert lib().orc_gemv_f16_rows(_ptr(w16), n, k, _ptr(x), rows, _ptr(sel), sel.size, _ptr(y), threads) == 0
    return y


def gemv_q8_0_grouped(blocks, n_experts, n, k, x, expert, x_index, y=None):
    blocks = _c(blocks, np.uint8)
    x = _c(x, np.float32)
    expert = _c(expert, np.int32)
    x_index = _c(x_index, np.int32)
    m = expert.size
    if y is None:
        y = np.full((m, n), np.nan, np.float32)
    bad = lib().orc_gemv_q8_0_grouped(_ptr(blocks), n_experts, n, k, _ptr(x), x.shape[0], _ptr(expert),
                                      _ptr(x_index), m, _ptr(y))
    return y, bad


# ------------------------------------------------------------------- MoE ---
def route_topk(logits, topk):
    logits = _c(logits, np.float32)
    rows, E = logits.shape
    ex = np.empty((rows, topk), np.int32)
    p = np.empty((rows, topk), np.float64)
    assert lib().orc_route_topk(_ptr(logits), rows, E, topk, _ptr(ex), _ptr(p)) == 0
    return ex, p


def swiglu(g, u):
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.empty(g.shape, np.float32)
    lib().orc_swiglu(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


# ------------------------------------------------------------ FP8 lane ---
FP8_GROUP = 128


def e4m3_encode(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_decode(codes):
    codes = np.asarray(codes, np.uint8)
    table = np.array([lib().orc_e4m3_decode(c) for c in range(256)], np.float64)
    return table[codes]


def quantize_fp8_weights(w):
    """[n][k] fp32 -> (codes [n][k] uint8, scales [ceil(n/128)][k/128] fp32)."""
    w = _c(w, np.float32)
    n, k = w.shape
    codes = np.empty((n, k), np.uint8)
    scales = np.empty(((n + FP8_GROUP - 1) // FP8_GROUP, k // FP8_GROUP), np.float32)
    assert lib().orc_quantize_fp8_weights(_ptr(w), n, k, _ptr(codes), _ptr(scales)) == 0
    return codes, scales


def quantize_fp8_acts(x):
    x = _c(x, np.float32)
    rows, k = x.shape
    codes = np.empty((rows, k), np.uint8)
    scales = np.empty((rows, k // FP8_GROUP), np.float32)
    assert lib().orc_quantize_fp8_acts(_ptr(x), rows, k, _ptr(codes), _ptr(scales)) == 0
    return codes, scales


def gemv_fp8(codes, scales, x, sel=None, threads=1):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    x = _c(x, np.float32)
    n, k = codes.shape
    rows = x.shape[0]
    if sel is not None:
        sel = _c(sel, np.int64)
    ns = n if sel is None else sel.size
    y = np.empty((rows, ns), np.float32)
    assert lib().orc_gemv_fp8(_ptr(codes), _ptr(scales), n, k, _ptr(x), rows, None if sel is None else _ptr(sel),
                              0 if sel is None else sel.size, _ptr(y), threads) == 0
    return y


def add_rmsnorm(x, residual, gamma, eps):
    """h = x + residual (fp32), y = h / sqrt(mean(h^2) + eps) * gamma (float64)."""
    x = _c(x, np.float32)
    rows, k = x.shape
    res = None if residual is None else _c(residual, np.float32)
    gamma = _c(gamma, np.float32)
    h = np.empty((rows, k), np.float32)
    y = np.empty((rows, k), np.float64)
    lib().orc_add_rmsnorm(_ptr(x), None if res is None else _ptr(res), _ptr(gamma), float(eps), rows, k, _ptr(h),
                          _ptr(y))
    return h, y


def moe_step(x, router16, topk, gate, up, down, ffn, sgate, sup, sdown):
    """gate/up: uint8 [E][ffn][hidden/32][34]; down: [E][hidden][ffn/32][34]."""
    x = _c(x, np.float32)
    rows, hidden = x.shape
    router16 = _c(router16, np.uint16)
    E = router16.shape[0]
    y = np.empty((rows, hidden), np.float32)
    ex = np.empty((rows, topk), np.int32)
    p = np.empty((rows, topk), np.float64)
    logits = np.empty((rows, E), np.float32)
    args = [_c(a, np.uint8) for a in (gate, up, down, sgate, sup, sdown)]
    assert lib().orc_moe_step(_ptr(x), rows, hidden, _ptr(router16), E, topk, _ptr(args[0]), _ptr(args[1]),
                              _ptr(args[2]), ffn, _ptr(args[3]), _ptr(args[4]), _ptr(args[5]), _ptr(y), _ptr(ex),
                              _ptr(p), _ptr(logits)) == 0
    return y, ex, p, logits

"""ctypes binding of libqgemv (include/qgemv.h): argument marshalling only.

Every function takes torch tensors on the current HIP device, passes their
data pointers and torch's current stream to the C ABI, and raises QGError on a
negative status.  All arithmetic runs in the library's HIP kernels; there is no
fallback: if libqgemv.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

Q8_0, Q4_0, F16, FP8, Q4_K = 1, 2, 3, 4, 5
MAX_ROWS = 16
MAX_PREP_ROWS = 8192
MAX_ASSIGN = 2048
MAX_SET = 8
FUSED_ROWS = 2


def set_fuses(fmt, rows):
    """Whether qgemv_set_rows quantizes inside its GEMV launch when every projection brings a workspace (and its
    rows fit the launch's staging area): at 1-2 rows, except Q4_0 and Q4_K at two rows."""
    return 1 <= rows <= FUSED_ROWS and not (rows == 2 and fmt != Q8_0)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")
_lib = None


class QGError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{detail} (status {status})")
        self.status = status


class _Proj(C.Structure):
    _fields_ = [("w_image", C.c_void_p), ("n", C.c_int64), ("k", C.c_int64), ("ws", C.c_void_p),
                ("ws_bytes", C.c_size_t), ("y", C.c_void_p)]


class _ProjRows(C.Structure):
    _fields_ = [("w_image", C.c_void_p), ("n", C.c_int64), ("k", C.c_int64), ("x", C.c_void_p), ("ws", C.c_void_p),
                ("ws_bytes", C.c_size_t), ("y", C.c_void_p)]


class _Act(C.Structure):
    _fields_ = [("x", C.c_void_p), ("k", C.c_int64), ("ws", C.c_void_p), ("ws_bytes", C.c_size_t)]


_SIGS = {
    "qg_image_bytes": (C.c_size_t, [C.c_int, C.c_int64, C.c_int64]),
    "qg_pack_image": (C.c_int, [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p]),
    "qg_unpack_image": (C.c_int, [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p]),
    "qg_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int64]),
    "qg_fp8_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int64]),
    "qg_prepare_fp8": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qgemv_fp8_prepared": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_size_t, C.c_int,
                                     C.c_void_p, C.c_void_p]),
    "qgemv_fp8": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p,
                            C.c_size_t, C.c_void_p]),
    "qg_grouped_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int64, C.c_int]),
    "qg_status_string": (C.c_char_p, [C.c_int]),
    "qg_last_error_detail": (C.c_int, [C.c_char_p, C.c_size_t]),
    "qg_device_supported": (C.c_int, [C.c_int]),
    "qg_quantize_weights": (C.c_int, [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]),
    "qg_prepare_rows": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qg_add_rmsnorm_prepare": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_float, C.c_int, C.c_int64,
                                         C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qgemv_prepared": (C.c_int, [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_size_t, C.c_int,
                                 C.c_void_p, C.c_void_p]),
    "qgemv_q8_0": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p,
                             C.c_size_t, C.c_void_p]),
    "qgemv_q8_0_noalloc": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p,
                                     C.c_void_p]),
    "qgemv_q4_0": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p,
                             C.c_size_t, C.c_void_p]),
    "qgemv_q4_k": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p,
                             C.c_size_t, C.c_void_p]),
    "qg_f16_image": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]),
    "gemv_f16": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "qgemv_set": (C.c_int, [C.c_int, C.POINTER(_Proj), C.c_int, C.c_int, C.c_void_p]),
    "qg_prepare_rows_set": (C.c_int, [C.POINTER(_Act), C.c_int, C.c_int, C.c_void_p]),
    "qgemv_set_rows": (C.c_int, [C.c_int, C.POINTER(_ProjRows), C.c_int, C.c_int, C.c_void_p]),
    "qgemv_q8_0_grouped": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p,
                                     C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qg_grouped_status": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_void_p]),
    "qg_fp8_grouped_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int64, C.c_int]),
    "qgemv_fp8_grouped": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p,
                                    C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qg_moe_route": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_void_p]),
    "qg_swiglu": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_void_p, C.c_void_p]),
    "qg_moe_combine": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int64, C.c_void_p, C.c_void_p]),
    "qg_moe_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_int]),
    "qg_moe_step": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_size_t, C.c_void_p]),
    "qg_moe_fp8_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_int]),
    "qg_moe_step_fp8": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_int, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_size_t, C.c_void_p]),
    "qg_quantize_rows_q8": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p]),
    "qgemv_blockdots_pairs": (C.c_int, [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_size_t, C.c_int,
                                        C.c_void_p, C.c_void_p]),
    "qg_read_probe": (C.c_int, [C.c_void_p, C.c_size_t, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "qgemv_blockdots": (C.c_int, [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p,
                                  C.c_void_p]),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status < 0:
        buf = C.create_string_buffer(512)
        lib().qg_last_error_detail(buf, 512)
        raise QGError(status, buf.value.decode())
    return status


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ------------------------------------------------------------- host side ---
def image_bytes(fmt, n, k):
    return int(lib().qg_image_bytes(fmt, n, k))


def workspace_bytes(rows, k):
    return int(lib().qg_workspace_bytes(rows, k))


def grouped_workspace_bytes(x_rows, k, m):
    return int(lib().qg_grouped_workspace_bytes(x_rows, k, m))


def pack_image(fmt, blocks, n, k):
    """Canonical blocks (numpy uint8; F16: the [n][k] halfwords, any 16-bit dtype) -> device-layout image
    bytes (numpy uint8)."""
    if fmt == F16:
        blocks = np.ascontiguousarray(blocks).view(np.uint16)
        if blocks.shape != (n, k):
            raise ValueError(f"F16 weights must be [{n}][{k}] halfwords")
    blocks = np.ascontiguousarray(blocks).view(np.uint8) if fmt == F16 else np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty(image_bytes(fmt, n, k), np.uint8)
    _check(lib().qg_pack_image(fmt, blocks.ctypes.data_as(C.c_void_p), n, k, out.ctypes.data_as(C.c_void_p)))
    return out


def pack_fp8(codes, scales):
    """Canonical block-FP8 weights (codes [n][k] uint8, scales [ceil(n/128)][k/128] fp32) -> FP8 image bytes."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    if scales.shape != ((n + 127) // 128, k // 128):
        raise ValueError("scales must be [ceil(n/128)][k/128]")
    canon = np.concatenate([codes.ravel(), scales.view(np.uint8).ravel()])
    return pack_image(FP8, canon, n, k)


def unpack_fp8(image, n, k):
    canon = unpack_image(FP8, image, n, k)
    return canon[:n * k].reshape(n, k), canon[n * k:].view(np.float32).reshape((n + 127) // 128, k // 128)


def unpack_image(fmt, image, n, k):
    image = np.ascontiguousarray(image, dtype=np.uint8)
    if fmt == FP8:
        out = np.empty(n * k + ((n + 127) // 128) * (k // 128) * 4, np.uint8)
    elif fmt == F16:
        out = np.empty((n, k), np.uint16)
    elif fmt == Q4_K:
        out = np.empty((n, k // 256, 144), np.uint8)
    else:
        out = np.empty((n, k // 32, 34 if fmt == Q8_0 else 18), np.uint8)
    _check(lib().qg_unpack_image(fmt, image.ctypes.data_as(C.c_void_p), n, k, out.ctypes.data_as(C.c_void_p)))
    return out


def device_supported(device=0):
    """True when HIP device `device` is a gfx950 carrying this library's kernels (qg_device_supported)."""
    return bool(lib().qg_device_supported(device))


def status_string(status):
    return lib().qg_status_string(status).decode()


def empty_image(fmt, n, k, device="cuda"):
    # zeroed, so the alignment gaps between planes hold zeros as in pack_image
    return torch.zeros(image_bytes(fmt, n, k), dtype=torch.uint8, device=device)


def empty_ws(rows, k, device="cuda"):
    return torch.empty(workspace_bytes(rows, k), dtype=torch.uint8, device=device)


# ------------------------------------------------------------ device side ---
def quantize_weights(fmt, w, image=None):
    _dev(w, torch.float32, "w")
    n, k = w.shape
    if image is None:
        image = empty_image(fmt, n, k, w.device)
    _check(lib().qg_quantize_weights(fmt, _p(w), n, k, _p(image), _stream()))
    return image


def prepare_rows(x, ws=None):
    _dev(x, torch.float32, "x")
    rows, k = x.shape
    if ws is None:
        ws = empty_ws(rows, k, x.device)
    _check(lib().qg_prepare_rows(_p(x), rows, k, _p(ws), ws.numel(), _stream()))
    return ws


def prepare_rows_set(xs, wss):
    rows = xs[0].shape[0]
    arr = (_Act * len(xs))()
    for i, (x, ws) in enumerate(zip(xs, wss)):
        _dev(x, torch.float32, "x")
        arr[i] = _Act(x.data_ptr(), x.shape[1], ws.data_ptr(), ws.numel())
    _check(lib().qg_prepare_rows_set(arr, len(xs), rows, _stream()))


def qgemv_prepared(fmt, image, n, k, ws, rows, y=None):
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=image.device)
    _check(lib().qgemv_prepared(fmt, _p(image), n, k, _p(ws), ws.numel(), rows, _p(y), _stream()))
    return y


def _qgemv(fn, image, n, k, x, y, ws):
    _dev(x, torch.float32, "x")
    rows = x.shape[0]
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = empty_ws(max(rows, 1), k, x.device)
    _check(fn(_p(image), n, k, _p(x), rows, _p(y), _p(ws), ws.numel(), _stream()))
    return y


def fp8_workspace_bytes(rows, k):
    return int(lib().qg_fp8_workspace_bytes(rows, k))


def prepare_fp8(x, ws=None):
    """FP8 activation groups of x [rows][k] (qg_prepare_fp8): the workspace tensor."""
    _dev(x, torch.float32, "x")
    rows, k = x.shape
    if ws is None:
        ws = torch.empty(max(1, fp8_workspace_bytes(rows, k)), dtype=torch.uint8, device=x.device)
    _check(lib().qg_prepare_fp8(_p(x), rows, k, _p(ws), ws.numel(), _stream()))
    return ws


def qgemv_fp8(image, n, k, x, y=None, ws=None):
    _dev(x, torch.float32, "x")
    rows = x.shape[0]
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, fp8_workspace_bytes(max(rows, 1), k)), dtype=torch.uint8, device=x.device)
    _check(lib().qgemv_fp8(_p(image), n, k, _p(x), rows, _p(y), _p(ws), ws.numel(), _stream()))
    return y


def qgemv_fp8_prepared(image, n, k, ws, rows, y=None):
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=ws.device)
    _check(lib().qgemv_fp8_prepared(_p(image), n, k, _p(ws), ws.numel(), rows, _p(y), _stream()))
    return y


def add_rmsnorm_prepare(x, gamma, eps, residual=None, ws=None, h_out=None, y_out=None):
    """qg_add_rmsnorm_prepare: h = x + residual, y = RMS norm of h times gamma, A1 of y into ws (a new
    workspace when ws is None and neither h_out nor y_out is asked for).  Returns (ws, h_out, y_out)."""
    _dev(x, torch.float32, "x")
    _dev(gamma, torch.float32, "gamma")
    rows, k = x.shape
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    if ws is None and h_out is None and y_out is None:
        ws = empty_ws(max(rows, 1), k, x.device)
    _check(lib().qg_add_rmsnorm_prepare(_p(x), _p(residual), _p(gamma), float(eps), rows, k, _p(h_out), _p(y_out),
                                        _p(ws), 0 if ws is None else ws.numel(), _stream()))
    return ws, h_out, y_out


def qgemv_q8_0(image, n, k, x, y=None, ws=None):
    return _qgemv(lib().qgemv_q8_0, image, n, k, x, y, ws)


NOALLOC_SCRATCH_BYTES = 1 << 20


def qgemv_q8_0_noalloc(image, n, k, x, y=None):
    """qgemv_q8_0 on the library's static workspace (qgemv_q8_0_noalloc): no workspace argument, nothing
    allocated by the library.  y is allocated here (by torch) unless given."""
    _dev(x, torch.float32, "x")
    rows = x.shape[0]
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=x.device)
    _check(lib().qgemv_q8_0_noalloc(_p(image), n, k, _p(x), rows, _p(y), _stream()))
    return y


def qgemv_q4_0(image, n, k, x, y=None, ws=None):
    return _qgemv(lib().qgemv_q4_0, image, n, k, x, y, ws)


def qgemv_q4_k(image, n, k, x, y=None, ws=None):
    return _qgemv(lib().qgemv_q4_k, image, n, k, x, y, ws)


def f16_image(w16, out=None):
    """The F16 image (qg_f16_image) of a row-major [n][k] halfword device matrix."""
    _dev(w16, None, "w16")
    if w16.dtype not in (torch.float16, torch.int16, torch.uint16):
        raise ValueError("w16 must hold fp16 bits")
    n, k = w16.shape
    if out is None:
        out = torch.empty(max(1, image_bytes(F16, n, k)), dtype=torch.uint8, device=w16.device)
    _check(lib().qg_f16_image(_p(w16), n, k, _p(out), _stream()))
    return out


def gemv_f16(image, n, k, x, y=None):
    """f16 lane: y [rows][n] from the F16 image of W [n][k] and x [rows][k] fp32."""
    _dev(x, torch.float32, "x")
    rows = x.shape[0]
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=x.device)
    _check(lib().gemv_f16(_p(image), n, k, _p(x), rows, _p(y), _stream()))
    return y


def qgemv_set(fmt, projs, rows):
    """projs: list of (image, n, k, ws, y)."""
    arr = (_Proj * len(projs))()
    for i, (image, n, k, ws, y) in enumerate(projs):
        arr[i] = _Proj(image.data_ptr(), n, k, ws.data_ptr(), ws.numel(), y.data_ptr())
    _check(lib().qgemv_set(fmt, arr, len(projs), rows, _stream()))


def qgemv_set_rows(fmt, projs, rows):
    """projs: list of (image, n, k, x, ws, y); ws may be None when rows <= FUSED_ROWS."""
    arr = (_ProjRows * len(projs))()
    for i, (image, n, k, x, ws, y) in enumerate(projs):
        _dev(x, torch.float32, "x")
        arr[i] = _ProjRows(image.data_ptr(), n, k, x.data_ptr(), 0 if ws is None else ws.data_ptr(),
                           0 if ws is None else ws.numel(), y.data_ptr())
    _check(lib().qgemv_set_rows(fmt, arr, len(projs), rows, _stream()))


def qgemv_q8_0_grouped(images, n_experts, n, k, x, expert, x_index, y=None, ws=None):
    _dev(x, torch.float32, "x")
    _dev(expert, torch.int32, "expert")
    _dev(x_index, torch.int32, "x_index")
    x_rows = x.shape[0]
    m = expert.numel()
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(grouped_workspace_bytes(x_rows, k, m), dtype=torch.uint8, device=x.device)
    _check(lib().qgemv_q8_0_grouped(_p(images), n_experts, n, k, _p(x), x_rows, _p(expert), _p(x_index), m, _p(y),
                                    _p(ws), ws.numel(), _stream()))
    return y, ws


def fp8_grouped_workspace_bytes(x_rows, k, m):
    return lib().qg_fp8_grouped_workspace_bytes(x_rows, k, m)


def qgemv_fp8_grouped(images, n_experts, n, k, x, expert, x_index, y=None, ws=None):
    """FP8-lane grouped routed-expert GEMV (qgemv_fp8_grouped); returns (y [m][n], ws)."""
    _dev(x, torch.float32, "x")
    _dev(expert, torch.int32, "expert")
    _dev(x_index, torch.int32, "x_index")
    x_rows = x.shape[0]
    m = expert.numel()
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, fp8_grouped_workspace_bytes(x_rows, k, m)), dtype=torch.uint8, device=x.device)
    _check(lib().qgemv_fp8_grouped(_p(images), n_experts, n, k, _p(x), x_rows, _p(expert), _p(x_index), m, _p(y),
                                   _p(ws), ws.numel(), _stream()))
    return y, ws


def grouped_status(ws):
    bad = C.c_int32(0)
    _check(lib().qg_grouped_status(_p(ws), C.byref(bad), _stream()))
    return bad.value


def moe_route(logits, topk, shared_expert=-1):
    _dev(logits, torch.float32, "logits")
    rows, E = logits.shape
    slots = topk + (1 if shared_expert >= 0 else 0)
    dev = logits.device
    expert = torch.empty(rows * slots, dtype=torch.int32, device=dev)
    x_index = torch.empty(rows * slots, dtype=torch.int32, device=dev)
    weight = torch.empty(rows * slots, dtype=torch.float32, device=dev)
    _check(lib().qg_moe_route(_p(logits), rows, E, topk, shared_expert, _p(expert), _p(x_index), _p(weight),
                              _stream()))
    return expert, x_index, weight


def swiglu(gu, ffn, h=None):
    _dev(gu, torch.float32, "gu")
    m = gu.shape[0]
    if h is None:
        h = torch.empty((m, ffn), dtype=torch.float32, device=gu.device)
    _check(lib().qg_swiglu(_p(gu), m, ffn, _p(h), _stream()))
    return h


def moe_combine(o, weight, rows, slots, y=None):
    _dev(o, torch.float32, "o")
    hidden = o.shape[1]
    if y is None:
        y = torch.empty((rows, hidden), dtype=torch.float32, device=o.device)
    _check(lib().qg_moe_combine(_p(o), _p(weight), rows, slots, hidden, _p(y), _stream()))
    return y


def moe_workspace_bytes(rows, n_experts, hidden, ffn, topk, shared):
    return lib().qg_moe_workspace_bytes(rows, n_experts, hidden, ffn, topk, int(shared))


def moe_fp8_workspace_bytes(rows, n_experts, hidden, ffn, topk, shared):
    return lib().qg_moe_fp8_workspace_bytes(rows, n_experts, hidden, ffn, topk, int(shared))


def moe_step_fp8_fused(x, router_image, n_experts, topk, gu_images, down_images, ffn, shared=True, ws=None):
    """The routed MoE step in the FP8 lane in one library call (qg_moe_step_fp8).  Returns y, the routing
    (expert, weight) as [rows * slots] tensors, and the router logits."""
    _dev(x, torch.float32, "x")
    rows, hidden = x.shape
    slots = topk + (1 if shared else 0)
    dev = x.device
    y = torch.empty((rows, hidden), dtype=torch.float32, device=dev)
    logits = torch.empty((rows, n_experts), dtype=torch.float32, device=dev)
    expert = torch.empty(rows * slots, dtype=torch.int32, device=dev)
    weight = torch.empty(rows * slots, dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(1, moe_fp8_workspace_bytes(rows, n_experts, hidden, ffn, topk, shared)),
                         dtype=torch.uint8, device=dev)
    _check(lib().qg_moe_step_fp8(_p(router_image), n_experts, hidden, ffn, topk, int(shared), _p(gu_images),
                                 _p(down_images), _p(x), rows, _p(y), _p(logits), _p(expert), _p(weight), _p(ws),
                                 ws.numel(), _stream()))
    return y, (expert, weight), logits


def moe_step_fp8(x, router_image, n_experts, topk, gu_images, down_images, ffn, shared_expert=None):
    """The routed MoE step in the FP8 lane composed of library calls only (see moe_step)."""
    rows, hidden = x.shape
    n_images = n_experts + (1 if shared_expert is not None else 0)
    logits = gemv_f16(router_image, n_experts, hidden, x)
    expert, x_index, weight = moe_route(logits, topk, -1 if shared_expert is None else shared_expert)
    m = expert.numel()
    gu, _ = qgemv_fp8_grouped(gu_images, n_images, 2 * ffn, hidden, x, expert, x_index)
    h = swiglu(gu, ffn)
    ident = torch.arange(m, dtype=torch.int32, device=x.device)
    o, _ = qgemv_fp8_grouped(down_images, n_images, hidden, ffn, h, expert, ident)
    y = moe_combine(o, weight, rows, m // rows)
    return y, (expert, x_index, weight), logits


def moe_step_fused(x, router_image, n_experts, topk, gu_images, down_images, ffn, shared=True, ws=None):
    """The routed MoE step of moe_step in one library call (qg_moe_step).  Returns y and the routing
    (expert, weight) as [rows * slots] tensors, and the router logits."""
    _dev(x, torch.float32, "x")
    rows, hidden = x.shape
    slots = topk + (1 if shared else 0)
    dev = x.device
    y = torch.empty((rows, hidden), dtype=torch.float32, device=dev)
    logits = torch.empty((rows, n_experts), dtype=torch.float32, device=dev)
    expert = torch.empty(rows * slots, dtype=torch.int32, device=dev)
    weight = torch.empty(rows * slots, dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(1, moe_workspace_bytes(rows, n_experts, hidden, ffn, topk, shared)), dtype=torch.uint8,
                         device=dev)
    _check(lib().qg_moe_step(_p(router_image), n_experts, hidden, ffn, topk, int(shared), _p(gu_images), _p(down_images),
                             _p(x), rows, _p(y), _p(logits), _p(expert), _p(weight), _p(ws), ws.numel(), _stream()))
    return y, (expert, weight), logits


def quantize_rows_q8(x):
    _dev(x, torch.float32, "x")
    rows, k = x.shape
    qx = torch.empty((rows, k), dtype=torch.int8, device=x.device)
    dx = torch.empty((rows, k // 32), dtype=torch.float32, device=x.device)
    sx = torch.empty((rows, k // 32), dtype=torch.int32, device=x.device)
    _check(lib().qg_quantize_rows_q8(_p(x), rows, k, _p(qx), _p(dx), _p(sx), _stream()))
    return qx, dx, sx


def blockdots(fmt, image, n, k, qx):
    _dev(qx, torch.int8, "qx")
    rows = qx.shape[0]
    isum = torch.empty((rows, n, k // 32), dtype=torch.int32, device=qx.device)
    _check(lib().qgemv_blockdots(fmt, _p(image), n, k, _p(qx), rows, _p(isum), _stream()))
    return isum


def blockdots_pairs(fmt, image, n, k, ws, rows):
    """The 3..16-row kernel's block dots from a pair-order workspace (prepare_rows of `rows` rows)."""
    isum = torch.empty((rows, n, k // 32), dtype=torch.int32, device=ws.device)
    _check(lib().qgemv_blockdots_pairs(fmt, _p(image), n, k, _p(ws), ws.numel(), rows, _p(isum), _stream()))
    return isum


# ------------------------------------------------------------- MoE step ---
def moe_step(x, router_image, n_experts, topk, gu_images, down_images, ffn, shared_expert=None):
    """Routed MoE decode step, composed of library calls only.

    router_image: F16 image of the fp16 [n_experts][hidden] router; gu_images: n_experts (+1 shared) stacked Q8_0
    images of [2*ffn][hidden] (gate rows, then up rows); down_images: the same
    experts' [hidden][ffn] images.  The shared expert, if given, is the stacked
    index `shared_expert` and joins every row with weight 1.
    Returns y [rows][hidden] and the routing (expert, x_index, weight).
    """
    rows, hidden = x.shape
    n_images = n_experts + (1 if shared_expert is not None else 0)
    logits = gemv_f16(router_image, n_experts, hidden, x)
    expert, x_index, weight = moe_route(logits, topk, -1 if shared_expert is None else shared_expert)
    m = expert.numel()
    gu, _ = qgemv_q8_0_grouped(gu_images, n_images, 2 * ffn, hidden, x, expert, x_index)
    h = swiglu(gu, ffn)
    ident = torch.arange(m, dtype=torch.int32, device=x.device)
    o, _ = qgemv_q8_0_grouped(down_images, n_images, hidden, ffn, h, expert, ident)
    y = moe_combine(o, weight, rows, m // rows)
    return y, (expert, x_index, weight), logits

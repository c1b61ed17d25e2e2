"""NVFP4 oracle -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

A plain, slow CPU reference (``nvfp4_oracle.cpp``, fp64 exhaustive-search
encoders and fp64 GEMMs) of what the NVFP4 hot path computes, wrapped with
ctypes and numpy.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the HIP library never does,
and this module imports nothing from the HIP package.

Sources are cited per function in the C++ file: the QUADS explainer (§1, §2.1,
§2.2-A, §2.2-B), the TRACE post ("Fonctionnement, côté ingénierie") and the
public NVFP4/OCP format definitions for the block size, scale formats and
rounding the pages leave open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float


def build(force: bool = False) -> str:
    """Compile the oracle with g++ into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-pthread", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            L.orc_e2m1_value.restype = ctypes.c_double
            L.orc_e2m1_value.argtypes = [ctypes.c_int]
            L.orc_e4m3_value.restype = ctypes.c_double
            L.orc_e4m3_value.argtypes = [ctypes.c_int]
            L.orc_tensor_scale.restype = _F
            L.orc_tensor_scale.argtypes = [_F]
            L.orc_float_to_bf16.restype = ctypes.c_uint16
            L.orc_float_to_bf16.argtypes = [_F]
            L.orc_float_to_bf16_array.argtypes = [_P, _I64, _P]
            L.orc_double_to_bf16.restype = ctypes.c_uint16
            L.orc_double_to_bf16.argtypes = [ctypes.c_double]
            L.orc_threads.restype = ctypes.c_int
            for name in ("orc_quantize", "orc_quantize_threshold_form"):
                f = getattr(L, name)
                f.restype = ctypes.c_int
                f.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P]
            L.orc_dequantize_f32.argtypes = [_P, _P, _F, _I64, _I64, _P]
            L.orc_guidance_record.restype = ctypes.c_int
            L.orc_guidance_record.argtypes = [_P, ctypes.c_int, _I64, _I64, _P, _P, _F,
                                              ctypes.c_int, _P]
            L.orc_guided_quantize.restype = ctypes.c_int
            L.orc_guided_quantize.argtypes = [_P, ctypes.c_int, _I64, _I64, _P, _P, _F,
                                              ctypes.c_int, _P]
            L.orc_dequantize_bf16.argtypes = [_P, _P, _F, _I64, _I64, _P]
            L.orc_residual_scores.argtypes = [_P, ctypes.c_int, _I64, _P, _P, _F, _I64, _I64, _P]
            L.orc_residual_scores_chunk128.argtypes = [_P, ctypes.c_int, _I64, _P, _P, _F, _I64,
                                                       _I64, _P]
            L.orc_topk.argtypes = [_P, _I64, _I64, _P]
            L.orc_residual_columns_bf16.argtypes = [_P, ctypes.c_int, _I64, _P, _P, _F, _I64,
                                                    _I64, _P, _I64, _P]
            L.orc_route.argtypes = [_P, _I64, _I64, _I64, _P, _P]
            L.orc_permute.restype = ctypes.c_int
            L.orc_permute.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P]
            L.orc_moe_gemm_w4a4.argtypes = [_P, _P, _F, _P, ctypes.c_int, _I64, _P, _I64, _P, _P,
                                            _P, _I64, _P, _P, _I64, _P, _I64, _P]
            L.orc_swiglu_bf16.argtypes = [_P, _I64, _I64, _P]
            L.orc_swiglu_backward.argtypes = [_P, ctypes.c_int, _I64, _I64, _P, _P]
            L.orc_combine_backward.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
            L.orc_combine_bf16.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
            L.orc_qat_fwd.argtypes = [_P, _I64, _P, _P, _I64, _I64, _P, _P, _P, _I64, _P, _I64, _P]
            L.orc_qat_dgrad.argtypes = [_P, _I64, _P, _P, _I64, _I64, _P, _P, _P, _I64, _P, _I64, _P]
            L.orc_qat_wgrad.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _P, _P, _I64, _P]
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return int(lib().orc_threads())


def e2m1_value(idx: int) -> float:
    return lib().orc_e2m1_value(idx)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def tensor_scale(amax: float) -> float:
    return lib().orc_tensor_scale(amax)


def to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_float_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _as_input(x):
    """Return (contiguous array, dtype code): float32 -> F32, uint16 (bf16 bits) -> BF16."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    return _c(x, np.float32), F32


def quantize(x, amax_in=None, threshold_form=False, K=None):
    """NVFP4 quantization of a [rows, K] tensor (fp32, or bf16 given as uint16 bits).
    With K given, x is [rows, ldx] and its first K columns are the tensor
    (row stride ldx = x.shape[1]).

    Returns (codes [rows, K/2] u8, scales [rows, K/16] u8, s_t float)."""
    xa, dt = _as_input(x)
    rows, ldx = xa.shape
    K = ldx if K is None else int(K)
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)
    st = np.zeros(1, np.float32)
    amax = None if amax_in is None else np.array([amax_in], np.float32)
    fn = lib().orc_quantize_threshold_form if threshold_form else lib().orc_quantize
    rc = fn(_ptr(xa), dt, rows, K, ldx, _ptr(amax), _ptr(codes), _ptr(scales), _ptr(st))
    if rc != 0:
        raise ValueError("oracle quantize failed: %d" % rc)
    return codes, scales, float(st[0])


GUIDE_MANTISSA, GUIDE_DIRECTION = 0, 1


def guidance_record(codes, scales, s_t, mode, x=None):
    """TRACE guidance record of a quantized [rows, K] tensor: bits [rows, K/8]
    (element c in bit c % 8 of byte c // 8).  Mantissa mode keeps each code's
    mantissa bit; direction mode keeps whether the rollout rounded |x| up
    (x needed)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    xa, dt = (None, F32) if x is None else _as_input(x)
    bits = np.empty((rows, K // 8), np.uint8)
    rc = lib().orc_guidance_record(_ptr(xa), dt, rows, K, _ptr(codes), _ptr(scales), s_t, mode,
                                   _ptr(bits))
    if rc != 0:
        raise ValueError("oracle guidance_record failed: %d" % rc)
    return bits


def guided_quantize(w, bits, scales, s_t, mode):
    """Codes [rows, K/2] of a (drifted) master tensor w rebuilt from a guidance
    record (bits, cached scales, cached s_t)."""
    wa, dt = _as_input(w)
    rows, K = wa.shape
    bits = _c(bits, np.uint8)
    scales = _c(scales, np.uint8)
    codes = np.empty((rows, K // 2), np.uint8)
    rc = lib().orc_guided_quantize(_ptr(wa), dt, rows, K, _ptr(bits), _ptr(scales), s_t, mode,
                                   _ptr(codes))
    if rc != 0:
        raise ValueError("oracle guided_quantize failed: %d" % rc)
    return codes


def dequantize(codes, scales, s_t, out="f32"):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    if out == "f32":
        y = np.empty((rows, K), np.float32)
        lib().orc_dequantize_f32(_ptr(codes), _ptr(scales), s_t, rows, K, _ptr(y))
    else:
        y = np.empty((rows, K), np.uint16)
        lib().orc_dequantize_bf16(_ptr(codes), _ptr(scales), s_t, rows, K, _ptr(y))
    return y


def residual_scores(x, codes, scales, s_t, order="sub16", K=None):
    """Per-channel residual score sum |x - deq(q(x))| (fp32 sums).  order
    "sub16": 16-row sequential sub-chunk sums, summed in order within 128-row
    chunks, chunks in order (the order the library computes); "chunk128": a
    sequential sum inside each 128-row chunk, chunks in order.  With K given,
    x is [rows, ldx] and its first K columns are the tensor."""
    xa, dt = _as_input(x)
    rows, ldx = xa.shape
    K = ldx if K is None else int(K)
    s = np.empty(K, np.float32)
    fn = {"sub16": lib().orc_residual_scores,
          "chunk128": lib().orc_residual_scores_chunk128}[order]
    fn(_ptr(xa), dt, ldx, _ptr(_c(codes, np.uint8)), _ptr(_c(scales, np.uint8)), s_t, rows, K,
       _ptr(s))
    return s


def double_to_bf16(v: float) -> int:
    """bf16 bit pattern of the fp64 value v, rounded once, to nearest even."""
    return int(lib().orc_double_to_bf16(float(v)))


def topk(scores, k):
    scores = _c(scores, np.float32)
    idx = np.empty(k, np.int32)
    lib().orc_topk(_ptr(scores), scores.size, k, _ptr(idx))
    return idx


def residual_columns_bf16(x, codes, scales, s_t, idx, K=None):
    """bf16(fl32(x - deq(q(x))))[:, idx]; with K given, x is [rows, ldx] and
    its first K columns are the tensor."""
    xa, dt = _as_input(x)
    rows, ldx = xa.shape
    K = ldx if K is None else int(K)
    idx = _c(idx, np.int32)
    out = np.empty((rows, idx.size), np.uint16)
    lib().orc_residual_columns_bf16(_ptr(xa), dt, ldx, _ptr(_c(codes, np.uint8)),
                                    _ptr(_c(scales, np.uint8)), s_t, rows, K, _ptr(idx),
                                    idx.size, _ptr(out))
    return out


def route(logits, topk_):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, topk_), np.int32)
    w = np.empty((T, topk_), np.float32)
    lib().orc_route(_ptr(logits), T, E, topk_, _ptr(ids), _ptr(w))
    return ids, w


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, topk_ = ids.shape
    P = T * topk_
    sp = np.empty(P, np.int32)
    off = np.empty(E + 1, np.int32)
    pos = np.empty(P, np.int32)
    rc = lib().orc_permute(_ptr(ids), T, topk_, E, _ptr(sp), _ptr(off), _ptr(pos))
    if rc != 0:
        raise ValueError("oracle permute failed: %d" % rc)
    return sp, off, pos


def moe_gemm_w4a4(a_codes, a_scales, a_st, x_hi, comp_idx, w_codes, w_scales, w_st,
                  row_token, row_expert, cols=None):
    """fp64 rows of the W4A4 + compensation GEMM; see orc_moe_gemm_w4a4."""
    a_codes = _c(a_codes, np.uint8)
    a_scales = _c(a_scales, np.uint8)
    K = a_codes.shape[1] * 2
    xa, dt = _as_input(x_hi)
    comp_idx = _c(comp_idx if comp_idx is not None else np.zeros(0), np.int32)
    w_codes = _c(w_codes, np.uint8)
    w_scales = _c(w_scales, np.uint8)
    if w_codes.ndim == 2:
        w_codes, w_scales = w_codes[None], w_scales[None]
    N = w_codes.shape[1]
    w_st = _c(np.atleast_1d(w_st), np.float32)
    row_token = _c(row_token, np.int32)
    row_expert = _c(row_expert, np.int32)
    colsa = None if cols is None else _c(cols, np.int32)
    ncol = N if cols is None else colsa.size
    out = np.empty((row_token.size, ncol), np.float64)
    lib().orc_moe_gemm_w4a4(_ptr(a_codes), _ptr(a_scales), a_st, _ptr(xa), dt, K, _ptr(comp_idx),
                            comp_idx.size, _ptr(w_codes), _ptr(w_scales), _ptr(w_st), N,
                            _ptr(row_token), _ptr(row_expert), row_token.size, _ptr(colsa), ncol,
                            _ptr(out))
    return out


def swiglu_bf16(y):
    y = _c(y, np.float64)
    rows, two_i = y.shape
    h = np.empty((rows, two_i // 2), np.uint16)
    lib().orc_swiglu_bf16(_ptr(y), rows, two_i // 2, _ptr(h))
    return h


def swiglu_backward(y1, dh_bf16):
    """fp64 [rows, 2I] gradient of h = silu(g) u with respect to (g, u), given
    the pre-activation y1 [rows, 2I] (fp32, or bf16 as uint16) and dh (bf16)."""
    ya, dt = _as_input(y1)
    rows, two_i = ya.shape
    dh = _c(dh_bf16, np.uint16)
    out = np.empty((rows, two_i), np.float64)
    lib().orc_swiglu_backward(_ptr(ya), dt, rows, two_i // 2, _ptr(dh), _ptr(out))
    return out


def combine_backward(dout_bf16, y_bf16, pos, w):
    """(dy bf16 [P, N], dw fp64 [T, topk]) of out = sum_j w y[pos]."""
    dout = _c(dout_bf16, np.uint16)
    y = _c(y_bf16, np.uint16)
    w = _c(w, np.float32)
    T, topk_ = w.shape
    N = dout.shape[1]
    dy = np.zeros((y.shape[0], N), np.uint16)
    dw = np.empty((T, topk_), np.float64)
    lib().orc_combine_backward(_ptr(dout), _ptr(y), _ptr(_c(pos, np.int32)), _ptr(w), T, topk_, N,
                               _ptr(dy), _ptr(dw))
    return dy, dw


def combine_bf16(y, pos, w):
    y = _c(y, np.float32)
    w = _c(w, np.float32)
    T, topk_ = w.shape
    N = y.shape[1]
    out = np.empty((T, N), np.uint16)
    lib().orc_combine_bf16(_ptr(y), _ptr(_c(pos, np.int32)), _ptr(w), T, topk_, N, _ptr(out))
    return out


def qat_fwd(a_bf16, a_row, row_expert, w_codes, w_scales, w_st, cols=None):
    a = _c(a_bf16, np.uint16)
    K = a.shape[1]
    w_codes = _c(w_codes, np.uint8)
    w_scales = _c(w_scales, np.uint8)
    if w_codes.ndim == 2:
        w_codes, w_scales = w_codes[None], w_scales[None]
    N = w_codes.shape[1]
    a_row = _c(a_row, np.int32)
    row_expert = _c(row_expert, np.int32)
    colsa = None if cols is None else _c(cols, np.int32)
    ncol = N if cols is None else colsa.size
    out = np.empty((a_row.size, ncol), np.float64)
    lib().orc_qat_fwd(_ptr(a), K, _ptr(a_row), _ptr(row_expert), a_row.size, K, _ptr(w_codes),
                      _ptr(w_scales), _ptr(_c(np.atleast_1d(w_st), np.float32)), N, _ptr(colsa),
                      ncol, _ptr(out))
    return out


def qat_dgrad(dy_bf16, dy_row, row_expert, w_codes, w_scales, w_st, cols=None):
    dy = _c(dy_bf16, np.uint16)
    N = dy.shape[1]
    w_codes = _c(w_codes, np.uint8)
    w_scales = _c(w_scales, np.uint8)
    if w_codes.ndim == 2:
        w_codes, w_scales = w_codes[None], w_scales[None]
    K = w_codes.shape[2] * 2
    dy_row = _c(dy_row, np.int32)
    row_expert = _c(row_expert, np.int32)
    colsa = None if cols is None else _c(cols, np.int32)
    ncol = K if cols is None else colsa.size
    out = np.empty((dy_row.size, ncol), np.float64)
    lib().orc_qat_dgrad(_ptr(dy), N, _ptr(dy_row), _ptr(row_expert), dy_row.size, N,
                        _ptr(w_codes), _ptr(w_scales), _ptr(_c(np.atleast_1d(w_st), np.float32)),
                        K, _ptr(colsa), ncol, _ptr(out))
    return out


def qat_wgrad(dy_bf16, a_bf16, a_row, p0, p1, ns, cs):
    dy = _c(dy_bf16, np.uint16)
    a = _c(a_bf16, np.uint16)
    ns = _c(ns, np.int32)
    cs = _c(cs, np.int32)
    out = np.empty(ns.size, np.float64)
    lib().orc_qat_wgrad(_ptr(dy), dy.shape[1], _ptr(a), a.shape[1], _ptr(_c(a_row, np.int32)),
                        p0, p1, _ptr(ns), _ptr(cs), ns.size, _ptr(out))
    return out

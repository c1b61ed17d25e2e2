"""Thin Python binding of libnvq.so (include/nvq.h): argument marshalling only.

torch provides device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: if
the library is missing or the device is not a GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvq.so")

NVQ_F32, NVQ_BF16 = 0, 1
NVQ_EPI_NONE, NVQ_EPI_SWIGLU = 0, 1
NVQ_GEMM_AUTO, NVQ_GEMM_DEQ16, NVQ_GEMM_FP8_BLOCK, NVQ_GEMM_DEQ16_WIDE = 0, 1, 2, 3
NVQ_QAT_FWD, NVQ_QAT_DGRAD, NVQ_QAT_WGRAD = 0, 1, 2
NVQ_STATUS_NONFINITE, NVQ_STATUS_BAD_EXPERT = 1, 2
NVQ_GUIDE_MANTISSA, NVQ_GUIDE_DIRECTION = 0, 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_lock = threading.Lock()
_lib = None


class NvqError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({status_string(code)})")
        self.code = code


class MoeGemmArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _SZ), ("rows", _I64), ("K", _I64), ("N", _I64), ("E", _I64),
        ("a_rows", _I64), ("a_row", _P), ("expert_offsets", _P), ("a_codes", _P),
        ("a_scales", _P), ("a_tensor_scale", _P), ("a_resid", _P), ("comp_idx", _P),
        ("k", _I32), ("w_codes", _P), ("w_scales", _P), ("w_tensor_scale", _P),
        ("epilogue", _I32), ("path", _I32), ("out_bf16", _P), ("out_f32", _P),
        ("ws", _P), ("ws_bytes", _SZ), ("a_row_div", _I32), ("w_codes_cm", _P),
        ("w_scales_cm", _P), ("h_amax", _P), ("comb_pair", _P), ("comb_pos", _P),
        ("comb_weights", _P), ("comb_T", _I64), ("comb_topk", _I32), ("comb_out", _P),
    ]


class QatGemmArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _SZ), ("mode", _I32), ("accumulate", _I32), ("rows", _I64), ("K", _I64),
        ("N", _I64), ("E", _I64), ("x_rows", _I64), ("a_row", _P), ("expert_offsets", _P),
        ("x", _P), ("dy", _P), ("w_codes", _P), ("w_scales", _P), ("w_tensor_scale", _P),
        ("out_bf16", _P), ("out_f32", _P), ("dw", _P), ("ws", _P), ("ws_bytes", _SZ),
    ]


# (name, restype, argtypes)
_SIGS = [
    ("nvq_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("nvq_device_status", ctypes.c_int, [_P, _P, ctypes.POINTER(ctypes.c_uint32)]),
    ("nvfp4_quantize_workspace_bytes", _SZ, [_I64, _I64, _I64]),
    ("nvfp4_quantize", ctypes.c_int,
     [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("nvfp4_quantize_noalloc", ctypes.c_int,
     [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    ("nvfp4_dequantize", ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _P]),
    ("nvfp4_guidance_record", ctypes.c_int,
     [_P, ctypes.c_int, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P]),
    ("nvfp4_guided_quantize", ctypes.c_int,
     [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, ctypes.c_int, _P, _P, _SZ, _P]),
    ("residual_topk_workspace_bytes", _SZ, [_I64, _I64, _I32]),
    ("residual_topk_channels", ctypes.c_int,
     [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    ("nvq_moe_route", ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    ("nvq_moe_permute_workspace_bytes", _SZ, [_I64, _I64, _I64]),
    ("nvq_moe_permute", ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    ("nvq_moe_combine", ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P]),
    ("nvq_swiglu_forward", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, _P]),
    ("nvq_swiglu_backward", ctypes.c_int, [_P, ctypes.c_int, _P, _I64, _I64, _P, _P]),
    ("nvq_moe_combine_backward", ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P]),
    ("nvfp4_channel_major", ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P, _P]),
    ("moe_gemm_workspace_bytes", _SZ, [_I64, _I64, _I64, _I32]),
    ("moe_gemm_workspace_bytes_comb", _SZ, [_I64, _I64, _I64, _I32, _I64]),
    ("moe_grouped_gemm_w4a4_comp", ctypes.c_int, [ctypes.POINTER(MoeGemmArgs), _P]),
    ("qat_gemm_workspace_bytes", _SZ, [_I64, _I64]),
    ("qat_fakequant_gemm_w4a16", ctypes.c_int, [ctypes.POINTER(QatGemmArgs), _P]),
]

EXPORTED = [s[0] for s in _SIGS]


def load(path: str = LIB_PATH):
    """Load libnvq.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m qat_nvfp4_quantize_amd.build`")
            L = ctypes.CDLL(path)
            for name, res, args in _SIGS:
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def status_string(code: int) -> str:
    try:
        return load().nvq_status_string(code).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(fn, rc):
    if rc != 0:
        raise NvqError(fn, rc)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dev_rows(t, name):
    """A GPU tensor whose rows may be strided: [rows, K] or [batch, rows, K]
    with unit element stride and (for 3-D) items rows * ldx elements apart.
    Returns ldx, the row stride in elements."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() not in (2, 3) or t.stride(-1) != 1:
        raise ValueError(f"{name} must be [rows, K] or [batch, rows, K] with unit column stride")
    rows, K = t.shape[-2], t.shape[-1]
    many = t.dim() == 3 and t.shape[0] > 1
    if rows > 1:
        ldx = t.stride(-2)
    else:  # one row per item: the item stride is the row stride
        ldx = t.stride(0) if many else K
    if many and t.stride(0) != rows * ldx:
        raise ValueError(f"{name}: batch items must be rows * ldx elements apart")
    return ldx


def _dtype_code(t):
    if t.dtype == torch.float32:
        return NVQ_F32
    if t.dtype == torch.bfloat16:
        return NVQ_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def device_status(ws: torch.Tensor) -> int:
    v = ctypes.c_uint32(0)
    _check("nvq_device_status", load().nvq_device_status(_ptr(ws), _stream(), ctypes.byref(v)))
    return v.value


# ----------------------------------------------------------------- quantize --
def nvfp4_quantize(x, amax_in=None, score=False, ws=None, out=None):
    """NVFP4-quantize x [rows, K] or [batch, rows, K] (fp32/bf16); rows may be
    strided (a column slice of a wider tensor).

    Returns (codes u8 [..., K/2], scales u8 [..., K/16], tensor_scale f32 [batch],
    score f32 [K] or None, ws)."""
    ldx = _dev_rows(x, "x")
    L = load()
    batch, rows, K = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
    lead = x.shape[:-1]
    if out is None:
        codes = torch.empty(*lead, K // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*lead, K // 16, dtype=torch.uint8, device=x.device)
        st = torch.empty(batch, dtype=torch.float32, device=x.device)
        sc = torch.empty(K, dtype=torch.float32, device=x.device) if score else None
    else:
        codes, scales, st, sc = out
    if ws is None:
        ws = workspace(L.nvfp4_quantize_workspace_bytes(batch, rows, K), x.device)
    if amax_in is not None:
        _dev(amax_in, "amax_in")
    rc = L.nvfp4_quantize(_ptr(x), _dtype_code(x), batch, rows, K, ldx, _ptr(amax_in),
                          _ptr(codes), _ptr(scales), _ptr(st), _ptr(sc), _ptr(ws), ws.numel(),
                          _stream())
    _check("nvfp4_quantize", rc)
    return codes, scales, st, sc, ws


NVQ_QUANTIZE_NOALLOC_SCRATCH_BYTES = 16 << 20


def nvfp4_quantize_noalloc(x, amax_in=None, score=False, out=None):
    """nvfp4_quantize without a workspace: the library's static per-device
    scratch serves the call (calls on one GPU must not overlap).  Returns
    (codes, scales, tensor_scale, score or None)."""
    ldx = _dev_rows(x, "x")
    batch, rows, K = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
    lead = x.shape[:-1]
    if out is None:
        codes = torch.empty(*lead, K // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*lead, K // 16, dtype=torch.uint8, device=x.device)
        st = torch.empty(batch, dtype=torch.float32, device=x.device)
        sc = torch.empty(K, dtype=torch.float32, device=x.device) if score else None
    else:
        codes, scales, st, sc = out
    if amax_in is not None:
        _dev(amax_in, "amax_in")
    rc = load().nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x), batch, rows, K, ldx,
                                       _ptr(amax_in), _ptr(codes), _ptr(scales), _ptr(st),
                                       _ptr(sc), _stream())
    _check("nvfp4_quantize_noalloc", rc)
    return codes, scales, st, sc


def nvfp4_dequantize(codes, scales, tensor_scale, out_dtype=torch.float32, batch=None, out=None):
    _dev(codes, "codes")
    K = codes.shape[-1] * 2
    if batch is None:
        batch = tensor_scale.numel()
    rows = codes.numel() // (K // 2) // batch
    y = out if out is not None else torch.empty(*codes.shape[:-1], K, dtype=out_dtype,
                                                device=codes.device)
    rc = load().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tensor_scale), batch, rows, K,
                                 _ptr(y), _dtype_code(y), _stream())
    _check("nvfp4_dequantize", rc)
    return y


def _batch_rows(t, per_row, batch):
    """(batch, rows) of a [rows, n] or [batch, rows, n] tensor."""
    if batch is None:
        batch = t.shape[0] if t.dim() == 3 else 1
    return batch, t.numel() // per_row // batch


def nvfp4_guidance_record(codes, mode, x=None, scales=None, tensor_scale=None, batch=None,
                          out=None):
    """TRACE guidance record of an NVFP4 record: bits u8 [..., K/8].  Mantissa
    mode needs only the codes; direction mode needs x (the quantized values),
    scales and tensor_scale."""
    _dev(codes, "codes")
    K = codes.shape[-1] * 2
    batch, rows = _batch_rows(codes, K // 2, batch)
    bits = out if out is not None else torch.empty(
        *codes.shape[:-1], K // 8, dtype=torch.uint8, device=codes.device)
    xd = _dtype_code(x) if x is not None else NVQ_F32
    rc = load().nvfp4_guidance_record(_ptr(x), xd, _ptr(codes), _ptr(scales), _ptr(tensor_scale),
                                      batch, rows, K, mode, _ptr(bits), _stream())
    _check("nvfp4_guidance_record", rc)
    return bits


def nvfp4_guided_quantize(w, bits, scales, tensor_scale, mode, ws=None, out=None):
    """Codes u8 [..., K/2] of master values w rebuilt from a guidance record
    (bits, the rollout's scales and tensor scales).  ws (optional, >= 256
    bytes) receives the non-finite status bit."""
    _dev(w, "w")
    K = w.shape[-1]
    batch, rows = _batch_rows(w, K, None)
    codes = out if out is not None else torch.empty(
        *w.shape[:-1], K // 2, dtype=torch.uint8, device=w.device)
    rc = load().nvfp4_guided_quantize(_ptr(w), _dtype_code(w), batch, rows, K, _ptr(bits),
                                      _ptr(scales), _ptr(tensor_scale), mode, _ptr(codes),
                                      _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check("nvfp4_guided_quantize", rc)
    return codes


def residual_topk_channels(x, codes, scales, tensor_scale, k, scores=None, want_scores=False,
                           want_resid=True, ws=None):
    """Returns (idx int32 [k], resid bf16 [rows, k] or None, scores f32 [K] or None).
    x [rows, K] may have strided rows."""
    ldx = _dev_rows(x, "x")
    L = load()
    rows, K = x.shape
    idx = torch.empty(max(k, 1), dtype=torch.int32, device=x.device)
    resid = torch.empty(rows, max(k, 1), dtype=torch.bfloat16, device=x.device) if want_resid else None
    sc_out = torch.empty(K, dtype=torch.float32, device=x.device) if want_scores else None
    if ws is None:
        ws = workspace(L.residual_topk_workspace_bytes(rows, K, k), x.device)
    rc = L.residual_topk_channels(_ptr(x), _dtype_code(x), rows, K, ldx, _ptr(codes), _ptr(scales),
                                  _ptr(tensor_scale), _ptr(scores), _ptr(sc_out), k, _ptr(idx),
                                  _ptr(resid), _ptr(ws), ws.numel(), _stream())
    _check("residual_topk_channels", rc)
    return idx[:k], (resid[:, :k] if resid is not None else None), sc_out


# ---------------------------------------------------------------- MoE glue --
def nvq_moe_route(logits, topk):
    _dev(logits, "logits")
    T, E = logits.shape
    ids = torch.empty(T, topk, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, topk, dtype=torch.float32, device=logits.device)
    _check("nvq_moe_route", load().nvq_moe_route(_ptr(logits), T, E, topk, _ptr(ids), _ptr(w),
                                                 _stream()))
    return ids, w


def nvq_moe_permute(ids, E, ws=None):
    _dev(ids, "ids")
    L = load()
    T, topk = ids.shape
    P = T * topk
    sp = torch.empty(P, dtype=torch.int32, device=ids.device)
    off = torch.empty(E + 1, dtype=torch.int32, device=ids.device)
    pos = torch.empty(P, dtype=torch.int32, device=ids.device)
    if ws is None:
        ws = workspace(L.nvq_moe_permute_workspace_bytes(T, topk, E), ids.device)
    _check("nvq_moe_permute", L.nvq_moe_permute(_ptr(ids), T, topk, E, _ptr(sp), _ptr(off),
                                                _ptr(pos), _ptr(ws), ws.numel(), _stream()))
    return sp, off, pos, ws


def nvq_moe_combine(y, pos, weights, out=None, out_amax=None):
    """out bf16 [T, N]; out_amax (optional fp32 [1] on the GPU) receives max |out|."""
    _dev(y, "y")
    T, topk = weights.shape
    N = y.shape[1]
    if out is None:
        out = torch.empty(T, N, dtype=torch.bfloat16, device=y.device)
    _check("nvq_moe_combine", load().nvq_moe_combine(_ptr(y), _ptr(pos), _ptr(weights), T, topk,
                                                     N, _ptr(out), _ptr(out_amax), _stream()))
    return out


def nvq_swiglu_forward(y1, out=None):
    """h bf16 [rows, I] = silu(y1[:, :I]) * y1[:, I:] (y1 fp32 or bf16 [rows, 2I])."""
    _dev(y1, "y1")
    rows, two_i = y1.shape
    h = out if out is not None else torch.empty(rows, two_i // 2, dtype=torch.bfloat16,
                                                device=y1.device)
    _check("nvq_swiglu_forward", load().nvq_swiglu_forward(_ptr(y1), _dtype_code(y1), rows,
                                                           two_i // 2, _ptr(h), _stream()))
    return h


def nvq_swiglu_backward(y1, dh, out=None):
    """dy1 bf16 [rows, 2I]: gradient of h = silu(g) u w.r.t. (g, u) given dh."""
    _dev(y1, "y1")
    _dev(dh, "dh")
    rows, two_i = y1.shape
    dy1 = out if out is not None else torch.empty(rows, two_i, dtype=torch.bfloat16,
                                                  device=y1.device)
    _check("nvq_swiglu_backward", load().nvq_swiglu_backward(
        _ptr(y1), _dtype_code(y1), _ptr(dh), rows, two_i // 2, _ptr(dy1), _stream()))
    return dy1


def nvq_moe_combine_backward(dout, pos, weights, rows, y=None, want_dw=True, out=None):
    """(dy bf16 [rows, N] in sorted-pair order, dw fp32 [T, topk] or None)."""
    _dev(dout, "dout")
    T, N = dout.shape
    topk = weights.shape[1]
    if out is not None:
        dy, dw = out
    else:
        dy = torch.empty(rows, N, dtype=torch.bfloat16, device=dout.device)
        dw = torch.empty(T, topk, dtype=torch.float32, device=dout.device) if want_dw else None
    _check("nvq_moe_combine_backward", load().nvq_moe_combine_backward(
        _ptr(dout), _ptr(y), _ptr(pos), _ptr(weights), T, topk, N, _ptr(dy), _ptr(dw), _stream()))
    return dy, dw


# ------------------------------------------------------------------- GEMMs --
def nvfp4_channel_major(codes, scales, out=None):
    """Channel-major copy of a weight record: codes [B, N, K/2] -> [B, K, N/2],
    scales [B, N, K/16] -> [B, K/16, N].  Returns (codes_cm, scales_cm)."""
    _dev(codes, "codes")
    L = load()
    if codes.dim() == 2:
        codes, scales = codes.unsqueeze(0), scales.unsqueeze(0)
    B, N, Kh = codes.shape
    K = Kh * 2
    if out is None:
        out = (torch.empty(B, K, N // 2, dtype=torch.uint8, device=codes.device),
               torch.empty(B, K // 16, N, dtype=torch.uint8, device=codes.device))
    _check("nvfp4_channel_major",
           L.nvfp4_channel_major(_ptr(codes), _ptr(scales), B, N, K, _ptr(out[0]), _ptr(out[1]),
                                 _stream()))
    return out


def moe_grouped_gemm_w4a4_comp(a_codes, a_scales, a_tensor_scale, w_codes, w_scales,
                               w_tensor_scale, expert_offsets, rows, a_row=None, a_resid=None,
                               comp_idx=None, epilogue=NVQ_EPI_NONE, path=NVQ_GEMM_AUTO,
                               want_bf16=True, want_f32=False, ws=None, a_row_div=0, out=None,
                               w_cm=None, h_amax=None, comb=None):
    """Returns (out_bf16 or None, out_f32 or None).  w_cm: optional
    (codes_cm, scales_cm) from nvfp4_channel_major for the compensation gather.
    comb: optional (sorted_pair, pos, weights, out) -- the layer's combine fused
    into this call, written to out bf16 [T, N]."""
    L = load()
    E, N, Kh = w_codes.shape
    K = Kh * 2
    dev = w_codes.device
    k = 0 if comp_idx is None else int(comp_idx.numel())
    n_out = N // 2 if epilogue == NVQ_EPI_SWIGLU else N
    if out is not None:
        ob, of = out
    else:
        ob = torch.empty(rows, n_out, dtype=torch.bfloat16, device=dev) if want_bf16 else None
        of = torch.empty(rows, N, dtype=torch.float32, device=dev) if want_f32 else None
    if ws is None:
        if comb is None:
            ws = workspace(L.moe_gemm_workspace_bytes(rows, E, N, k), dev)
        else:
            ws = workspace(L.moe_gemm_workspace_bytes_comb(rows, E, N, k, comb[2].shape[0]), dev)
    a = MoeGemmArgs()
    a.struct_size = ctypes.sizeof(MoeGemmArgs)
    a.rows, a.K, a.N, a.E = rows, K, N, E
    a.a_rows = a_codes.shape[0]
    a.a_row = _ptr(a_row)
    a.expert_offsets = _ptr(expert_offsets)
    a.a_codes, a.a_scales, a.a_tensor_scale = _ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale)
    a.a_resid = _ptr(a_resid)
    a.comp_idx = _ptr(comp_idx)
    a.k = k
    a.w_codes, a.w_scales, a.w_tensor_scale = _ptr(w_codes), _ptr(w_scales), _ptr(w_tensor_scale)
    a.epilogue, a.path = epilogue, path
    a.out_bf16, a.out_f32 = _ptr(ob), _ptr(of)
    a.ws, a.ws_bytes = _ptr(ws), ws.numel()
    a.a_row_div = int(a_row_div)
    if w_cm is not None:
        a.w_codes_cm, a.w_scales_cm = _ptr(w_cm[0]), _ptr(w_cm[1])
    a.h_amax = _ptr(h_amax)
    if comb is not None:
        sp, pos, wts, cout = comb
        a.comb_pair, a.comb_pos, a.comb_weights = _ptr(sp), _ptr(pos), _ptr(wts)
        a.comb_T, a.comb_topk = wts.shape[0], wts.shape[1]
        a.comb_out = _ptr(cout)
    _check("moe_grouped_gemm_w4a4_comp", L.moe_grouped_gemm_w4a4_comp(ctypes.byref(a), _stream()))
    return ob, of


def qat_fakequant_gemm_w4a16(mode, w_codes, w_scales, w_tensor_scale, expert_offsets, rows,
                             x=None, dy=None, a_row=None, dw=None, accumulate=False,
                             want_bf16=True, want_f32=False, ws=None, out=None):
    """FWD: returns (y_bf16, y_f32); DGRAD: (dx_bf16, dx_f32); WGRAD: dw [E, N, K] fp32."""
    L = load()
    E, N, Kh = w_codes.shape
    K = Kh * 2
    dev = w_codes.device
    ob = of = None
    if mode in (NVQ_QAT_FWD, NVQ_QAT_DGRAD):
        cols = N if mode == NVQ_QAT_FWD else K
        if out is not None:
            ob, of = out
        else:
            ob = torch.empty(rows, cols, dtype=torch.bfloat16, device=dev) if want_bf16 else None
            of = torch.empty(rows, cols, dtype=torch.float32, device=dev) if want_f32 else None
    elif dw is None:
        dw = torch.empty(E, N, K, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(L.qat_gemm_workspace_bytes(rows, E), dev)
    a = QatGemmArgs()
    a.struct_size = ctypes.sizeof(QatGemmArgs)
    a.mode, a.accumulate = mode, int(bool(accumulate))
    a.rows, a.K, a.N, a.E = rows, K, N, E
    a.x_rows = 0 if x is None else x.shape[0]
    a.a_row = _ptr(a_row)
    a.expert_offsets = _ptr(expert_offsets)
    a.x, a.dy = _ptr(x), _ptr(dy)
    a.w_codes, a.w_scales, a.w_tensor_scale = _ptr(w_codes), _ptr(w_scales), _ptr(w_tensor_scale)
    a.out_bf16, a.out_f32 = _ptr(ob), _ptr(of)
    a.dw = _ptr(dw)
    a.ws, a.ws_bytes = _ptr(ws), ws.numel()
    _check("qat_fakequant_gemm_w4a16", L.qat_fakequant_gemm_w4a16(ctypes.byref(a), _stream()))
    if mode == NVQ_QAT_WGRAD:
        return dw
    return ob, of

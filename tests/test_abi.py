"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from qat_nvfp4_quantize_amd import nvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvq.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def _lib():
    if not os.path.exists(nvq.LIB_PATH):
        pytest.skip("libnvq.so not built")
    return nvq.load()


def test_header_declares_the_five_entry_points():
    names = _declared_functions()
    for n in ("nvfp4_quantize", "nvfp4_dequantize", "residual_topk_channels",
              "moe_grouped_gemm_w4a4_comp", "qat_fakequant_gemm_w4a16"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    missing = [n for n in _declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(nvq.EXPORTED) == _declared_functions()


def test_status_strings():
    L = _lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.nvq_status_string(code)


def test_host_side_validation_launches_nothing():
    L = _lib()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every call below fails validation first
    # channel-major relayout: null pointer, N not a multiple of 16, misaligned codes
    assert L.nvfp4_channel_major(None, fake, 1, 32, 32, fake, fake, None) == -1
    assert L.nvfp4_channel_major(fake, fake, 1, 24, 32, fake, fake, None) == -2
    assert L.nvfp4_channel_major(P(0x1004), fake, 1, 32, 32, fake, fake, None) == -3
    # null x
    assert L.nvfp4_quantize(None, 1, 1, 4, 32, 0, None, fake, fake, fake, None, fake, 1 << 20,
                            None) == -1
    # K not a multiple of 16
    assert L.nvfp4_quantize(fake, 1, 1, 4, 24, 0, None, fake, fake, fake, None, fake, 1 << 20,
                            None) == -2
    # bad dtype
    assert L.nvfp4_quantize(fake, 7, 1, 4, 32, 0, None, fake, fake, fake, None, fake, 1 << 20,
                            None) == -1
    # misaligned x
    assert L.nvfp4_quantize(P(0x1002), 1, 1, 4, 32, 0, None, fake, fake, fake, None, fake, 1 << 20,
                            None) == -3
    # row stride: shorter than a row, or rows not 16-byte aligned (bf16: ldx % 8)
    assert L.nvfp4_quantize(fake, 1, 1, 4, 32, 16, None, fake, fake, fake, None, fake, 1 << 20,
                            None) == -2
    assert L.nvfp4_quantize(fake, 1, 1, 4, 32, 36, None, fake, fake, fake, None, fake, 1 << 20,
                            None) == -3
    assert L.nvfp4_quantize(fake, 0, 1, 4, 32, 34, None, fake, fake, fake, None, fake, 1 << 20,
                            None) == -3
    # workspace too small
    need = L.nvfp4_quantize_workspace_bytes(1, 4, 32)
    assert need >= 256
    assert L.nvfp4_quantize(fake, 1, 1, 4, 32, 0, None, fake, fake, fake, None, fake, need - 1,
                            None) == -4
    # scores need batch == 1
    assert L.nvfp4_quantize(fake, 1, 2, 4, 32, 0, None, fake, fake, fake, fake, fake, 1 << 20,
                            None) == -2
    # k > K; row stride shorter than a row
    assert L.residual_topk_channels(fake, 1, 4, 32, 0, fake, fake, fake, None, None, 33, fake, None,
                                    fake, 1 << 20, None) == -2
    assert L.residual_topk_channels(fake, 1, 4, 32, 31, fake, fake, fake, None, None, 3, fake,
                                    None, fake, 1 << 20, None) == -2
    # route: topk > E, E too large
    assert L.nvq_moe_route(fake, 4, 8, 9, fake, fake, None) == -2
    assert L.nvq_moe_route(fake, 4, 2048, 8, fake, fake, None) == -2
    assert L.nvq_moe_combine(fake, fake, fake, 4, 2, 12, fake, None, None) == -2
    assert L.nvq_moe_combine(fake, fake, fake, 4, 2, 16, fake, P(0x1002), None) == -3
    assert L.nvfp4_dequantize(fake, fake, fake, 1, 4, 24, fake, 0, None) == -2


def test_gemm_args_validation():
    L = _lib()
    a = nvq.MoeGemmArgs()
    a.struct_size = 8  # too small for this ABI
    assert L.moe_grouped_gemm_w4a4_comp(ctypes.byref(a), None) in (-1, -6)
    assert L.moe_grouped_gemm_w4a4_comp(None, None) in (-1, -6)
    q = nvq.QatGemmArgs()
    q.struct_size = 8
    assert L.qat_fakequant_gemm_w4a16(ctypes.byref(q), None) in (-1, -6)


def test_guided_rounding_validation():
    L = _lib()
    P = ctypes.c_void_p
    fake = P(0x1000)
    # record: bad mode, direction mode without x, K % 16, misaligned codes / bits / x
    assert L.nvfp4_guidance_record(None, 0, fake, None, None, 1, 4, 32, 2, fake, None) == -1
    assert L.nvfp4_guidance_record(None, 0, fake, fake, fake, 1, 4, 32, 1, fake, None) == -1
    assert L.nvfp4_guidance_record(None, 0, fake, None, None, 1, 4, 24, 0, fake, None) == -2
    assert L.nvfp4_guidance_record(None, 0, P(0x1004), None, None, 1, 4, 32, 0, fake, None) == -3
    assert L.nvfp4_guidance_record(None, 0, fake, None, None, 1, 4, 32, 0, P(0x1001), None) == -3
    assert L.nvfp4_guidance_record(P(0x1008), 1, fake, fake, fake, 1, 4, 32, 1, fake, None) == -3
    # no rows: nothing to do, NULL buffers allowed
    assert L.nvfp4_guidance_record(None, 0, None, None, None, 1, 0, 32, 0, None, None) == 0
    # guided requantization: bad dtype / mode, null pointers, shape, alignment, workspace
    assert L.nvfp4_guided_quantize(fake, 5, 1, 4, 32, fake, fake, fake, 0, fake, None, 0, None) == -1
    assert L.nvfp4_guided_quantize(fake, 1, 1, 4, 32, fake, fake, fake, 3, fake, None, 0, None) == -1
    assert L.nvfp4_guided_quantize(fake, 1, 1, 4, 32, None, fake, fake, 0, fake, None, 0, None) == -1
    assert L.nvfp4_guided_quantize(fake, 1, 1, 4, 40, fake, fake, fake, 0, fake, None, 0, None) == -2
    assert L.nvfp4_guided_quantize(fake, 1, 0, 4, 32, fake, fake, fake, 0, fake, None, 0, None) == -2
    assert L.nvfp4_guided_quantize(P(0x1008), 1, 1, 4, 32, fake, fake, fake, 0, fake, None, 0,
                                   None) == -3
    assert L.nvfp4_guided_quantize(fake, 1, 1, 4, 32, fake, fake, fake, 0, P(0x1004), None, 0,
                                   None) == -3
    assert L.nvfp4_guided_quantize(fake, 1, 1, 4, 32, fake, fake, fake, 0, fake, P(0x1080), 256,
                                   None) == -3
    assert L.nvfp4_guided_quantize(fake, 1, 1, 4, 32, fake, fake, fake, 0, fake, fake, 255,
                                   None) == -4


def test_backward_glue_validation():
    L = _lib()
    P = ctypes.c_void_p
    fake = P(0x1000)
    # SwiGLU: bad dtype, I % 8, misaligned, null with rows
    assert L.nvq_swiglu_forward(fake, 7, 4, 16, fake, None) == -1
    assert L.nvq_swiglu_forward(fake, 1, 4, 12, fake, None) == -2
    assert L.nvq_swiglu_forward(P(0x1008), 1, 4, 16, fake, None) == -3
    assert L.nvq_swiglu_forward(None, 1, 4, 16, fake, None) == -1
    assert L.nvq_swiglu_forward(None, 1, 0, 16, None, None) == 0  # no rows
    assert L.nvq_swiglu_backward(fake, 1, fake, 4, 16, P(0x1004), None) == -3
    assert L.nvq_swiglu_backward(fake, 1, None, 4, 16, fake, None) == -1
    # combine backward: N % 8, topk < 1, dw without y, misaligned
    assert L.nvq_moe_combine_backward(fake, fake, fake, fake, 4, 2, 12, fake, None, None) == -2
    assert L.nvq_moe_combine_backward(fake, fake, fake, fake, 4, 0, 16, fake, None, None) == -2
    assert L.nvq_moe_combine_backward(fake, None, fake, fake, 4, 2, 16, fake, fake, None) == -1
    assert L.nvq_moe_combine_backward(P(0x1002), fake, fake, fake, 4, 2, 16, fake, None, None) == -3
    assert L.nvq_moe_combine_backward(None, None, None, None, 0, 2, 16, None, None, None) == 0


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No library means an error, never a CPU fallback."""
    from qat_nvfp4_quantize_amd import nvq as mod

    saved = mod._lib
    mod._lib = None
    try:
        with pytest.raises(RuntimeError):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

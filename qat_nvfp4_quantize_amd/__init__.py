"""NVFP4 quantization, W4A4 MoE grouped GEMM with residual compensation and
asymmetric W4A16 QAT GEMMs for MI355X (gfx950).

The compute lives in ``libnvq.so`` (hand-written HIP kernels behind a C ABI,
``include/nvq.h``).  ``qat_nvfp4_quantize_amd.nvq`` is the thin ctypes binding
with the same entry-point names; it loads the library lazily and raises if it
is missing -- there is no CPU fallback.
"""

"""The allocation-free quantizer entry point (nvfp4_quantize_noalloc, for
callers that cannot allocate) against nvfp4_quantize with a caller workspace:
identical records and residual scores on calls in a row, the second one
smaller than the first, so the shared scratch keeps the previous call's
contents; a request beyond the scratch size is refused before any launch."""
import ctypes

import numpy as np
import pytest

from helpers import assert_bits_equal, log, to_gpu, to_np
from qat_nvfp4_quantize_amd import inputs

pytestmark = pytest.mark.gpu


def _same(ref, got, what):
    for name, a, b in zip(("codes", "scales", "s_t", "score"), ref[:4], got[:4]):
        if a is None:
            assert b is None, (what, name)
            continue
        assert_bits_equal(to_np(b), to_np(a), f"{what} {name}")


def test_noalloc_quantize_matches_the_workspace_entry_point():
    import torch

    from qat_nvfp4_quantize_amd import nvq

    g = np.random.default_rng(404)
    small = (g.standard_t(3, (300, 2064)) * np.exp(g.uniform(-3, 3, (1, 2064)))).astype(np.float32)
    wide = inputs.to_bf16_bits(g.standard_normal((3, 40, 96)).astype(np.float32))
    cases = [
        ("sweep 8192x7168 bf16, scored", to_gpu(inputs.quant_sweep()), True, None),
        ("300x2064 f32, scored", to_gpu(small), True, None),
        ("3x40x80 bf16 strided items, no score", to_gpu(wide)[:, :, :80], False, None),
        ("300x2064 f32, amax_in", to_gpu(small), True, 7.5),
    ]
    for what, xg, score, amax in cases:
        log(f"[noalloc] {what}")
        a = None if amax is None else torch.tensor([amax], dtype=torch.float32, device="cuda")
        ref = nvq.nvfp4_quantize(xg, amax_in=a, score=score)
        got = nvq.nvfp4_quantize_noalloc(xg, amax_in=a, score=score)
        torch.cuda.synchronize()
        _same(ref, got, what)


def test_noalloc_refuses_requests_beyond_its_scratch():
    from qat_nvfp4_quantize_amd import nvq

    L = nvq.load()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the size check fails first
    rows, K = 200000, 8192  # residual chunk partials alone: 1563 x 8192 x 4 B > 16 MiB
    assert L.nvfp4_quantize_workspace_bytes(1, rows, K) > nvq.NVQ_QUANTIZE_NOALLOC_SCRATCH_BYTES
    assert L.nvfp4_quantize_noalloc(fake, 1, 1, rows, K, 0, None, fake, fake, fake, fake,
                                    None) == -4

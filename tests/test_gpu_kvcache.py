"""GPU parity of the NVFP4 quantizer and dequantizer on FP4 KV-cache shapes
(TRACE post, results: FP4 weights, activations and KV cache in the rollout):
K and V caches of one attention layer quantized as two tensors with 16-element
blocks along the head dimension, a static tensor scale shared with the decode
steps that append to the cache, and a dynamic (own amax) variant.  Bit-exact
against the oracle on sampled rows of the full cache and on whole small caches."""
import numpy as np
import pytest

import oracle
from helpers import assert_bits_equal, log, to_gpu, to_np
from qat_nvfp4_quantize_amd import inputs

pytestmark = pytest.mark.gpu


def _nvq():
    from qat_nvfp4_quantize_amd import nvq

    return nvq


def _sample_rows(n):
    r = np.arange(0, n, 97)
    return np.unique(np.concatenate([r, [0, n - 1]]))


def _check_sampled(kv_bits_item, codes, scales, amax, what):
    rows = _sample_rows(kv_bits_item.shape[0])
    x = kv_bits_item[rows]
    oc, os_, ost = oracle.quantize(x, amax_in=amax)
    assert_bits_equal(to_np(codes)[rows], oc, what + " codes")
    assert_bits_equal(to_np(scales)[rows], os_, what + " scales")
    return rows, oc, os_, ost


def test_kv_cache_static_scale_full_size():
    import torch

    nvq = _nvq()
    kv = inputs.kv_cache(device="cuda")
    log(f"[kv] static scale {tuple(kv.shape)}")
    amax = torch.full((2,), inputs.KV_STATIC_AMAX, dtype=torch.float32, device="cuda")
    codes, scales, st, _, ws = nvq.nvfp4_quantize(kv, amax_in=amax)
    deq = nvq.nvfp4_dequantize(codes, scales, st, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert to_np(st).tolist() == [2.0 ** -6, 2.0 ** -6]
    assert nvq.device_status(ws) == 0
    for i, name in enumerate("KV"):
        xi = to_np(kv[i])
        rows, oc, os_, ost = _check_sampled(xi, codes[i], scales[i], inputs.KV_STATIC_AMAX, name)
        assert ost == 2.0 ** -6
        assert_bits_equal(to_np(deq[i])[rows], oracle.dequantize(oc, os_, ost, out="bf16"),
                          name + " dequantized bf16")


def test_kv_cache_dynamic_scale_full_size():
    import torch

    nvq = _nvq()
    kv = inputs.kv_cache(device="cuda")
    codes, scales, st, _, _ = nvq.nvfp4_quantize(kv)
    torch.cuda.synchronize()
    for i, name in enumerate("KV"):
        xi = to_np(kv[i])
        amax = float(np.abs(inputs.bf16_bits_to_f32(xi)).max())
        assert float(to_np(st)[i]) == oracle.tensor_scale(np.float32(amax)), name
        _check_sampled(xi, codes[i], scales[i], amax, name + " dynamic")


def test_kv_append_uses_the_cache_scale():
    import torch

    nvq = _nvq()
    new = inputs.kv_append()
    amax = torch.full((2,), inputs.KV_STATIC_AMAX, dtype=torch.float32, device="cuda")
    codes, scales, st, _, _ = nvq.nvfp4_quantize(to_gpu(new), amax_in=amax)
    deq = nvq.nvfp4_dequantize(codes, scales, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    sat = 0
    for i in range(2):
        oc, os_, ost = oracle.quantize(new[i], amax_in=inputs.KV_STATIC_AMAX)
        assert_bits_equal(to_np(codes[i]), oc, f"append {i} codes")
        assert_bits_equal(to_np(scales[i]), os_, f"append {i} scales")
        assert_bits_equal(to_np(deq[i]), oracle.dequantize(oc, os_, ost), f"append {i} deq")
        sat += int((os_ == 0x7E).sum())
    assert sat > 0  # values beyond the static amax saturate the block scale


@pytest.mark.parametrize("B,Hkv,S,D", [(3, 2, 37, 64), (1, 1, 1, 16), (2, 4, 129, 256)])
def test_small_ragged_caches_whole(B, Hkv, S, D):
    import torch

    nvq = _nvq()
    kv = inputs.kv_cache(B=B, Hkv=Hkv, S=S, D=D, wid=60 + D)
    for amax_in in (None, inputs.KV_STATIC_AMAX):
        a = None if amax_in is None else torch.full((2,), amax_in, device="cuda")
        codes, scales, st, _, _ = nvq.nvfp4_quantize(to_gpu(kv), amax_in=a)
        deq = nvq.nvfp4_dequantize(codes, scales, st, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        for i in range(2):
            oc, os_, ost = oracle.quantize(kv[i], amax_in=amax_in)
            assert float(to_np(st)[i]) == ost
            assert_bits_equal(to_np(codes[i]), oc, f"{B}x{Hkv}x{S}x{D} item {i} codes")
            assert_bits_equal(to_np(scales[i]), os_, f"{B}x{Hkv}x{S}x{D} item {i} scales")
            assert_bits_equal(to_np(deq[i]), oracle.dequantize(oc, os_, ost, out="bf16"),
                              f"{B}x{Hkv}x{S}x{D} item {i} deq")

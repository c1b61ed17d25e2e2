"""GPU parity of rollout-guided rounding (nvfp4_guidance_record,
nvfp4_guided_quantize; TRACE post, "L'idée centrale de TRACE" and
"Fonctionnement, côté ingénierie") against the oracle: bit-exact record bits
and rebuilt codes, on hand-worked cases, ragged and extreme tensors, stacked
expert weights, and the trainer layer's full-size weights."""
import numpy as np
import pytest

import oracle
from helpers import assert_bits_equal, log, to_gpu, to_np
from qat_nvfp4_quantize_amd import inputs

pytestmark = pytest.mark.gpu

MODES = (0, 1)  # mantissa, direction


def _nvq():
    from qat_nvfp4_quantize_amd import nvq

    return nvq


def _f32(x):
    return inputs.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def _check(x, w, what, modes=MODES):
    """Rollout side quantizes x and records; trainer side rebuilds codes for w.
    GPU and oracle each run the whole chain on the same seeded inputs."""
    import torch

    nvq = _nvq()
    log(f"[guided] {what} shape={x.shape} dtype={x.dtype}")
    xg, wg = to_gpu(x), to_gpu(w)
    codes, scales, st, _, _ = nvq.nvfp4_quantize(xg)
    oc, os_, ost = oracle.quantize(x)
    torch.cuda.synchronize()
    assert_bits_equal(to_np(codes), oc, what + " rollout codes")
    assert_bits_equal(to_np(scales), os_, what + " rollout scales")
    ws = nvq.workspace(256, "cuda")
    for m in modes:
        bits = nvq.nvfp4_guidance_record(codes, m, x=xg, scales=scales, tensor_scale=st)
        got = nvq.nvfp4_guided_quantize(wg, bits, scales, st, m, ws=ws)
        same = nvq.nvfp4_guided_quantize(xg, bits, scales, st, m)
        torch.cuda.synchronize()
        obits = oracle.guidance_record(oc, os_, ost, m, x)
        assert_bits_equal(to_np(bits), obits, f"{what} bits mode {m}")
        assert_bits_equal(to_np(got), oracle.guided_quantize(w, obits, os_, ost, m),
                          f"{what} guided codes mode {m}")
        assert_bits_equal(to_np(same), oc, f"{what} no-drift codes mode {m}")
        assert nvq.device_status(ws) == 0


def _golden():
    from conftest import read_golden

    rows = [[v.strip() for v in line.split("|")] for line in read_golden("guided_rounding.txt")]
    x = np.zeros((len(rows), 32), np.float32)
    x[:, 0] = 2688.0
    x[:, 16] = [float(r[1]) for r in rows]
    w = x.copy()
    x[:, 17] = [float(r[2]) for r in rows]
    w[:, 17] = [float(r[3]) for r in rows]
    return rows, x, w


def test_hand_worked_cases():
    import torch

    nvq = _nvq()
    rows, x, w = _golden()
    _check(x, w, "golden")
    codes, scales, st, _, _ = nvq.nvfp4_quantize(to_gpu(x))
    for m, col in zip(MODES, (8, 9)):
        bits = nvq.nvfp4_guidance_record(codes, m, x=to_gpu(x), scales=scales, tensor_scale=st)
        got = to_np(nvq.nvfp4_guided_quantize(to_gpu(w), bits, scales, st, m))
        torch.cuda.synchronize()
        nib = (got[:, 8] >> 4) & 0xF  # element 17 is the high nibble of byte 8
        assert nib.tolist() == [int(r[col], 16) for r in rows], m


def _tensor(seed, rows, K, dtype="f32", st_scale=1.0):
    g = np.random.default_rng(seed)
    x = g.standard_t(3, (rows, K)) * np.exp(g.uniform(-3, 3, (rows, 1))) * st_scale
    x = x.astype(np.float32)
    x[g.random((rows, K)) < 0.03] = 0.0
    x[g.random((rows, K)) < 0.01] = -0.0
    return inputs.to_bf16_bits(x) if dtype == "bf16" else x


def _drift(x, seed, rel=0.3):
    g = np.random.default_rng(seed + 1000)
    xf = _f32(x).astype(np.float64)
    w = (xf + g.standard_normal(xf.shape) * (rel * np.abs(xf) + 1e-3 * np.abs(xf).max()))
    w = w.astype(np.float32)
    return inputs.to_bf16_bits(w) if x.dtype == np.uint16 else w


@pytest.mark.parametrize("rows,K", [(1, 16), (17, 48), (129, 784), (300, 2064)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_shapes_under_drift(rows, K, dtype):
    x = _tensor(rows * 31 + K, rows, K, dtype)
    _check(x, _drift(x, rows + K), f"ragged {rows}x{K} {dtype}")


@pytest.mark.parametrize("st_scale", [3e-37, 1e-20, 1e30])
def test_extreme_tensor_scales(st_scale):
    x = _tensor(5, 64, 256, "f32", st_scale)
    _check(x, _drift(x, 5), f"extreme s_t x{st_scale:g}")


def test_subnormal_scales_and_grid_point_drift():
    g = np.random.default_rng(9)
    x = g.standard_normal((64, 128)).astype(np.float32)
    x[:, 0] = np.float32(2688.0 * 8)  # s_t = 8
    x[:, 16:] *= np.float32(2.0 ** -6) * g.uniform(0.05, 4, (64, 1)).astype(np.float32)
    oc, os_, ost = oracle.quantize(x)
    assert ost == 8.0
    # drifted values exactly on the scaled grid of each block (the on-grid corner)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    s_b = np.array([oracle.e4m3_value(int(c)) for c in os_.ravel()]).reshape(os_.shape)
    w = (grid[g.integers(0, 8, x.shape)] * np.repeat(s_b, 16, axis=1) * ost).astype(np.float32)
    w *= np.where(g.random(x.shape) < 0.5, -1, 1).astype(np.float32)
    _check(x, w, "subnormal scales, grid-point drift")


def test_arbitrary_record_and_zero_scales():
    import torch

    nvq = _nvq()
    g = np.random.default_rng(13)
    rows, K = 96, 512
    w = (g.standard_normal((rows, K)) * np.exp(g.uniform(-5, 5, (rows, 1)))).astype(np.float32)
    bits = g.integers(0, 256, (rows, K // 8)).astype(np.uint8)
    scales = g.integers(0, 0x7F, (rows, K // 16)).astype(np.uint8)
    scales[:, ::5] = 0
    for st in (0.0234375, 0.0, 1.1754944e-38):
        for m in MODES:
            got = nvq.nvfp4_guided_quantize(to_gpu(w), to_gpu(bits), to_gpu(scales),
                                            torch.tensor([st], device="cuda"), m)
            assert_bits_equal(to_np(got), oracle.guided_quantize(w, bits, scales, st, m),
                              f"arbitrary record s_t={st} mode {m}")


def test_stacked_expert_weights_use_their_own_scales():
    import torch

    nvq = _nvq()
    s = inputs.small_moe()
    w = inputs.weights(s, "dn", [0, 1, 2])                       # [3, N, K] bf16 bits
    w[1] = inputs.to_bf16_bits(inputs.bf16_bits_to_f32(w[1]) * np.float32(37.0))
    wd = np.stack([inputs.drifted_expert_weight(s, "dn", e) for e in (0, 1, 2)])
    wd[1] = inputs.to_bf16_bits(inputs.bf16_bits_to_f32(wd[1]) * np.float32(37.0))
    codes, scales, st, _, _ = nvq.nvfp4_quantize(to_gpu(w))
    for m in MODES:
        bits = nvq.nvfp4_guidance_record(codes, m, x=to_gpu(w), scales=scales, tensor_scale=st)
        got = to_np(nvq.nvfp4_guided_quantize(to_gpu(wd), bits, scales, st, m))
        torch.cuda.synchronize()
        for e in range(3):
            oc, os_, ost = oracle.quantize(w[e])
            assert float(to_np(st)[e]) == ost
            ob = oracle.guidance_record(oc, os_, ost, m, w[e])
            assert_bits_equal(to_np(bits)[e], ob, f"expert {e} bits mode {m}")
            assert_bits_equal(got[e], oracle.guided_quantize(wd[e], ob, os_, ost, m),
                              f"expert {e} codes mode {m}")


def test_mantissa_record_needs_only_codes():
    nvq = _nvq()
    x = _tensor(21, 40, 96)
    codes, scales, st, _, _ = nvq.nvfp4_quantize(to_gpu(x))
    bits = nvq.nvfp4_guidance_record(codes, 0)
    oc, os_, ost = oracle.quantize(x)
    ob = oracle.guidance_record(oc, os_, ost, 0)
    assert_bits_equal(to_np(bits), ob, "mantissa bits")
    # a bits buffer that is only 2-byte aligned takes the one-block-per-thread kernel
    import torch

    buf = torch.zeros(bits.numel() + 2, dtype=torch.uint8, device="cuda")
    view = buf[2:].view(bits.shape)
    nvq.nvfp4_guidance_record(codes, 0, out=view)
    assert_bits_equal(to_np(view), ob, "mantissa bits, 2-byte aligned output")


def test_nonfinite_master_sets_status_and_empty_inputs():
    import torch

    nvq = _nvq()
    x = _tensor(3, 8, 64)
    codes, scales, st, _, _ = nvq.nvfp4_quantize(to_gpu(x))
    bits = nvq.nvfp4_guidance_record(codes, 0)
    w = x.copy()
    w[3, 7] = np.nan
    ws = nvq.workspace(256, "cuda")
    nvq.nvfp4_guided_quantize(to_gpu(w), bits, scales, st, 0, ws=ws)
    assert nvq.device_status(ws) & nvq.NVQ_STATUS_NONFINITE
    nvq.nvfp4_guided_quantize(to_gpu(x), bits, scales, st, 0, ws=ws)
    assert nvq.device_status(ws) == 0  # the status word is cleared per call
    e = torch.empty(0, 64, dtype=torch.float32, device="cuda")
    out = nvq.nvfp4_guided_quantize(e, torch.empty(0, 8, dtype=torch.uint8, device="cuda"),
                                    torch.empty(0, 4, dtype=torch.uint8, device="cuda"), st, 1)
    assert out.shape == (0, 32)
    b = nvq.nvfp4_guidance_record(torch.empty(0, 32, dtype=torch.uint8, device="cuda"), 0)
    assert b.shape == (0, 8)


def test_qat_layer_weights_full_size():
    """The trainer layer's gate/up and down weights at full size, drawn on the
    GPU: no drift gives back the rollout codes on every element; drifted
    masters match the oracle on sampled experts."""
    import torch

    nvq = _nvq()
    s = inputs.QAT
    for proj in ("gu", "dn"):
        w = inputs.weights_device(s, proj)
        wd = inputs.drift_device(w, s, proj)
        log(f"[guided] full {proj} {tuple(w.shape)}")
        codes, scales, st, _, _ = nvq.nvfp4_quantize(w)
        for m in MODES:
            bits = nvq.nvfp4_guidance_record(codes, m, x=w, scales=scales, tensor_scale=st)
            same = nvq.nvfp4_guided_quantize(w, bits, scales, st, m)
            got = nvq.nvfp4_guided_quantize(wd, bits, scales, st, m)
            assert torch.equal(same, codes), (proj, m)
            changed = int((got != codes).sum())
            assert changed > 0
            for e in (0, 77, s.E - 1):
                # the oracle quantizes and records the whole expert itself
                we, wde = to_np(w[e]), to_np(wd[e])
                oc, os_, ost = oracle.quantize(we)
                assert_bits_equal(to_np(codes[e]), oc, f"{proj} e{e} rollout codes")
                assert float(to_np(st)[e]) == ost
                ob = oracle.guidance_record(oc, os_, ost, m, we)
                assert_bits_equal(to_np(bits[e]), ob, f"{proj} e{e} bits mode {m}")
                assert_bits_equal(to_np(got[e]), oracle.guided_quantize(wde, ob, os_, ost, m),
                                  f"{proj} e{e} guided mode {m}")
            del bits, same, got
        del w, wd, codes, scales
        torch.cuda.empty_cache()

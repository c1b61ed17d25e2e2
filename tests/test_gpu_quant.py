"""GPU parity of the NVFP4 quantizer path (nvfp4_quantize, nvfp4_dequantize,
residual_topk_channels) against the oracle: bit-exact codes, scales, tensor
scales, residual scores, top-k indices and compensation residuals."""
import numpy as np
import pytest

import oracle
from helpers import assert_bits_equal, log, to_gpu, to_np
from qat_nvfp4_quantize_amd import inputs

pytestmark = pytest.mark.gpu


def _nvq():
    from qat_nvfp4_quantize_amd import nvq

    return nvq


def _check_quant(x, k=None, amax_in=None, what=""):
    """Quantize x (numpy f32 or bf16 bits) on the GPU and compare with the oracle."""
    import torch

    nvq = _nvq()
    log(f"[quant] {what} shape={x.shape} dtype={x.dtype} k={k} amax_in={amax_in}")
    xg = to_gpu(x)
    amax_g = None if amax_in is None else torch.tensor([amax_in], dtype=torch.float32, device="cuda")
    codes, scales, st, score, ws = nvq.nvfp4_quantize(xg, amax_in=amax_g, score=True)
    torch.cuda.synchronize()
    oc, os_, ost = oracle.quantize(x, amax_in=amax_in)
    assert_bits_equal(to_np(st), np.array([ost], np.float32), what + " s_t")
    assert_bits_equal(to_np(scales), os_, what + " scales")
    assert_bits_equal(to_np(codes), oc, what + " codes")
    osc = oracle.residual_scores(x, oc, os_, ost)
    assert_bits_equal(to_np(score), osc, what + " scores")
    assert nvq.device_status(ws) == 0
    if k is not None:
        idx, resid, sc2 = nvq.residual_topk_channels(xg, codes, scales, st, k, scores=score,
                                                     want_scores=True)
        oidx = oracle.topk(osc, k)
        assert_bits_equal(to_np(idx), oidx, what + " topk")
        assert_bits_equal(to_np(resid), oracle.residual_columns_bf16(x, oc, os_, ost, oidx),
                          what + " resid")
        # recomputing the score from the record gives the same bits
        idx2, _, sc3 = nvq.residual_topk_channels(xg, codes, scales, st, k, want_scores=True,
                                                  want_resid=False)
        assert_bits_equal(to_np(sc3), osc, what + " scores (recomputed)")
        assert_bits_equal(to_np(idx2), oidx, what + " topk (recomputed)")
    return codes, scales, st


def test_dense_check_workload_activation_and_weight():
    x, w, k = inputs.dense_check()
    _check_quant(x, k=k, what="dense X")
    _check_quant(w, k=k, what="dense W^T")


def test_quant_sweep_full_size_bit_exact():
    x = inputs.quant_sweep()
    _check_quant(x, k=64, what="sweep 8192x7168 bf16")


@pytest.mark.parametrize("rows,K", [(1, 16), (15, 48), (17, 784), (300, 2064), (129, 1024)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_shapes(rows, K, dtype):
    g = np.random.default_rng(rows * 7 + K)
    x = (g.standard_t(3, (rows, K)) * np.exp(g.uniform(-4, 4, (rows, 1)))).astype(np.float32)
    x[g.random((rows, K)) < 0.05] = 0.0
    x[g.random((rows, K)) < 0.02] = -0.0
    if dtype == "bf16":
        x = inputs.to_bf16_bits(x)
    _check_quant(x, k=min(5, K), what=f"ragged {rows}x{K} {dtype}")


def test_golden_blocks_and_near_ties():
    from test_oracle_quant import _golden_blocks, _near_tie_tensor

    blocks = _golden_blocks()
    x = np.array([v for b in blocks for v in b[1]], np.float32).reshape(1, -1)
    codes, scales, st = _check_quant(x, what="golden")
    for i, (name, vals, sc, packed, rsum) in enumerate(blocks):
        assert to_np(scales)[0, i] == sc, name
        assert bytes(to_np(codes)[0, 8 * i:8 * i + 8]) == packed, name
    for seed in range(3):
        _check_quant(_near_tie_tensor(seed), k=8, what=f"near-ties {seed}")
    _check_quant(inputs.to_bf16_bits(_near_tie_tensor(9)), what="near-ties bf16")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_scale_midpoints_under_full_mantissa_tensor_scale(seed):
    """Block maxima on and one ulp around E4M3 midpoints (times 6 s_t) and
    elements near E2M1 midpoints, with a tensor scale that has a full mantissa
    (the fma decisions of the fast path), in fp32 and bf16."""
    from test_oracle_quant import _scale_tie_tensor

    for amax in (1.2345678e3, 3.0e-3, 7.77e-20):
        x = _scale_tie_tensor(seed, amax)
        _check_quant(x, k=8, what=f"scale ties {seed} {amax}")
        _check_quant(inputs.to_bf16_bits(x), what=f"scale ties bf16 {seed} {amax}")


def test_extreme_tensor_scales_and_denormals():
    g = np.random.default_rng(11)
    base = g.standard_normal((64, 128)).astype(np.float32)
    for scale in (1e-38, 1e-30, 1e-12, 1e12, 1e30, 1e37):
        _check_quant((base * np.float32(scale)).astype(np.float32), what=f"scale {scale}")
    den = (g.standard_normal((16, 64)) * 1e-40).astype(np.float32)  # fp32 subnormals
    _check_quant(den, what="subnormal inputs")
    den[0, 0] = 1.0
    _check_quant(den, what="subnormal with a normal amax")


def test_all_zero_and_negative_zero():
    x = np.zeros((20, 32), np.float32)
    x[3] = -0.0
    _check_quant(x, k=4, what="zeros")


def test_amax_override_saturates():
    g = np.random.default_rng(12)
    x = (g.standard_normal((40, 64)) * 10).astype(np.float32)
    _check_quant(x, amax_in=float(np.abs(x).max()) / 7, what="amax_in small")
    _check_quant(x, amax_in=float(np.abs(x).max()) * 3, what="amax_in large")


def test_batched_weights_have_per_item_scales():
    import torch

    nvq = _nvq()
    s = inputs.small_moe()
    w = inputs.weights(s, "gu")  # [E, 2I, H] bf16 bits
    codes, scales, st, _, ws = nvq.nvfp4_quantize(to_gpu(w))
    torch.cuda.synchronize()
    for e in range(s.E):
        oc, os_, ost = oracle.quantize(w[e])
        assert_bits_equal(to_np(st)[e:e + 1], np.array([ost], np.float32), f"w s_t {e}")
        assert_bits_equal(to_np(scales)[e], os_, f"w scales {e}")
        assert_bits_equal(to_np(codes)[e], oc, f"w codes {e}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bit_exact(out):
    import torch

    nvq = _nvq()
    x = inputs.to_bf16_bits((np.random.default_rng(13).standard_t(3, (96, 512)) * 3).astype(np.float32))
    codes, scales, st, _, _ = nvq.nvfp4_quantize(to_gpu(x))
    y = nvq.nvfp4_dequantize(codes, scales, st, torch.float32 if out == "f32" else torch.bfloat16)
    oc, os_, ost = oracle.quantize(x)
    assert_bits_equal(to_np(y), oracle.dequantize(oc, os_, ost, out=out), "dequant " + out)


def test_nonfinite_input_sets_status():
    nvq = _nvq()
    x = np.ones((4, 32), np.float32)
    x[2, 5] = np.inf
    _, _, _, _, ws = nvq.nvfp4_quantize(to_gpu(x))
    assert nvq.device_status(ws) & nvq.NVQ_STATUS_NONFINITE


def test_repeat_runs_are_bitwise_identical():
    nvq = _nvq()
    x = to_gpu(inputs.quant_sweep(M=1024, K=2048))
    a = [to_np(t) for t in nvq.nvfp4_quantize(x, score=True)[:4]]
    b = [to_np(t) for t in nvq.nvfp4_quantize(x, score=True)[:4]]
    for u, v in zip(a, b):
        assert_bits_equal(u, v, "repeat")


@pytest.mark.parametrize("K,k", [(16, 1), (48, 3), (64, 64), (1008, 17), (7168, 64), (7168, 1024),
                                 (7168, 1025), (4096, 4096), (20000, 128), (100000, 1000)])
def test_topk_on_given_scores_ties_and_sizes(K, k):
    """residual_topk_channels on caller scores: heavy exact ties, negative
    values and both zeros (ties break to the lower index; -0 equals +0).
    k <= 1024 runs the radix select, larger k the bitonic sort."""
    import torch

    nvq = _nvq()
    g = np.random.default_rng(K * 7 + k)
    sc = g.integers(-3, 12, K).astype(np.float32) * np.float32(0.25)
    sc[g.random(K) < 0.1] = np.float32(-0.0)
    sc[g.random(K) < 0.05] = g.standard_normal(int((g.random(K) < 0.05).sum()) or 1)[0]
    sc[g.random(K) < 0.01] = np.float32(3.0e38)
    log(f"[topk] K={K} k={k}")
    x = torch.empty(0, K, dtype=torch.float32, device="cuda")
    idx, _, _ = nvq.residual_topk_channels(x, None, None, None, k, scores=to_gpu(sc),
                                           want_resid=False)
    torch.cuda.synchronize()
    assert_bits_equal(to_np(idx), oracle.topk(sc, k), f"topk K={K} k={k}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_no_rows(dtype):
    """Zero rows: no codes, s_t = fl32(amax / 2688) with the amax of nothing 0
    (or the given amax), every channel score the empty sum 0 -- as the oracle."""
    import torch

    nvq = _nvq()
    K = 64
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = torch.empty(0, K, dtype=tdt, device="cuda")
    for amax in (None, 3.5):
        amax_t = None if amax is None else torch.tensor([amax], dtype=torch.float32, device="cuda")
        codes, scales, st, score, _ = nvq.nvfp4_quantize(x, amax_in=amax_t, score=True)
        torch.cuda.synchronize()
        oc, osc, ost = oracle.quantize(np.zeros((0, K), np.float32), amax_in=amax)
        assert codes.shape == (0, K // 2) and scales.shape == (0, K // 16)
        assert_bits_equal(to_np(st), np.array([ost], np.float32), f"s_t of no rows (amax {amax})")
        assert_bits_equal(to_np(score), oracle.residual_scores(np.zeros((0, K), np.float32), oc, osc, ost),
                          "scores of no rows")


@pytest.mark.parametrize("rows,K,ldx,dtype", [(300, 272, 336, "bf16"), (129, 1040, 1044, "f32"),
                                              (17, 16, 32, "bf16"), (1, 48, 64, "f32")])
def test_row_strided_input(rows, K, ldx, dtype):
    """x given as the first K columns of a wider [rows, ldx] tensor (row stride
    ldx): the same record, scores, channels and residuals as the oracle on
    those columns; the padding columns (filled with huge values) are never
    read.  Also without a score (the strided score-free path) and stacked
    [3, rows, K] items with their own tensor scales."""
    import torch

    nvq = _nvq()
    g = np.random.default_rng(rows + K + ldx)
    wide = (g.standard_t(4, (rows, ldx)) * np.exp(g.uniform(-3, 3, (1, ldx)))).astype(np.float32)
    wide[:, K:] = np.float32(3e38)  # never part of the tensor
    if dtype == "bf16":
        wide = inputs.to_bf16_bits(wide)
    log(f"[quant] strided {rows}x{K} ldx={ldx} {dtype}")
    xg = to_gpu(wide)[:, :K]
    assert xg.stride(0) == ldx and not xg.is_contiguous() or rows == 1
    codes, scales, st, score, ws = nvq.nvfp4_quantize(xg, score=True)
    k = min(7, K)
    idx, resid, sc2 = nvq.residual_topk_channels(xg, codes, scales, st, k, want_scores=True)
    c2, s2, st2, _, _ = nvq.nvfp4_quantize(xg)  # score-free
    torch.cuda.synchronize()
    oc, os_, ost = oracle.quantize(wide, K=K)
    assert_bits_equal(to_np(st), np.array([ost], np.float32), "strided s_t")
    assert_bits_equal(to_np(codes), oc, "strided codes")
    assert_bits_equal(to_np(scales), os_, "strided scales")
    assert_bits_equal(to_np(c2), oc, "strided codes (no score)")
    assert_bits_equal(to_np(s2), os_, "strided scales (no score)")
    assert_bits_equal(to_np(st2), np.array([ost], np.float32), "strided s_t (no score)")
    osc = oracle.residual_scores(wide, oc, os_, ost, K=K)
    assert_bits_equal(to_np(score), osc, "strided scores")
    assert_bits_equal(to_np(sc2), osc, "strided scores (recomputed)")
    oidx = oracle.topk(osc, k)
    assert_bits_equal(to_np(idx), oidx, "strided topk")
    assert_bits_equal(to_np(resid), oracle.residual_columns_bf16(wide, oc, os_, ost, oidx, K=K),
                      "strided resid")
    assert nvq.device_status(ws) == 0
    # stacked items, each [rows, K] inside [rows, ldx]
    items = np.stack([wide, wide[::-1].copy(), (wide.view(np.uint16) ^ 0x8000).view(wide.dtype)
                      if dtype == "bf16" else -wide])
    xb = to_gpu(items)[:, :, :K]
    cb, sb, stb, _, _ = nvq.nvfp4_quantize(xb)
    torch.cuda.synchronize()
    for b in range(3):
        oc, os_, ost = oracle.quantize(items[b], K=K)
        assert_bits_equal(to_np(stb)[b:b + 1], np.array([ost], np.float32), f"item {b} s_t")
        assert_bits_equal(to_np(cb)[b], oc, f"item {b} codes")
        assert_bits_equal(to_np(sb)[b], os_, f"item {b} scales")


@pytest.mark.parametrize("case", ["bf16", "f32_tiny_scale", "bf16_strided"])
def test_row_tile_edges(case):
    """The row-tile kernel on ragged edges.  Scored calls on tensors with few
    rows run the thread-per-block tile, so the small cases above exercise
    that one; 80017 rows x 48 columns gives the row tile 626 workgroups (more
    than two per CU), with a partial last chunk and 3 of 64 lanes active per
    row.  Also the fp64 path of extreme tensor scales and a row stride."""
    import torch

    nvq = _nvq()
    rows, K = 80017, 48
    g = np.random.default_rng({"bf16": 1, "f32_tiny_scale": 2, "bf16_strided": 3}[case])
    x = (g.standard_t(3, (rows, K)) * np.exp(g.uniform(-4, 4, (rows, 1)))).astype(np.float32)
    x[g.random((rows, K)) < 0.03] = 0.0
    if case == "f32_tiny_scale":
        x = (x * np.float32(1e-38)).astype(np.float32)  # tensor scale below 2^-100: the fp64 path
        _check_quant(x, k=5, what="row tile f32 tiny scale")
        return
    if case == "bf16":
        _check_quant(inputs.to_bf16_bits(x), k=5, what="row tile bf16")
        return
    ldx = 64
    wide = np.full((rows, ldx), 3e38, np.float32)
    wide[:, :K] = x
    wide = inputs.to_bf16_bits(wide)
    log(f"[quant] row tile strided {rows}x{K} ldx={ldx}")
    xg = to_gpu(wide)[:, :K]
    codes, scales, st, score, ws = nvq.nvfp4_quantize(xg, score=True)
    torch.cuda.synchronize()
    oc, os_, ost = oracle.quantize(wide, K=K)
    assert_bits_equal(to_np(st), np.array([ost], np.float32), "row tile strided s_t")
    assert_bits_equal(to_np(codes), oc, "row tile strided codes")
    assert_bits_equal(to_np(scales), os_, "row tile strided scales")
    assert_bits_equal(to_np(score), oracle.residual_scores(wide, oc, os_, ost, K=K), "row tile strided scores")
    assert nvq.device_status(ws) == 0


@pytest.mark.parametrize("case", ["ragged", "strided", "partial_grid", "tiny_scale", "nonfinite"])
def test_sweep_size_ragged_edges(case):
    """Scored bf16 tensors of about the sweep's size with ragged edges:
    8100 x 7008 has a partial last chunk (36 rows) and a partial last group of
    block columns; 6200 x 7168 leaves part of the chip idle in the last wave of
    workgroups; a row stride; a tensor scale below 2^-100 (fp64 decisions);
    and an infinite element (status)."""
    import torch

    nvq = _nvq()
    rows, K, ldx = {"ragged": (8100, 7008, None), "strided": (8192, 7168, 7200),
                    "partial_grid": (6200, 7168, None), "tiny_scale": (8192, 7168, None),
                    "nonfinite": (8192, 7168, None)}[case]
    g = np.random.default_rng({"ragged": 11, "strided": 12, "partial_grid": 13, "tiny_scale": 14,
                               "nonfinite": 15}[case])
    x = g.standard_t(4, (rows, K)).astype(np.float32)
    x[:, g.random(K) < 0.005] *= 50.0
    if case == "tiny_scale":
        x = (x * np.float32(1e-31)).astype(np.float32)
    if case == "nonfinite":
        x[4097, 3001] = np.inf
        _, _, _, _, ws = nvq.nvfp4_quantize(to_gpu(inputs.to_bf16_bits(x)), score=True)
        assert nvq.device_status(ws) & nvq.NVQ_STATUS_NONFINITE
        return
    if ldx is None:
        _check_quant(inputs.to_bf16_bits(x), what=f"sweep-size {case}")
        return
    wide = np.full((rows, ldx), 3e38, np.float32)
    wide[:, :K] = x
    wide = inputs.to_bf16_bits(wide)
    log(f"[quant] sweep-size strided {rows}x{K} ldx={ldx}")
    codes, scales, st, score, ws = nvq.nvfp4_quantize(to_gpu(wide)[:, :K], score=True)
    torch.cuda.synchronize()
    oc, os_, ost = oracle.quantize(wide, K=K)
    assert_bits_equal(to_np(st), np.array([ost], np.float32), "sweep-size strided s_t")
    assert_bits_equal(to_np(codes), oc, "sweep-size strided codes")
    assert_bits_equal(to_np(scales), os_, "sweep-size strided scales")
    assert_bits_equal(to_np(score), oracle.residual_scores(wide, oc, os_, ost, K=K), "sweep-size strided scores")
    assert nvq.device_status(ws) == 0

"""Pins of the oracle's residual scores, top-k, routing, permutation, GEMMs,
SwiGLU, combine and QAT GEMMs against library routines (numpy/scipy/torch),
exact rational arithmetic and closed-form identities -- never against a retyped
copy of the oracle's own formula."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from qat_nvfp4_quantize_amd import inputs


def _x(seed, rows, K):
    g = np.random.default_rng(seed)
    x = (g.standard_t(4, (rows, K)) * g.uniform(0.5, 2, (1, K))).astype(np.float32)
    return x


def test_residual_scores_follow_chunked_sequential_fp32_order():
    # 300 rows: chunks of 128, 128 and a ragged 44 (sub-chunks of 16, last one 12 rows).
    x = _x(0, 300, 64)
    codes, scales, st = oracle.quantize(x)
    v = oracle.dequantize(codes, scales, st)
    r = np.abs(x - v)  # numpy float32 subtraction, IEEE

    def seq(a):  # sequential fp32 sum over axis 0 (cumsum accumulates in order)
        return np.cumsum(a, axis=0, dtype=np.float32)[-1]

    parts = []
    for m0 in range(0, 300, 128):
        subs = [seq(r[s0:min(300, s0 + 16)]) for s0 in range(m0, min(300, m0 + 128), 16)]
        parts.append(seq(np.stack(subs)))
    ref = seq(np.stack(parts))
    got = oracle.residual_scores(x, codes, scales, st)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # bf16 input path gives the same as its fp32 image
    xb = inputs.to_bf16_bits(x)
    cb, sb, stb = oracle.quantize(xb)
    gb = oracle.residual_scores(xb, cb, sb, stb)
    xf = inputs.bf16_bits_to_f32(xb)
    assert np.array_equal(gb, oracle.residual_scores(xf, *oracle.quantize(xf)))


def test_residual_scores_chunk128_order_pinned_by_cumsum():
    # the plainer order: one sequential fp32 sum per 128-row chunk, chunks in order
    x = _x(3, 300, 64)
    codes, scales, st = oracle.quantize(x)
    r = np.abs(x - oracle.dequantize(codes, scales, st))

    def seq(a):
        return np.cumsum(a, axis=0, dtype=np.float32)[-1]

    ref = seq(np.stack([seq(r[m0:m0 + 128]) for m0 in range(0, 300, 128)]))
    got = oracle.residual_scores(x, codes, scales, st, order="chunk128")
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("workload", ["dense", "sweep", "decode_x", "prefill_x"])
def test_score_order_choice_selects_the_same_channels(workload):
    """The pages fix no summation order for the residual score.  On the
    activations of every workload, the order the library computes (16-row
    sub-chunks inside 128-row chunks) and a plain sequential sum per 128-row
    chunk select the same top-k channels in the same rank order, and the two
    scores differ by no more than the fp32 summation bound."""
    if workload == "dense":
        x, _, k = inputs.dense_check()
    elif workload == "sweep":
        x, k = inputs.quant_sweep(), 64
    elif workload == "decode_x":
        x, k = inputs.activations(inputs.DECODE), inputs.DECODE.k
    else:
        x, k = inputs.activations(inputs.PREFILL), inputs.PREFILL.k
    codes, scales, st = oracle.quantize(x)
    a = oracle.residual_scores(x, codes, scales, st, order="sub16")
    b = oracle.residual_scores(x, codes, scales, st, order="chunk128")
    assert np.array_equal(oracle.topk(a, k), oracle.topk(b, k))
    # both are fp32 sums of the same M non-negative terms: each within
    # (M - 1) u of the exact sum (relative), u = 2^-24
    M = x.shape[0]
    rel = np.abs(a.astype(np.float64) - b) / np.maximum(b.astype(np.float64), 1e-300)
    assert rel.max() <= 2 * (M - 1) * 2.0 ** -24


def test_residual_scores_zero_on_grid_and_golden_outlier():
    x = np.zeros((3, 16), np.float32)
    x[0, 0] = 2688.0  # s_t = 1
    x[1, :] = [6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -2, -1.5, -1, -0.5, 0]
    x[2, :] = [100] + [0.125] * 15
    codes, scales, st = oracle.quantize(x)
    s = oracle.residual_scores(x, codes, scales, st)
    # only row 2 leaves residuals; its block scale is 16: 100 -> 96, 0.125 -> 0
    assert s[0] == 4.0 and np.all(s[1:] == np.float32(0.125))


def test_topk_matches_lexsort_with_ties():
    g = np.random.default_rng(1)
    s = g.integers(0, 20, 500).astype(np.float32)  # many exact ties
    for k in (0, 1, 7, 64, 500):
        ref = np.lexsort((np.arange(500), -s))[:k]
        assert np.array_equal(oracle.topk(s, k), ref)


def test_route_matches_stable_sort_and_softmax():
    g = np.random.default_rng(2)
    T, E, topk = 200, 32, 8
    logits = g.standard_normal((T, E)).astype(np.float32)
    logits[:20, :] = np.round(logits[:20, :])  # ties
    ids, w = oracle.route(logits, topk)
    ref_ids = np.stack([np.lexsort((np.arange(E), -row))[:topk] for row in logits])
    assert np.array_equal(ids, ref_ids)
    sel = np.take_along_axis(logits.astype(np.float64), ref_ids, 1)
    ref_w = scipy.special.softmax(sel, axis=1).astype(np.float32)
    np.testing.assert_allclose(w, ref_w, rtol=2 ** -23, atol=0)
    # equals the renormalised top-k of the full softmax
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    pick = np.take_along_axis(full, ref_ids, 1)
    np.testing.assert_allclose(w, pick / pick.sum(1, keepdims=True), rtol=1e-6)


def test_permute_matches_stable_argsort():
    g = np.random.default_rng(3)
    T, topk, E = 500, 4, 16
    ids = g.integers(0, E - 3, (T, topk)).astype(np.int32)  # last 3 experts empty
    sp, off, pos = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    ref = np.argsort(flat, kind="stable")
    assert np.array_equal(sp, ref)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(sp[pos], np.arange(T * topk))
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, E]], np.int32), E)


def _dequant_f64(codes, scales, st):
    """Exact real values G * s_b * s_t with numpy and torch's E4M3 decoding."""
    g = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    sb = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn)
    sb = np.repeat(sb.to(torch.float64).numpy(), 16, axis=1)
    v = g[nib & 7] * sb * float(st)
    return np.where(nib & 8, -v, v)


def _dense_case(seed=4):
    x, w, k = inputs.dense_check()
    qa = oracle.quantize(x)
    qw = oracle.quantize(w)
    s = oracle.topk(oracle.residual_scores(x, *qa), k)
    return x, w, k, qa, qw, s


def test_w4a4_gemm_matches_numpy_matmul_with_compensation():
    x, w, k, qa, qw, s = _dense_case()
    M, N = x.shape[0], w.shape[0]
    got = oracle.moe_gemm_w4a4(qa[0], qa[1], qa[2], x, s, qw[0], qw[1], qw[2],
                               np.arange(M), np.zeros(M))
    A = _dequant_f64(*qa)
    W = _dequant_f64(*qw)
    v = oracle.dequantize(*qa)
    rb = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(x - v)).astype(np.float64)
    ref = A @ W.T + rb[:, s] @ W[:, s].T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the compensation moves the W4A4 output toward the unquantized-activation product
    plain = oracle.moe_gemm_w4a4(qa[0], qa[1], qa[2], x, None, qw[0], qw[1], qw[2],
                                 np.arange(M), np.zeros(M))
    target = x.astype(np.float64) @ W.T
    assert np.abs(got - target).sum() < np.abs(plain - target).sum()


def test_compensation_limits_k0_and_kfull():
    x, w, _, qa, qw, _ = _dense_case()
    M, K = x.shape
    A = _dequant_f64(*qa)
    W = _dequant_f64(*qw)
    rows = np.arange(M)
    k0 = oracle.moe_gemm_w4a4(qa[0], qa[1], qa[2], x, np.zeros(0), qw[0], qw[1], qw[2], rows,
                              np.zeros(M))
    np.testing.assert_allclose(k0, A @ W.T, rtol=1e-12, atol=1e-12)
    allc = oracle.topk(oracle.residual_scores(x, *qa), K)
    kf = oracle.moe_gemm_w4a4(qa[0], qa[1], qa[2], x, allc, qw[0], qw[1], qw[2], rows,
                              np.zeros(M))
    # k = K: (A^ + bf16(r)) W^T, within 2^-9 |r| |w| of the W4A16 product x W^T
    trainer = x.astype(np.float64) @ W.T
    v = oracle.dequantize(*qa)
    rn = np.linalg.norm((x - v).astype(np.float64), axis=1)[:, None]
    wn = np.linalg.norm(W, axis=1)[None, :]
    assert np.all(np.abs(kf - trainer) <= 2.0 ** -9 * rn * wn + 1e-12)


def test_w4a4_gemm_exact_brute_force_4x16x16():
    # Power-of-two tensor scales make every product and 16-term sum exact in fp64.
    g = np.random.default_rng(5)
    a = (g.standard_normal((4, 16)) * 3).astype(np.float32)
    a[0, 0] = 2688.0 / 8  # amax -> s_t = 1/8
    w = (g.standard_normal((16, 16))).astype(np.float32)
    w[0, 0] = 2688.0 * 4  # s_t = 4
    qa, qw = oracle.quantize(a), oracle.quantize(w)
    assert qa[2] == 0.125 and qw[2] == 4.0
    s = np.array([3, 0, 9], np.int32)
    got = oracle.moe_gemm_w4a4(qa[0], qa[1], qa[2], a, s, qw[0], qw[1], qw[2], np.arange(4),
                               np.zeros(4))
    A = oracle.dequantize(*qa)  # exact in fp32 here
    W = oracle.dequantize(*qw)
    R = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(a - A))
    for i in range(4):
        for n in range(16):
            exact = sum(Fraction(float(A[i, c])) * Fraction(float(W[n, c])) for c in range(16))
            exact += sum(Fraction(float(R[i, c])) * Fraction(float(W[n, c])) for c in s)
            assert Fraction(got[i, n]) == exact


def test_moe_rows_pick_token_and_expert():
    g = np.random.default_rng(6)
    T, K, N, E = 10, 32, 8, 3
    x = g.standard_normal((T, K)).astype(np.float32)
    qa = oracle.quantize(x)
    ws = [oracle.quantize(g.standard_normal((N, K)).astype(np.float32)) for _ in range(E)]
    wc = np.stack([q[0] for q in ws])
    wsc = np.stack([q[1] for q in ws])
    wst = np.array([q[2] for q in ws], np.float32)
    rt = np.array([3, 3, 7, 0], np.int32)
    re = np.array([2, 0, 1, 2], np.int32)
    comp = np.array([5, 1], np.int32)
    got = oracle.moe_gemm_w4a4(qa[0], qa[1], qa[2], x, comp, wc, wsc, wst, rt, re,
                               cols=np.array([7, 0, 2]))
    for i, (t, e) in enumerate(zip(rt, re)):
        one = oracle.moe_gemm_w4a4(qa[0][t:t + 1], qa[1][t:t + 1], qa[2], x[t:t + 1], comp,
                                   wc[e], wsc[e], wst[e], [0], [0])
        np.testing.assert_array_equal(got[i], one[0, [7, 0, 2]])


# Every finite non-negative bf16 value, ascending (bit patterns 0x0000..0x7F7F).
_BF16_POS = (np.arange(0x7F80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_nearest(v: float) -> int:
    """bf16 bit pattern nearest the real number v (an fp64 value), ties to the
    even pattern, by exact rational comparison of the two bracketing bf16
    values; beyond the largest finite value, the IEEE overflow rule (at or
    above max + half an ulp -> infinity)."""
    a = abs(v)
    sign = 0x8000 if np.signbit(v) else 0
    big = Fraction(_BF16_POS[-1]) + Fraction(2) ** 119  # max + half ulp (ulp 2^120)
    if Fraction(a) >= big:
        return sign | 0x7F80
    i = int(np.searchsorted(_BF16_POS, a, side="right")) - 1  # _BF16_POS[i] <= a
    if i == len(_BF16_POS) - 1 or _BF16_POS[i] == a:
        return sign | i
    lo, hi = Fraction(_BF16_POS[i]), Fraction(_BF16_POS[i + 1])
    d_lo, d_hi = Fraction(a) - lo, hi - Fraction(a)
    pick = i if (d_lo < d_hi or (d_lo == d_hi and i % 2 == 0)) else i + 1
    return sign | pick


def test_double_to_bf16_rounds_once_to_nearest_even():
    # ties, a value a double rounding through fp32 would get wrong, subnormals,
    # the overflow threshold, signed zero, and random fp64 values
    cases = [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, 1.0 + 3 * 2 ** -8,
             -(1.0 + 2 ** -8 + 2 ** -40), 2 ** -133, 2 ** -134, 3 * 2 ** -134, 2 ** -135,
             2 ** -126 - 2 ** -134, 2 ** -126 - 2 ** -135, 3.3895313892515355e38,
             float(_BF16_POS[-1]) + 2 ** 119, float(_BF16_POS[-1]) + 2 ** 119 - 2 ** 80, 1e300,
             -1e-300, 1e-50]
    g = np.random.default_rng(17)
    cases += list(g.standard_normal(300) * np.exp2(g.integers(-140, 128, 300)))
    cases += list(np.float64(g.standard_normal(200).astype(np.float32)) * (1 + 2.0 ** -30))
    for v in cases:
        assert oracle.double_to_bf16(v) == _bf16_nearest(v), v
    # fp32 inputs agree with torch's fp32 -> bf16 rounding (one rounding either way)
    f = g.standard_normal(1000).astype(np.float32)
    tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert all(oracle.double_to_bf16(float(a)) == int(b) for a, b in zip(f, tb))


def test_swiglu_closed_form():
    y = np.array([[0.0, 1.0, -3.0, 2.0, 5.0, 0.5],
                  [40.0, -40.0, 1e-3, 7.0, 7.0, -2.0]])
    h = oracle.swiglu_bf16(y)
    import math
    for r in range(2):
        for i in range(3):
            gte, up = y[r, i], y[r, 3 + i]
            ref = gte * up / (1.0 + math.exp(-gte))
            assert h[r, i] == _bf16_nearest(ref)


def test_combine_matches_numpy():
    g = np.random.default_rng(7)
    T, topk, N, E = 50, 4, 24, 6
    ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    _, w = oracle.route(g.standard_normal((T, E)).astype(np.float32), topk)
    sp, off, pos = oracle.permute(ids, E)
    y = g.standard_normal((T * topk, N)).astype(np.float32)
    got = oracle.combine_bf16(y, pos, w)
    ref = np.einsum("tj,tjn->tn", w.astype(np.float64),
                    y.astype(np.float64)[pos.reshape(T, topk)])
    refb = np.array([_bf16_nearest(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    assert np.array_equal(got, refb)


def _qat_case(seed=8):
    g = np.random.default_rng(seed)
    T, K, N, E, topk = 40, 64, 48, 3, 2
    xb = inputs.to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    ws = [oracle.quantize(inputs.to_bf16_bits(0.02 * g.standard_normal((N, K)).astype(np.float32)))
          for _ in range(E)]
    wc = np.stack([q[0] for q in ws])
    wsc = np.stack([q[1] for q in ws])
    wst = np.array([q[2] for q in ws], np.float32)
    ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    sp, off, pos = oracle.permute(ids, E)
    a_row = sp // topk
    row_e = np.repeat(np.arange(E), np.diff(off)).astype(np.int32)
    dy = inputs.to_bf16_bits(g.standard_normal((T * topk, N)).astype(np.float32))
    return xb, wc, wsc, wst, off, a_row, row_e, dy


def test_qat_forward_equals_dense_gemm_on_dequantized_cache():
    xb, wc, wsc, wst, off, a_row, row_e, dy = _qat_case()
    y = oracle.qat_fwd(xb, a_row, row_e, wc, wsc, wst)
    X = inputs.bf16_bits_to_f32(xb).astype(np.float64)
    for e in range(len(wst)):
        W = _dequant_f64(wc[e], wsc[e], wst[e])
        rows = slice(off[e], off[e + 1])
        np.testing.assert_allclose(y[rows], X[a_row[rows]] @ W.T, rtol=1e-12, atol=1e-12)


def test_qat_adjoint_identities():
    xb, wc, wsc, wst, off, a_row, row_e, dy = _qat_case()
    N, K = wc.shape[1], wc.shape[2] * 2
    y = oracle.qat_fwd(xb, a_row, row_e, wc, wsc, wst)
    dx = oracle.qat_dgrad(dy, np.arange(len(a_row)), row_e, wc, wsc, wst)
    X = inputs.bf16_bits_to_f32(xb).astype(np.float64)[a_row]
    DY = inputs.bf16_bits_to_f32(dy).astype(np.float64)
    lhs = np.sum(DY * y)
    assert np.sum(dx * X) == pytest.approx(lhs, rel=1e-12)
    tot = 0.0
    nn, cc = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    for e in range(len(wst)):
        dw = oracle.qat_wgrad(dy, xb, a_row, off[e], off[e + 1], nn.ravel(), cc.ravel())
        W = _dequant_f64(wc[e], wsc[e], wst[e])
        tot += np.sum(dw.reshape(N, K) * W)
        rows = slice(off[e], off[e + 1])
        np.testing.assert_allclose(dw.reshape(N, K), DY[rows].T @ X[rows], rtol=1e-12, atol=1e-12)
    assert tot == pytest.approx(lhs, rel=1e-12)


def test_combine_leaves_out_dropped_pairs():
    """A pair the permutation dropped (pos < 0) contributes nothing: the result
    equals the combine over the remaining pairs, written out in numpy."""
    g = np.random.default_rng(21)
    T, topk, N = 5, 3, 16
    y = g.standard_normal((T * topk, N)).astype(np.float32)
    w = g.random((T, topk)).astype(np.float32)
    pos = np.arange(T * topk, dtype=np.int32)
    pos[[1, 7, 8]] = -1
    got = inputs.bf16_bits_to_f32(oracle.combine_bf16(y, pos, w))
    ref = np.zeros((T, N))
    for t in range(T):
        for j in range(topk):
            p = pos[t * topk + j]
            if p >= 0:
                ref[t] += np.float64(w[t, j]) * y[p].astype(np.float64)
    np.testing.assert_array_equal(got, inputs.bf16_bits_to_f32(inputs.to_bf16_bits(ref.astype(np.float32))))


def test_residual_columns_hand_worked_and_bf16_ties():
    """bf16 residual columns (QUADS explainer §2.2-B: the correction uses the
    activation's quantization residual on the selected channels). Hand-worked:
    with s_t = 1 and block scale 2, 9 + 2^-8 rounds to grid value 4 (value 8), so
    r = 1 + 2^-8, a bf16 tie that goes to the even 1.0; 9 + 3*2^-8 leaves
    1 + 3*2^-8, a tie that goes up to 1 + 2^-6; 7.2 rounds to 8 and leaves
    -0.8 (bf16 -0.80078125); 2.5 gives the quotient 1.25, a midpoint that
    goes to the even grid value 1.0 (value 2) and leaves 0.5."""
    x = np.zeros((2, 32), np.float32)
    x[0, 0] = 2688.0                       # tensor scale 1
    x[1, :16] = [12.0, 9.00390625, 9.01171875, 7.2, 2.5] + [0.0] * 11  # block max 12: s_b = 2
    x[1, 16:] = [100.0] + [0.125] * 15     # s_b = 16: 100 -> 96, 0.125 -> 0
    codes, scales, st = oracle.quantize(x)
    assert st == 1.0
    idx = np.array([1, 2, 3, 4, 16, 17, 0], np.int32)
    got = oracle.residual_columns_bf16(x, codes, scales, st, idx)
    assert got.dtype == np.uint16 and got.shape == (2, 7)
    assert got[0].tolist() == [0] * 7  # 2688 is 6 * 448 * 1, on the grid
    assert got[1].tolist() == [0x3F80, 0x3F82, 0xBF4D, 0x3F00, 0x4080, 0x3E00, 0]


def test_residual_columns_equal_bf16_of_x_minus_dequantize():
    x = _x(3, 77, 96)
    xb = inputs.to_bf16_bits(x)
    for inp in (x, xb):
        codes, scales, st = oracle.quantize(inp)
        xf = inputs.bf16_bits_to_f32(inp) if inp.dtype == np.uint16 else inp
        r = xf - oracle.dequantize(codes, scales, st)  # IEEE fp32 subtraction
        idx = np.array([95, 0, 17, 16, 50, 50], np.int32)
        got = oracle.residual_columns_bf16(inp, codes, scales, st, idx)
        assert np.array_equal(got, inputs.to_bf16_bits(r[:, idx]))
        assert oracle.residual_columns_bf16(inp, codes, scales, st, idx[:0]).shape == (77, 0)

"""GPU parity of moe_grouped_gemm_w4a4_comp against the oracle.

Tolerance (GEMM outputs, fp32-accumulated): |Y_gpu - Y_oracle| /
(||a_row||_2 * ||w_col||_2) <= 2e-3, with a_row the pre-quantization activation
row and w_col the dequantized weight row.  Codes, scales, routing and the
permutation feeding the GEMM are checked bit-exact on the way."""
import numpy as np
import pytest

import oracle
from helpers import assert_bits_equal, log, to_gpu, to_np
from qat_nvfp4_quantize_amd import inputs

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _nvq():
    from qat_nvfp4_quantize_amd import nvq

    return nvq


def check_tol(got, ref, a_rows_f32, w_deq, what):
    an = np.linalg.norm(a_rows_f32.astype(np.float64), axis=1)[:, None]
    wn = np.linalg.norm(w_deq.astype(np.float64), axis=1)[None, :]
    den = np.maximum(an * wn, 1e-30)
    err = np.abs(got.astype(np.float64) - ref) / den
    worst = float(err.max()) if err.size else 0.0
    log(f"[gemm] {what}: max normalized err {worst:.3e} over {err.size} outputs")
    assert worst <= TOL, (what, worst, np.unravel_index(np.argmax(err), err.shape))


def _w_deq(codes, scales, st):
    return oracle.dequantize(codes, scales, st).astype(np.float64)


def _path(name):
    """deq16: exact fp16 dequantization, 128-row tiles; deq16w: the same in
    256-row tiles; fp8_block: FP8 block products scaled in fp32."""
    nvq = _nvq()
    return {"deq16": nvq.NVQ_GEMM_DEQ16, "deq16w": nvq.NVQ_GEMM_DEQ16_WIDE,
            "fp8_block": nvq.NVQ_GEMM_FP8_BLOCK}[name]


@pytest.mark.parametrize("path", ["deq16", "deq16w", "fp8_block"])
def test_dense_check_workload(path):
    import torch

    nvq = _nvq()
    gp = _path(path)
    x, w, k = inputs.dense_check()
    xg, wg = to_gpu(x), to_gpu(w)
    qa = nvq.nvfp4_quantize(xg, score=True)
    qw = nvq.nvfp4_quantize(wg[None])
    idx, resid, _ = nvq.residual_topk_channels(xg, qa[0], qa[1], qa[2], k, scores=qa[3])
    off = torch.tensor([0, x.shape[0]], dtype=torch.int32, device="cuda")
    ob, of = nvq.moe_grouped_gemm_w4a4_comp(qa[0], qa[1], qa[2], qw[0], qw[1], qw[2], off,
                                            rows=x.shape[0], a_resid=resid.contiguous(),
                                            comp_idx=idx, want_f32=True, path=gp)
    torch.cuda.synchronize()
    oqa, oqw = oracle.quantize(x), oracle.quantize(w)
    oidx = oracle.topk(oracle.residual_scores(x, *oqa), k)
    assert_bits_equal(to_np(idx), oidx, "comp idx")
    ref = oracle.moe_gemm_w4a4(*oqa, x, oidx, *oqw, np.arange(64), np.zeros(64))
    check_tol(to_np(of), ref, x, _w_deq(*oqw), "dense f32")
    check_tol(inputs.bf16_bits_to_f32(to_np(ob)), ref, x, _w_deq(*oqw), "dense bf16")
    # k = 0 reproduces the plain W4A4 product
    ob0, of0 = nvq.moe_grouped_gemm_w4a4_comp(qa[0], qa[1], qa[2], qw[0], qw[1], qw[2], off,
                                              rows=x.shape[0], want_f32=True, path=gp)
    ref0 = oracle.moe_gemm_w4a4(*oqa, x, None, *oqw, np.arange(64), np.zeros(64))
    check_tol(to_np(of0), ref0, x, _w_deq(*oqw), "dense k=0")


class MoeRun:
    """Runs a MoE layer stage by stage on the GPU, keeping every intermediate."""

    def __init__(self, s, path=0):
        import torch

        nvq = _nvq()
        self.path = path
        self.s = s
        self.logits = inputs.logits(s)
        self.x = inputs.activations(s)
        log(f"[moe] generating weights E={s.E} H={s.H} I={s.I}")
        self.wgu = inputs.weights(s, "gu")
        self.wdn = inputs.weights(s, "dn")
        xg = to_gpu(self.x)
        self.ids, self.w = nvq.nvq_moe_route(to_gpu(self.logits), s.topk)
        self.sp, self.off, self.pos, _ = nvq.nvq_moe_permute(self.ids, s.E)
        self.a_row = (self.sp // s.topk).contiguous()
        self.qx = nvq.nvfp4_quantize(xg, score=True)
        self.idx1, self.r1, _ = nvq.residual_topk_channels(xg, *self.qx[:3], s.k, scores=self.qx[3])
        self.qgu = nvq.nvfp4_quantize(to_gpu(self.wgu))
        self.qdn = nvq.nvfp4_quantize(to_gpu(self.wdn))
        self.h, self.y1 = nvq.moe_grouped_gemm_w4a4_comp(
            self.qx[0], self.qx[1], self.qx[2], self.qgu[0], self.qgu[1], self.qgu[2], self.off,
            rows=s.P, a_row=self.a_row, a_resid=self.r1.contiguous(), comp_idx=self.idx1,
            epilogue=nvq.NVQ_EPI_SWIGLU, want_f32=True, path=path)
        torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["deq16", "deq16w", "fp8_block"])
@pytest.mark.parametrize("shape", ["small", "small_ragged"])
def test_small_moe_layer_stagewise(shape, path):
    """Every GEMM path (exact fp16 dequantization in 128- and 256-row tiles;
    FP8 block products scaled in fp32) against the same oracle."""
    import torch

    nvq = _nvq()
    gp = _path(path)
    s = inputs.small_moe() if shape == "small" else inputs.small_moe(wid=101, T=77, E=5, topk=3, k=24)
    run = MoeRun(s, gp)
    x = run.x
    xf = inputs.bf16_bits_to_f32(x)
    oids, ow = oracle.route(run.logits, s.topk)
    assert_bits_equal(to_np(run.ids), oids, "ids")
    osp, ooff, opos = oracle.permute(oids, s.E)
    assert_bits_equal(to_np(run.sp), osp, "sorted pairs")
    oqx = oracle.quantize(x)
    oidx1 = oracle.topk(oracle.residual_scores(x, *oqx), s.k)
    assert_bits_equal(to_np(run.idx1), oidx1, "S1")
    wq = [oracle.quantize(run.wgu[e]) for e in range(s.E)]
    wc = np.stack([q[0] for q in wq])
    wsc = np.stack([q[1] for q in wq])
    wst = np.array([q[2] for q in wq], np.float32)
    assert_bits_equal(to_np(run.qgu[0]), wc, "W_gu codes")
    row_tok = osp // s.topk
    row_e = np.repeat(np.arange(s.E), np.diff(ooff)).astype(np.int32)
    ref_y1 = oracle.moe_gemm_w4a4(*oqx, x, oidx1, wc, wsc, wst, row_tok, row_e)
    wdeq = [_w_deq(wc[e], wsc[e], wst[e]) for e in range(s.E)]
    y1 = to_np(run.y1)
    for e in range(s.E):
        rows = slice(ooff[e], ooff[e + 1])
        if ooff[e + 1] > ooff[e]:
            check_tol(y1[rows], ref_y1[rows], xf[row_tok[rows]], wdeq[e], f"gate/up e={e}")
    # SwiGLU epilogue: h = bf16(silu(g) u) on the GPU's own fp32 pre-activation
    h_ref = oracle.swiglu_bf16(y1.astype(np.float64))
    h = to_np(run.h)
    hf, hr = inputs.bf16_bits_to_f32(h), inputs.bf16_bits_to_f32(h_ref)
    np.testing.assert_allclose(hf, hr, rtol=2 ** -7, atol=1e-6)
    # down projection on the oracle's own H (independent input): qH bit-exact, GEMM in tolerance
    H = oracle.swiglu_bf16(ref_y1)
    Hg = to_gpu(H)
    qh = nvq.nvfp4_quantize(Hg, score=True)
    oqh = oracle.quantize(H)
    assert_bits_equal(to_np(qh[0]), oqh[0], "qH codes")
    idx2, r2, _ = nvq.residual_topk_channels(Hg, *qh[:3], s.k, scores=qh[3])
    oidx2 = oracle.topk(oracle.residual_scores(H, *oqh), s.k)
    assert_bits_equal(to_np(idx2), oidx2, "S2")
    qdn = [oracle.quantize(run.wdn[e]) for e in range(s.E)]
    dc = np.stack([q[0] for q in qdn])
    dsc = np.stack([q[1] for q in qdn])
    dst = np.array([q[2] for q in qdn], np.float32)
    ob, of = nvq.moe_grouped_gemm_w4a4_comp(qh[0], qh[1], qh[2], run.qdn[0], run.qdn[1],
                                            run.qdn[2], run.off, rows=s.P,
                                            a_resid=r2.contiguous(), comp_idx=idx2, want_f32=True,
                                            path=gp)
    torch.cuda.synchronize()
    ref_y2 = oracle.moe_gemm_w4a4(*oqh, H, oidx2, dc, dsc, dst, np.arange(s.P), row_e)
    Hf = inputs.bf16_bits_to_f32(H)
    y2 = to_np(of)
    for e in range(s.E):
        rows = slice(ooff[e], ooff[e + 1])
        if ooff[e + 1] > ooff[e]:
            check_tol(y2[rows], ref_y2[rows], Hf[rows], _w_deq(dc[e], dsc[e], dst[e]), f"down e={e}")
    # combine, both sides on the GEMM's bf16 output: fp32 vs fp64 accumulation of
    # topk terms, then one bf16 rounding -> at most one bf16 ulp apart
    out = nvq.nvq_moe_combine(ob, run.pos, run.w)
    y2b = inputs.bf16_bits_to_f32(to_np(ob))
    ref_out = inputs.bf16_bits_to_f32(oracle.combine_bf16(y2b, opos, ow))
    got = inputs.bf16_bits_to_f32(to_np(out))
    mag = np.einsum("tj,tjn->tn", np.abs(ow), np.abs(y2b[opos.reshape(-1, s.topk)]))
    bound = 2.0 ** -7 * np.maximum(np.abs(got), np.abs(ref_out)) + 2.0 ** -20 * mag + 1e-30
    assert np.all(np.abs(got - ref_out) <= bound), float(np.max(np.abs(got - ref_out) / bound))


def _sample_rows(off, every=97):
    rows = set()
    for e in range(len(off) - 1):
        if off[e + 1] > off[e]:
            rows.add(int(off[e]))
            rows.add(int(off[e + 1] - 1))
    rows.update(range(0, int(off[-1]), every))
    return np.array(sorted(rows), np.int64)


def test_decode_layer_gate_up_sampled():
    """Full-size decode layer (T=4096, H=2048, E=128, I=768, top-8, k=64): gate/up
    GEMM in the launch configuration of the benchmark, checked on sampled rows."""
    s = inputs.DECODE
    run = MoeRun(s)
    x = run.x
    oqx = oracle.quantize(x)
    oidx1 = oracle.topk(oracle.residual_scores(x, *oqx), s.k)
    assert_bits_equal(to_np(run.idx1), oidx1, "S1")
    off = to_np(run.off)
    sp = to_np(run.sp)
    rows = _sample_rows(off, every=211)
    row_e = np.searchsorted(off, rows, side="right") - 1
    row_tok = sp[rows] // s.topk
    experts = sorted(set(row_e.tolist()))
    wq = {e: oracle.quantize(run.wgu[e]) for e in experts}
    wc = np.stack([wq[e][0] for e in experts])
    wsc = np.stack([wq[e][1] for e in experts])
    wst = np.array([wq[e][2] for e in experts], np.float32)
    local_e = np.array([experts.index(e) for e in row_e], np.int32)
    log(f"[decode] oracle on {len(rows)} sampled rows x {2 * s.I} cols")
    ref = oracle.moe_gemm_w4a4(*oqx, x, oidx1, wc, wsc, wst, row_tok, local_e)
    y1 = to_np(run.y1)[rows]
    xf = inputs.bf16_bits_to_f32(x)
    for i, e in enumerate(experts):
        sel = local_e == i
        check_tol(y1[sel], ref[sel], xf[row_tok[sel]], _w_deq(wc[i], wsc[i], wst[i]), f"decode e={e}")


@pytest.mark.parametrize("path", ["deq16", "deq16w", "fp8_block"])
@pytest.mark.parametrize("K,N,k,epi", [(128, 160, 8, "none"), (384, 384, 128, "none"),
                                       (384, 192, 0, "swiglu"), (128, 208, 128, "swiglu"),
                                       (256, 512, 72, "swiglu"), (256, 320, 200, "none")])
def test_grouped_gemm_edge_shapes(K, N, k, epi, path):
    """Direct grouped-GEMM calls on shapes the layer tests do not reach: an odd
    number of 128-element K steps (K = 384), partial column tiles (N = 160,
    208, 320, 384; SwiGLU halves of 96 and 104), k = K, k = 0, k not a
    multiple of 64, experts with no rows, one expert with more rows than one
    256-row tile and one with more than one 128-row tile, fp32 and bf16
    outputs, and rows read through a_row with a divisor."""
    # P = 360 sorted rows of 420 pairs
    _grouped_gemm_case(K, N, k, epi, path, counts=[0, 300, 3, 0, 57], T=140, topk=3)


@pytest.mark.parametrize("epi", ["none", "swiglu"])
@pytest.mark.parametrize("k", [16, 200])
def test_grouped_gemm_ragged_tail_tiles(epi, k):
    """Experts whose last 128-row tile holds 32 rows (served by the one-sub-tile
    copy of the main loop), 33 rows (the full loop), 1 row, or exactly fills
    its tile, with one compensation step and with two (k = 200: the second
    step loads its own operands): every row against the oracle."""
    _grouped_gemm_case(256, 256, k, epi, "deq16", counts=[32, 33, 160, 161, 0, 1, 64, 128], T=200, topk=3)


def _grouped_gemm_case(K, N, k, epi, path, counts, T, topk):
    import torch

    nvq = _nvq()
    gp = _path(path)
    swiglu = epi == "swiglu"
    g = np.random.default_rng(K * 1000 + N + k)
    counts = np.asarray(counts)
    E = len(counts)
    P = int(counts.sum())
    assert P <= T * topk
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pair = g.permutation(T * topk)[:P].astype(np.int32)  # sorted pair ids; token = pair // topk
    x = (g.standard_normal((T, K)) * np.exp(g.standard_normal((1, K)))).astype(np.float32)
    w = (g.standard_normal((E, N, K)) * 0.05).astype(np.float32)
    log(f"[gemm-edge] K={K} N={N} k={k} {epi} {path}")
    xg = to_gpu(x)
    qa = nvq.nvfp4_quantize(xg, score=True)
    qw = nvq.nvfp4_quantize(to_gpu(w))
    resid, idx = None, None
    if k > 0:
        idx, resid, _ = nvq.residual_topk_channels(xg, *qa[:3], k, scores=qa[3])
        resid = resid.contiguous()
    ob, of = nvq.moe_grouped_gemm_w4a4_comp(
        qa[0], qa[1], qa[2], qw[0], qw[1], qw[2], to_gpu(off), rows=P, a_row=to_gpu(pair),
        a_resid=resid, comp_idx=idx, epilogue=nvq.NVQ_EPI_SWIGLU if swiglu else nvq.NVQ_EPI_NONE,
        want_f32=True, path=gp, a_row_div=topk)
    torch.cuda.synchronize()
    if k > 0:
        # the compensation gathered from the channel-major record: same outputs, bit for bit
        wcm = nvq.nvfp4_channel_major(qw[0], qw[1])
        ob2, of2 = nvq.moe_grouped_gemm_w4a4_comp(
            qa[0], qa[1], qa[2], qw[0], qw[1], qw[2], to_gpu(off), rows=P, a_row=to_gpu(pair),
            a_resid=resid, comp_idx=idx,
            epilogue=nvq.NVQ_EPI_SWIGLU if swiglu else nvq.NVQ_EPI_NONE, want_f32=True, path=gp,
            a_row_div=topk, w_cm=wcm)
        torch.cuda.synchronize()
        assert_bits_equal(to_np(of2), to_np(of), "fp32 output with the channel-major record")
        assert_bits_equal(to_np(ob2), to_np(ob), "bf16 output with the channel-major record")
    oqa = oracle.quantize(x)
    oidx = oracle.topk(oracle.residual_scores(x, *oqa), k) if k > 0 else None
    if k > 0:
        assert_bits_equal(to_np(idx), oidx, "comp idx")
    wq = [oracle.quantize(w[e]) for e in range(E)]
    wc = np.stack([q[0] for q in wq])
    wsc = np.stack([q[1] for q in wq])
    wst = np.array([q[2] for q in wq], np.float32)
    assert_bits_equal(to_np(qw[0]), wc, "weight codes")
    row_tok = (pair // topk).astype(np.int32)
    row_e = np.repeat(np.arange(E), counts).astype(np.int32)
    ref = oracle.moe_gemm_w4a4(*oqa, x, oidx, wc, wsc, wst, row_tok, row_e)
    y = to_np(of)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        if off[e + 1] > off[e]:
            check_tol(y[rows], ref[rows], x[row_tok[rows]], _w_deq(wc[e], wsc[e], wst[e]),
                      f"edge e={e}")
    if swiglu:
        h_ref = oracle.swiglu_bf16(y.astype(np.float64))
        np.testing.assert_allclose(inputs.bf16_bits_to_f32(to_np(ob)), inputs.bf16_bits_to_f32(h_ref),
                                   rtol=2 ** -7, atol=1e-6)
    else:
        assert_bits_equal(to_np(ob), inputs.to_bf16_bits(y), "bf16 output = rounded fp32 output")


@pytest.mark.parametrize("B,N,K", [(2, 96, 160), (1, 208, 48), (3, 64, 64), (1, 16, 1040)])
def test_channel_major_record_layout(B, N, K):
    """nvfp4_channel_major is a pure relayout: random code and scale bytes,
    compared byte for byte with the same relayout in numpy (partial 64-wide
    tiles in both directions)."""
    import torch

    nvq = _nvq()
    g = np.random.default_rng(B * 7 + N * 3 + K)
    codes = g.integers(0, 256, (B, N, K // 2), dtype=np.uint8)
    scales = g.integers(0, 127, (B, N, K // 16), dtype=np.uint8)
    ccm, scm = nvq.nvfp4_channel_major(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    nib = np.empty((B, N, K), np.uint8)
    nib[..., 0::2] = codes & 15
    nib[..., 1::2] = codes >> 4
    t = nib.transpose(0, 2, 1)  # [B, K, N]
    want_codes = (t[..., 0::2] | (t[..., 1::2] << 4)).astype(np.uint8)
    assert_bits_equal(to_np(ccm), want_codes, "channel-major codes")
    assert_bits_equal(to_np(scm), np.ascontiguousarray(scales.transpose(0, 2, 1)), "channel-major scales")


def test_grouped_gemm_no_rows():
    """rows = 0 with k > 0: the call succeeds and launches nothing harmful; the
    empty outputs stay empty."""
    import torch

    nvq = _nvq()
    E, N, K, k = 4, 256, 256, 8
    g = np.random.default_rng(9)
    qw = nvq.nvfp4_quantize(to_gpu((g.standard_normal((E, N, K)) * 0.05).astype(np.float32)))
    qa = nvq.nvfp4_quantize(torch.empty(0, K, dtype=torch.float32, device="cuda"))
    off = to_gpu(np.zeros(E + 1, np.int32))
    idx = to_gpu(np.arange(k, dtype=np.int32))
    resid = torch.empty(0, k, dtype=torch.bfloat16, device="cuda")
    ob, of = nvq.moe_grouped_gemm_w4a4_comp(qa[0], qa[1], qa[2], qw[0], qw[1], qw[2], off, rows=0,
                                            a_resid=resid, comp_idx=idx, want_f32=True)
    torch.cuda.synchronize()
    assert ob.shape == (0, N) and of.shape == (0, N)


@pytest.mark.parametrize("path", ["deq16", "fp8_block"])
def test_h_amax_from_the_swiglu_epilogue(path):
    """max |h| recorded by the gate/up epilogue on a small ragged layer (both
    paths), cleared per call, 0 without rows, refused with another epilogue,
    and not read when the caller's struct predates the field."""
    import ctypes

    import torch

    nvq = _nvq()
    gp = nvq.NVQ_GEMM_DEQ16 if path == "deq16" else nvq.NVQ_GEMM_FP8_BLOCK
    s = inputs.small_moe(wid=101, T=77, E=5, topk=3, k=24)
    run = MoeRun(s, gp)
    h_amax = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    h, _ = nvq.moe_grouped_gemm_w4a4_comp(
        run.qx[0], run.qx[1], run.qx[2], run.qgu[0], run.qgu[1], run.qgu[2], run.off, rows=s.P,
        a_row=run.a_row, a_resid=run.r1.contiguous(), comp_idx=run.idx1,
        epilogue=nvq.NVQ_EPI_SWIGLU, path=gp, h_amax=h_amax)
    torch.cuda.synchronize()
    assert float(to_np(h_amax)[0]) == float(np.abs(inputs.bf16_bits_to_f32(to_np(h))).max())
    assert float(to_np(h_amax)[0]) > 0
    # no rows: the amax of nothing is 0
    qa0 = nvq.nvfp4_quantize(torch.empty(0, s.H, dtype=torch.float32, device="cuda"))
    nvq.moe_grouped_gemm_w4a4_comp(qa0[0], qa0[1], qa0[2], run.qgu[0], run.qgu[1], run.qgu[2],
                                   to_gpu(np.zeros(s.E + 1, np.int32)), rows=0,
                                   epilogue=nvq.NVQ_EPI_SWIGLU, h_amax=h_amax)
    torch.cuda.synchronize()
    assert float(to_np(h_amax)[0]) == 0.0
    with pytest.raises(nvq.NvqError):
        nvq.moe_grouped_gemm_w4a4_comp(run.qx[0], run.qx[1], run.qx[2], run.qgu[0], run.qgu[1],
                                       run.qgu[2], run.off, rows=s.P, a_row=run.a_row,
                                       epilogue=nvq.NVQ_EPI_NONE, h_amax=h_amax)
    # a caller built against the earlier struct: the field is never read
    L = nvq.load()
    a = nvq.MoeGemmArgs()
    a.struct_size = nvq.MoeGemmArgs.h_amax.offset
    a.rows, a.K, a.N, a.E = s.P, s.H, 2 * s.I, s.E
    a.a_rows = s.T
    a.a_row, a.expert_offsets = ctypes.c_void_p(run.a_row.data_ptr()), ctypes.c_void_p(run.off.data_ptr())
    a.a_codes, a.a_scales = ctypes.c_void_p(run.qx[0].data_ptr()), ctypes.c_void_p(run.qx[1].data_ptr())
    a.a_tensor_scale = ctypes.c_void_p(run.qx[2].data_ptr())
    a.w_codes, a.w_scales = ctypes.c_void_p(run.qgu[0].data_ptr()), ctypes.c_void_p(run.qgu[1].data_ptr())
    a.w_tensor_scale = ctypes.c_void_p(run.qgu[2].data_ptr())
    a.epilogue, a.path = nvq.NVQ_EPI_SWIGLU, gp
    out = torch.empty(s.P, s.I, dtype=torch.bfloat16, device="cuda")
    a.out_bf16 = ctypes.c_void_p(out.data_ptr())
    ws = nvq.workspace(L.moe_gemm_workspace_bytes(s.P, s.E, 2 * s.I, 0), "cuda")
    a.ws, a.ws_bytes = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    h_amax.fill_(7.0)
    a.h_amax = ctypes.c_void_p(h_amax.data_ptr())
    assert L.moe_grouped_gemm_w4a4_comp(ctypes.byref(a), ctypes.c_void_p(
        torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    assert float(to_np(h_amax)[0]) == 7.0


def _prefill_weights(nvq, s, proj):
    """The benchmark's weights: drawn on the device, quantized there, with the
    channel-major copy the benchmark passes for the compensation gather."""
    w = inputs.weights_device(s, proj)
    q = nvq.nvfp4_quantize(w)
    cm = nvq.nvfp4_channel_major(q[0], q[1])
    return w, q, cm


def _check_sampled(nvq, s, y, rows, row_tok, row_e, oq, x_hi, oidx, w, q, what):
    """Oracle rows of the W4A4 + compensation GEMM for the sampled rows; the
    sampled experts' weights are quantized by the oracle from the same draw and
    checked bit-exact against the device record first."""
    experts = sorted(set(row_e.tolist()))
    wq = {}
    for e in experts:
        wb = to_np(w[e])
        wq[e] = oracle.quantize(wb)
        assert_bits_equal(to_np(q[0][e]), wq[e][0], f"{what} weight codes e={e}")
        assert_bits_equal(to_np(q[1][e]), wq[e][1], f"{what} weight scales e={e}")
    wc = np.stack([wq[e][0] for e in experts])
    wsc = np.stack([wq[e][1] for e in experts])
    wst = np.array([wq[e][2] for e in experts], np.float32)
    local_e = np.array([experts.index(e) for e in row_e], np.int32)
    log(f"[prefill] {what}: oracle on {len(rows)} sampled rows x {wc.shape[1]} cols, {len(experts)} experts")
    ref = oracle.moe_gemm_w4a4(*oq, x_hi, oidx, wc, wsc, wst, row_tok, local_e)
    xf = inputs.bf16_bits_to_f32(x_hi)
    for i, e in enumerate(experts):
        sel = local_e == i
        check_tol(y[sel], ref[sel], xf[row_tok[sel]], _w_deq(wc[i], wsc[i], wst[i]), f"{what} e={e}")


def test_prefill_gate_up_full_size_sampled():
    """Full-size prefill layer (T=32768, H=4096, E=128, I=1536, top-8, k=128)
    in the benchmark's launch configuration (sorted pair ids with a divisor,
    channel-major record for the compensation): routing and permutation from
    the oracle checked bit-exact, then the gate/up GEMM on sampled rows."""
    import torch

    nvq = _nvq()
    s = inputs.PREFILL
    logits, x = inputs.logits(s), inputs.activations(s)
    ids, _ = nvq.nvq_moe_route(to_gpu(logits), s.topk)
    sp, off, _, _ = nvq.nvq_moe_permute(ids, s.E)
    oids, _ = oracle.route(logits, s.topk)
    osp, ooff, _ = oracle.permute(oids, s.E)
    assert_bits_equal(to_np(sp), osp, "sorted pairs")
    assert_bits_equal(to_np(off), ooff, "expert offsets")
    xg = to_gpu(x)
    qx = nvq.nvfp4_quantize(xg, score=True)
    idx1, r1, _ = nvq.residual_topk_channels(xg, *qx[:3], s.k, scores=qx[3])
    w, q, cm = _prefill_weights(nvq, s, "gu")
    h_amax = torch.full((1,), 123.0, dtype=torch.float32, device="cuda")  # the call clears it
    h, y1 = nvq.moe_grouped_gemm_w4a4_comp(qx[0], qx[1], qx[2], q[0], q[1], q[2], off, rows=s.P, a_row=sp,
                                           a_resid=r1.contiguous(), comp_idx=idx1,
                                           epilogue=nvq.NVQ_EPI_SWIGLU, want_f32=True, a_row_div=s.topk,
                                           w_cm=cm, h_amax=h_amax)
    torch.cuda.synchronize()
    # the epilogue's max |h| is the amax of the stored H, and quantizing H with
    # it gives the same record as quantizing H on its own
    hb = to_np(h)
    assert float(to_np(h_amax)[0]) == float(np.abs(inputs.bf16_bits_to_f32(hb)).max())
    qa = nvq.nvfp4_quantize(h, amax_in=h_amax, score=True)
    qb = nvq.nvfp4_quantize(h, score=True)
    torch.cuda.synchronize()
    for u, v, what in zip(qa[:4], qb[:4], ("codes", "scales", "s_t", "scores")):
        assert_bits_equal(to_np(u), to_np(v), "H with epilogue amax: " + what)
    del h, hb, qa, qb
    oqx = oracle.quantize(x)
    assert_bits_equal(to_np(qx[0]), oqx[0], "X codes")
    oidx1 = oracle.topk(oracle.residual_scores(x, *oqx), s.k)
    assert_bits_equal(to_np(idx1), oidx1, "X channels")
    rows = _sample_rows(ooff, every=1499)
    row_e = np.searchsorted(ooff, rows, side="right") - 1
    _check_sampled(nvq, s, to_np(y1)[rows], rows, (osp[rows] // s.topk).astype(np.int32), row_e, oqx, x,
                   oidx1, w, q, "gate/up")


def _check_fused_combine(nvq, s, logits, qh, idx2, r2, q, cm, ooff):
    """The down projection with the layer's combine fused (bf16 output only,
    as the benchmark runs it): the fused output equals nvq_moe_combine on the
    same call's bf16 rows, bit for bit, on two calls in a row."""
    import torch

    oids, ow = oracle.route(logits, s.topk)
    osp, _, opos = oracle.permute(oids, s.E)
    spg, posg, wg = to_gpu(osp), to_gpu(opos), to_gpu(ow)
    for rep in range(2):
        cout = torch.empty(s.T, s.H, dtype=torch.bfloat16, device="cuda")
        ob, _ = nvq.moe_grouped_gemm_w4a4_comp(qh[0], qh[1], qh[2], q[0], q[1], q[2], to_gpu(ooff),
                                               rows=s.P, a_resid=r2.contiguous(), comp_idx=idx2,
                                               w_cm=cm, comb=(spg, posg, wg, cout))
        ref = nvq.nvq_moe_combine(ob, posg, wg)
        torch.cuda.synchronize()
        assert_bits_equal(to_np(cout), to_np(ref), f"fused combine, call {rep}")
        log(f"[gemm] fused combine {s.T}x{s.H} equals the separate combine (call {rep})")


@pytest.mark.parametrize("path", ["deq16", "fp8_block"])
@pytest.mark.parametrize("k", [0, 24])
def test_fused_combine_small_with_dropped_pairs(path, k):
    """The combine fused into the down projection on a small layer whose
    permutation dropped pairs (a bad expert id), including a token whose pairs
    were all dropped (its output is the empty sum, 0), a partial column tile
    (N = 384) and an expert with more rows than one tile: bit-equal to
    nvq_moe_combine on the call's own bf16 output, also on a second call."""
    import torch

    nvq = _nvq()
    g = np.random.default_rng(2024 + k)
    E, T, topk, K, N = 6, 150, 3, 256, 384
    # tokens 0..39 all route to expert 1 first, so it gets more than 128 rows
    ids = np.stack([g.permutation(E)[:topk] if t >= 40 else
                    np.concatenate([[1], g.permutation([e for e in range(E) if e != 1])[:topk - 1]])
                    for t in range(T)]).astype(np.int32)
    ids[g.random((T, topk)) < 0.06] = E + 2
    ids[7, :] = E + 2  # token 7: every pair dropped
    sp, off, pos, _ = nvq.nvq_moe_permute(to_gpu(ids), E)
    P = int(to_np(off)[-1])
    wts = to_gpu(g.random((T, topk)).astype(np.float32))
    x = (g.standard_normal((P, K)) * np.exp(g.standard_normal((1, K)))).astype(np.float32)
    xg = to_gpu(x)
    qa = nvq.nvfp4_quantize(xg, score=True)
    qw = nvq.nvfp4_quantize(to_gpu((g.standard_normal((E, N, K)) * 0.05).astype(np.float32)))
    resid, idx = None, None
    if k > 0:
        idx, resid, _ = nvq.residual_topk_channels(xg, *qa[:3], k, scores=qa[3])
        resid = resid.contiguous()
    log(f"[gemm] fused combine small k={k} {path} P={P}")
    for rep in range(2):
        cout = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
        ob, _ = nvq.moe_grouped_gemm_w4a4_comp(qa[0], qa[1], qa[2], qw[0], qw[1], qw[2], off, rows=P,
                                               a_resid=resid, comp_idx=idx, path=_path(path),
                                               comb=(sp, pos, wts, cout))
        ref = nvq.nvq_moe_combine(ob, pos, wts)
        torch.cuda.synchronize()
        assert_bits_equal(to_np(cout), to_np(ref), f"fused combine call {rep}")
        assert not to_np(cout)[7].any(), "token with every pair dropped"


def test_prefill_down_full_size_sampled():
    """Full-size prefill down projection (K=1536, N=4096, k=128, P=262144 rows)
    in the benchmark's launch configuration, on an independently drawn H of the
    layer's shape: H's record checked bit-exact, then sampled rows."""
    import torch

    nvq = _nvq()
    s = inputs.PREFILL
    logits = inputs.logits(s)
    oids, _ = oracle.route(logits, s.topk)
    _, ooff, _ = oracle.permute(oids, s.E)
    hb = inputs.hidden(s)
    hg = to_gpu(hb)
    qh = nvq.nvfp4_quantize(hg, score=True)
    idx2, r2, _ = nvq.residual_topk_channels(hg, *qh[:3], s.k, scores=qh[3])
    w, q, cm = _prefill_weights(nvq, s, "dn")
    _, y2 = nvq.moe_grouped_gemm_w4a4_comp(qh[0], qh[1], qh[2], q[0], q[1], q[2], to_gpu(ooff), rows=s.P,
                                           a_resid=r2.contiguous(), comp_idx=idx2, want_f32=True, w_cm=cm)
    torch.cuda.synchronize()
    oqh = oracle.quantize(hb)
    assert_bits_equal(to_np(qh[0]), oqh[0], "H codes")
    oidx2 = oracle.topk(oracle.residual_scores(hb, *oqh), s.k)
    assert_bits_equal(to_np(idx2), oidx2, "H channels")
    rows = _sample_rows(ooff, every=1499)
    row_e = np.searchsorted(ooff, rows, side="right") - 1
    _check_sampled(nvq, s, to_np(y2)[rows], rows, rows.astype(np.int32), row_e, oqh, hb, oidx2, w, q, "down")
    _check_fused_combine(nvq, s, logits, qh, idx2, r2, q, cm, ooff)


def test_decode_down_full_size_sampled():
    """Full-size decode down projection (K=768, N=2048, k=64, P=32768 rows) in
    the benchmark's launch configuration (channel-major record for the
    compensation), on an independently drawn H of the layer's shape: H's
    record and channels bit-exact, then sampled rows."""
    import torch

    nvq = _nvq()
    s = inputs.DECODE
    oids, _ = oracle.route(inputs.logits(s), s.topk)
    _, ooff, _ = oracle.permute(oids, s.E)
    hb = inputs.hidden(s)
    hg = to_gpu(hb)
    qh = nvq.nvfp4_quantize(hg, score=True)
    idx2, r2, _ = nvq.residual_topk_channels(hg, *qh[:3], s.k, scores=qh[3])
    w, q, cm = _prefill_weights(nvq, s, "dn")
    _, y2 = nvq.moe_grouped_gemm_w4a4_comp(qh[0], qh[1], qh[2], q[0], q[1], q[2], to_gpu(ooff), rows=s.P,
                                           a_resid=r2.contiguous(), comp_idx=idx2, want_f32=True, w_cm=cm)
    torch.cuda.synchronize()
    oqh = oracle.quantize(hb)
    assert_bits_equal(to_np(qh[0]), oqh[0], "H codes")
    oidx2 = oracle.topk(oracle.residual_scores(hb, *oqh), s.k)
    assert_bits_equal(to_np(idx2), oidx2, "H channels")
    rows = _sample_rows(ooff, every=173)
    row_e = np.searchsorted(ooff, rows, side="right") - 1
    _check_sampled(nvq, s, to_np(y2)[rows], rows, rows.astype(np.int32), row_e, oqh, hb, oidx2, w, q,
                   "decode down")
    _check_fused_combine(nvq, s, inputs.logits(s), qh, idx2, r2, q, cm, ooff)

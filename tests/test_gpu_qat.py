"""GPU parity of qat_fakequant_gemm_w4a16 (forward, input gradient, weight
gradient) against the oracle.  Tolerance as for the W4A4 GEMM:
|err| / (||a||_2 * ||b||_2) <= 2e-3 with a, b the two contracted vectors."""
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


def _norm_err(got, ref, an, bn, what):
    den = np.maximum(np.outer(an, bn), 1e-30)
    err = np.abs(got.astype(np.float64) - ref) / den
    worst = float(err.max()) if err.size else 0.0
    log(f"[qat] {what}: max normalized err {worst:.3e} over {err.size} outputs")
    assert worst <= TOL, (what, worst)


def _setup(s, proj):
    """Routing, permutation, x, dy and the quantized weight cache for one projection."""
    import torch

    nvq = _nvq()
    logits = inputs.logits(s)
    ids, w = nvq.nvq_moe_route(to_gpu(logits), s.topk)
    sp, off, pos, _ = nvq.nvq_moe_permute(ids, s.E)
    a_row = (sp // s.topk).to(torch.int32).contiguous()
    K, N = (s.H, 2 * s.I) if proj == "gu" else (s.I, s.H)
    g = np.random.default_rng(1234 + s.wid)
    x = inputs.to_bf16_bits(g.standard_normal((s.T if proj == "gu" else s.P, K)).astype(np.float32))
    dy = inputs.to_bf16_bits(g.standard_normal((s.P, N)).astype(np.float32))
    wm = inputs.weights(s, proj)  # bf16 master weights [E, N, K]
    q = nvq.nvfp4_quantize(to_gpu(wm))  # the rollout's cached record
    torch.cuda.synchronize()
    return dict(ids=ids, sp=sp, off=off, a_row=a_row, x=x, dy=dy, wm=wm, q=q, K=K, N=N,
                row_tok=to_np(sp) // s.topk, offn=to_np(off))


@pytest.mark.parametrize("proj", ["gu", "dn"])
def test_small_qat_all_modes(proj):
    import torch

    nvq = _nvq()
    s = inputs.small_moe(wid=102, T=120, H=256, E=6, I=128, topk=2)
    d = _setup(s, proj)
    K, N = d["K"], d["N"]
    wq = [oracle.quantize(d["wm"][e]) for e in range(s.E)]
    wc = np.stack([q[0] for q in wq])
    wsc = np.stack([q[1] for q in wq])
    wst = np.array([q[2] for q in wq], np.float32)
    assert_bits_equal(to_np(d["q"][0]), wc, "weight cache codes")
    off = d["offn"]
    row_e = np.repeat(np.arange(s.E), np.diff(off)).astype(np.int32)
    # forward rows: gate/up gathers token rows, down reads sorted rows directly
    x_row = d["row_tok"] if proj == "gu" else np.arange(s.P)
    a_row = d["a_row"] if proj == "gu" else None
    xg, dyg = to_gpu(d["x"]), to_gpu(d["dy"])
    yb, yf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *d["q"][:3], d["off"], s.P, x=xg,
                                         a_row=a_row, want_f32=True)
    dxb, dxf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *d["q"][:3], d["off"], s.P, dy=dyg,
                                           want_f32=True)
    # bf16 alone (staged through LDS for whole column tiles): the same bits
    dxb_only = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *d["q"][:3], d["off"], s.P, dy=dyg)[0]
    dw = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *d["q"][:3], d["off"], s.P, x=xg, dy=dyg,
                                      a_row=a_row)
    torch.cuda.synchronize()
    assert_bits_equal(to_np(dxb_only), to_np(dxb), "dx bf16 without the fp32 output")
    X = inputs.bf16_bits_to_f32(d["x"]).astype(np.float64)
    DY = inputs.bf16_bits_to_f32(d["dy"]).astype(np.float64)
    ref_y = oracle.qat_fwd(d["x"], x_row, row_e, wc, wsc, wst)
    ref_dx = oracle.qat_dgrad(d["dy"], np.arange(s.P), row_e, wc, wsc, wst)
    y, dx, dwn = to_np(yf), to_np(dxf), to_np(dw)
    for e in range(s.E):
        rows = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        W = oracle.dequantize(wc[e], wsc[e], wst[e]).astype(np.float64)
        _norm_err(y[rows], ref_y[rows], np.linalg.norm(X[x_row[rows]], axis=1),
                  np.linalg.norm(W, axis=1), f"{proj} fwd e={e}")
        _norm_err(dx[rows], ref_dx[rows], np.linalg.norm(DY[rows], axis=1),
                  np.linalg.norm(W, axis=0), f"{proj} dgrad e={e}")
        nn, cc = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
        ref_w = oracle.qat_wgrad(d["dy"], d["x"], x_row, off[e], off[e + 1], nn.ravel(), cc.ravel())
        _norm_err(dwn[e], ref_w.reshape(N, K), np.linalg.norm(DY[rows], axis=0),
                  np.linalg.norm(X[x_row[rows]], axis=0), f"{proj} wgrad e={e}")
    # bf16 outputs are the rounded fp32 outputs
    np.testing.assert_array_equal(to_np(yb), inputs.to_bf16_bits(y))
    np.testing.assert_array_equal(to_np(dxb), inputs.to_bf16_bits(dx))
    # accumulate: dw += dW
    dw2 = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *d["q"][:3], d["off"], s.P, x=xg, dy=dyg,
                                       a_row=a_row, dw=dw.clone(), accumulate=True)
    np.testing.assert_allclose(to_np(dw2), 2 * dwn, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("K,N,counts", [
    (128, 96, (0, 77, 130)),              # one forward step, partial column tile, empty expert
    (384, 160, (1, 0, 129, 255, 3)),      # odd forward step count, ragged row tiles
    (640, 288, (128, 0, 0, 200)),         # five forward steps, column tile + 32-column tail
    (160, 384, (300, 0, 257, 1)),         # three input-gradient steps, 32-column tail
    (96, 128, (0, 513, 40)),              # one input-gradient step, partial column tile
    (256, 256, (0, 300, 5, 129)),         # input gradient, wide weight path: 2 column tiles, 2 steps
    (384, 128, (77, 0, 260)),             # wide weight path: 3 column tiles, one step
])
def test_fwd_dgrad_edge_shapes(K, N, counts):
    """Forward, input and weight gradient on shapes off the tile grid: row
    tiles cut by expert ends, empty experts, odd and single contraction-step
    counts, partial column tiles (both the 128-step kernels and the 32-step
    one), expert segments of 1 and 3 rows and ragged 32-row weight-gradient
    steps, weight gradient accumulated."""
    import torch

    nvq = _nvq()
    g = np.random.default_rng(K * 31 + N)
    E, T = len(counts), 211
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = int(off[-1])
    row_e = np.repeat(np.arange(E), counts).astype(np.int32)
    x_row = g.integers(0, T, P).astype(np.int32)
    x = inputs.to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    dy = inputs.to_bf16_bits(g.standard_normal((P, N)).astype(np.float32))
    wm = inputs.to_bf16_bits((0.02 * g.standard_normal((E, N, K))).astype(np.float32))
    q = nvq.nvfp4_quantize(to_gpu(wm))
    offg = to_gpu(off)
    yb, yf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *q[:3], offg, P, x=to_gpu(x),
                                         a_row=to_gpu(x_row), want_f32=True)
    dxb, dxf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *q[:3], offg, P, dy=to_gpu(dy),
                                           want_f32=True)
    dxb_only = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *q[:3], offg, P, dy=to_gpu(dy))[0]
    dw = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *q[:3], offg, P, x=to_gpu(x),
                                      dy=to_gpu(dy), a_row=to_gpu(x_row))
    dw2 = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *q[:3], offg, P, x=to_gpu(x),
                                       dy=to_gpu(dy), a_row=to_gpu(x_row), dw=dw.clone(),
                                       accumulate=True)
    torch.cuda.synchronize()
    assert_bits_equal(to_np(dxb_only), to_np(dxb), "dx bf16 without the fp32 output")
    wq = [oracle.quantize(wm[e]) for e in range(E)]
    wc = np.stack([w[0] for w in wq])
    assert_bits_equal(to_np(q[0]), wc, "weight cache codes")
    wsc = np.stack([w[1] for w in wq])
    wst = np.array([w[2] for w in wq], np.float32)
    ref_y = oracle.qat_fwd(x, x_row, row_e, wc, wsc, wst)
    ref_dx = oracle.qat_dgrad(dy, np.arange(P), row_e, wc, wsc, wst)
    y, dx = to_np(yf), to_np(dxf)
    X = inputs.bf16_bits_to_f32(x).astype(np.float64)
    DY = inputs.bf16_bits_to_f32(dy).astype(np.float64)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        W = oracle.dequantize(wc[e], wsc[e], wst[e]).astype(np.float64)
        _norm_err(y[rows], ref_y[rows], np.linalg.norm(X[x_row[rows]], axis=1),
                  np.linalg.norm(W, axis=1), f"fwd K={K} N={N} e={e}")
        _norm_err(dx[rows], ref_dx[rows], np.linalg.norm(DY[rows], axis=1),
                  np.linalg.norm(W, axis=0), f"dgrad K={K} N={N} e={e}")
    dwn = to_np(dw)
    nn, cc = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:  # no rows: the gradient is zero
            assert not dwn[e].any(), f"wgrad of empty expert {e} not zero"
            continue
        ref_w = oracle.qat_wgrad(dy, x, x_row, off[e], off[e + 1], nn.ravel(), cc.ravel())
        _norm_err(dwn[e], ref_w.reshape(N, K), np.linalg.norm(DY[rows], axis=0),
                  np.linalg.norm(X[x_row[rows]], axis=0), f"wgrad K={K} N={N} e={e}")
    np.testing.assert_allclose(to_np(dw2), 2 * dwn, rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(to_np(yb), inputs.to_bf16_bits(y))
    np.testing.assert_array_equal(to_np(dxb), inputs.to_bf16_bits(dx))


def test_forward_uses_the_cached_rounding():
    """The forward's weight equals the rollout's dequantized record (QUADS §2.1:
    same quantize-dequantize path): FWD on the cache == dense GEMM on
    nvfp4_dequantize(cache), up to fp32 summation order."""
    import torch

    nvq = _nvq()
    s = inputs.small_moe(wid=103, T=64, H=256, E=1, I=128, topk=1)
    d = _setup(s, "gu")
    wdq = nvq.nvfp4_dequantize(*d["q"][:3], out_dtype=torch.float32)  # [1, N, K]
    xg = to_gpu(d["x"])
    _, yf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *d["q"][:3], d["off"], s.P, x=xg,
                                        a_row=d["a_row"], want_f32=True)
    ref = xg.float()[d["a_row"].long()] @ wdq[0].T
    torch.cuda.synchronize()
    X = inputs.bf16_bits_to_f32(d["x"]).astype(np.float64)[d["row_tok"]]
    W = to_np(wdq[0]).astype(np.float64)
    _norm_err(to_np(yf), to_np(ref).astype(np.float64), np.linalg.norm(X, axis=1),
              np.linalg.norm(W, axis=1), "fwd vs dense on dequantized cache")


@pytest.mark.parametrize("proj,guided", [("gu", False), ("gu", True), ("dn", True)])
def test_qat_layer_full_size_sampled(proj, guided):
    """Trainer QAT layer at full size (T=16384, H=4096, E=128, I=1536, top-8,
    P=131072) in the benchmark's launch configuration: forward, input and
    weight gradients of one projection on sampled outputs.  guided: the codes
    are the drifted masters' codes rebuilt from the rollout's mantissa record
    (what the benchmark's layer step runs); else the rollout's cached codes.
    gate/up: K=4096, N=3072, x gathered by token; down: K=1536, N=4096, x in
    sorted-pair order.  Rows: every 97th row of four experts plus each one's
    first and last row."""
    import torch

    nvq = _nvq()
    s = inputs.QAT
    log(f"[qat] full size {proj} guided={guided}: generating on device")
    logits = inputs.logits(s)
    ids, _ = nvq.nvq_moe_route(to_gpu(logits), s.topk)
    sp, off, _, _ = nvq.nvq_moe_permute(ids, s.E)
    K, N = (s.H, 2 * s.I) if proj == "gu" else (s.I, s.H)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77 if proj == "gu" else 78)
    if proj == "gu":
        x = torch.randn(s.T, K, generator=gen, device="cuda").to(torch.bfloat16)
        a_row = (sp // s.topk).to(torch.int32).contiguous()
    else:
        x = torch.randn(s.P, K, generator=gen, device="cuda").to(torch.bfloat16)
        a_row = None
    dy = torch.randn(s.P, N, generator=gen, device="cuda").to(torch.bfloat16)
    wm = inputs.weights_device(s, proj)
    q = nvq.nvfp4_quantize(wm)
    wd = None
    if guided:
        rec = nvq.nvfp4_guidance_record(q[0], nvq.NVQ_GUIDE_MANTISSA)
        wd = inputs.drift_device(wm, s, proj)
        codes = nvq.nvfp4_guided_quantize(wd, rec, q[1], q[2], nvq.NVQ_GUIDE_MANTISSA)
        del rec
    else:
        codes = q[0]
    rec_w = (codes, q[1], q[2])
    yb, yf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *rec_w, off, s.P, x=x, a_row=a_row,
                                         want_f32=True)
    dxb, dxf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *rec_w, off, s.P, dy=dy, want_f32=True)
    dxb_only = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *rec_w, off, s.P, dy=dy)[0]
    dw = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *rec_w, off, s.P, x=x, dy=dy, a_row=a_row)
    torch.cuda.synchronize()
    assert_bits_equal(to_np(dxb_only), to_np(dxb), "dx bf16 without the fp32 output")
    del dxb_only
    offn = to_np(off)
    x_of_row = to_np(sp) // s.topk if proj == "gu" else np.arange(s.P)
    xn = to_np(x)
    X = inputs.bf16_bits_to_f32(xn).astype(np.float64)
    for e in (0, 37, 90, 127):
        rows = np.arange(offn[e], offn[e + 1])
        if rows.size == 0:
            continue
        samp = np.unique(np.concatenate([rows[::97], rows[-1:]]))
        # the oracle builds the record itself from the expert's master weights
        wmb = to_np(wm[e])
        oq = oracle.quantize(wmb)
        assert_bits_equal(to_np(q[0][e]), oq[0], f"{proj} cache codes e={e}")
        assert float(to_np(q[2])[e]) == oq[2]
        ocodes = oq[0]
        if guided:
            orec = oracle.guidance_record(oq[0], oq[1], oq[2], oracle.GUIDE_MANTISSA)
            ocodes = oracle.guided_quantize(to_np(wd[e]), orec, oq[1], oq[2], oracle.GUIDE_MANTISSA)
            assert_bits_equal(to_np(codes[e]), ocodes, f"{proj} guided codes e={e}")
        W = oracle.dequantize(ocodes, oq[1], oq[2]).astype(np.float64)
        cols = np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
        ref = oracle.qat_fwd(xn, x_of_row[samp], np.zeros(samp.size, np.int32), ocodes, oq[1],
                             np.float32(oq[2]), cols=cols)
        _norm_err(to_np(yf)[samp][:, cols], ref, np.linalg.norm(X[x_of_row[samp]], axis=1),
                  np.linalg.norm(W[cols], axis=1), f"full {proj} fwd e={e}")
        dyn = to_np(dy[samp])
        cc = np.unique(np.concatenate([np.arange(0, K, 31), [K - 1]]))
        refd = oracle.qat_dgrad(dyn, np.arange(samp.size), np.zeros(samp.size, np.int32), ocodes,
                                oq[1], np.float32(oq[2]), cols=cc)
        DY = inputs.bf16_bits_to_f32(dyn).astype(np.float64)
        _norm_err(to_np(dxf)[samp][:, cc], refd, np.linalg.norm(DY, axis=1),
                  np.linalg.norm(W[:, cc], axis=0), f"full {proj} dgrad e={e}")
        ns = np.unique(np.concatenate([np.arange(0, N, 211), [N - 1]]))
        cs = np.unique(np.concatenate([np.arange(0, K, 223), [K - 1]]))
        nn, ccw = np.meshgrid(ns, cs, indexing="ij")
        dye = to_np(dy[offn[e]:offn[e + 1]])
        refw = oracle.qat_wgrad(dye, xn, x_of_row[rows], 0, rows.size, nn.ravel(), ccw.ravel())
        DYe = inputs.bf16_bits_to_f32(dye).astype(np.float64)
        Xe = X[x_of_row[rows]]
        _norm_err(to_np(dw[e])[np.ix_(ns, cs)], refw.reshape(ns.size, cs.size),
                  np.linalg.norm(DYe[:, ns], axis=0), np.linalg.norm(Xe[:, cs], axis=0),
                  f"full {proj} wgrad e={e}")
    # the bf16 outputs are the fp32 ones rounded
    rs = np.arange(0, s.P, 1013)
    assert_bits_equal(to_np(yb[rs]), inputs.to_bf16_bits(to_np(yf[rs])), f"{proj} fwd bf16")
    assert_bits_equal(to_np(dxb[rs]), inputs.to_bf16_bits(to_np(dxf[rs])), f"{proj} dgrad bf16")
    del wm, wd, q, codes, dw, x, dy
    torch.cuda.empty_cache()


def test_qat_no_rows():
    """No rows: forward and input gradient succeed with empty outputs; the
    weight gradient is zero, or unchanged with accumulate."""
    import torch

    nvq = _nvq()
    E, N, K = 3, 64, 128
    g = np.random.default_rng(5)
    wm = inputs.to_bf16_bits((0.02 * g.standard_normal((E, N, K))).astype(np.float32))
    q = nvq.nvfp4_quantize(to_gpu(wm))
    off = to_gpu(np.zeros(E + 1, np.int32))
    x = torch.empty(0, K, dtype=torch.bfloat16, device="cuda")
    dy = torch.empty(0, N, dtype=torch.bfloat16, device="cuda")
    yb, yf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *q[:3], off, 0, x=x, want_f32=True)
    dxb, dxf = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *q[:3], off, 0, dy=dy, want_f32=True)
    dw = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *q[:3], off, 0, x=x, dy=dy,
                                      dw=torch.full((E, N, K), 7.0, device="cuda"))
    dw2 = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *q[:3], off, 0, x=x, dy=dy,
                                       dw=torch.full((E, N, K), 7.0, device="cuda"), accumulate=True)
    torch.cuda.synchronize()
    assert yf.shape == (0, N) and dxf.shape == (0, K)
    assert not to_np(dw).any(), "weight gradient of no rows not zero"
    assert (to_np(dw2) == 7.0).all(), "accumulated weight gradient of no rows changed"

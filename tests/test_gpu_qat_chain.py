"""GPU parity of the chained QAT backward's glue (QUADS explainer §2.2-A: the
trainer's identity straight-through backward through the MoE layer):
nvq_swiglu_forward / nvq_swiglu_backward and nvq_moe_combine_backward against
the oracle, then the whole layer backward on a small MoE shape, every stage run
on the GPU from the oracle's own inputs to that stage and checked against the
oracle (the GEMM stages with the GEMM tolerance), plus the GPU's own chain
end to end."""
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


def _f(b):
    return inputs.bf16_bits_to_f32(b).astype(np.float64)


def _bf(x):
    return inputs.to_bf16_bits(np.asarray(x, np.float64).astype(np.float32))


def _check_swiglu_bwd(got_bits, ref, y1f, dh, what):
    I = ref.shape[1] // 2
    g, u, d = y1f[:, :I], y1f[:, I:], _f(dh)
    got = _f(got_bits)
    tol_g = 2.0 ** -8 * np.abs(ref[:, :I]) + 2.0 ** -18 * np.abs(d * u) * (1 + np.abs(g))
    tol_u = 2.0 ** -8 * np.abs(ref[:, I:]) + 2.0 ** -18 * np.abs(d * g)
    bad_g = np.abs(got[:, :I] - ref[:, :I]) > tol_g
    bad_u = np.abs(got[:, I:] - ref[:, I:]) > tol_u
    assert not bad_g.any() and not bad_u.any(), (what, np.argwhere(bad_g)[:3], np.argwhere(bad_u)[:3])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,I", [(1, 8), (37, 136), (256, 768)])
def test_swiglu_forward_and_backward(rows, I, dtype):
    nvq = _nvq()
    g = np.random.default_rng(rows + I)
    y1 = (g.standard_normal((rows, 2 * I)) * np.exp(g.uniform(-2, 2, (rows, 1)))).astype(np.float32)
    y1[:, :I][g.random((rows, I)) < 0.02] = np.float32(-95.0)  # exp(-g) overflows: gradients 0
    y1[:, :I][g.random((rows, I)) < 0.02] = np.float32(60.0)
    y1[:, :I][g.random((rows, I)) < 0.02] = np.float32(0.0)
    if dtype == "bf16":
        y1 = inputs.to_bf16_bits(y1)
    dh = inputs.to_bf16_bits(g.standard_normal((rows, I)).astype(np.float32))
    yg = to_gpu(y1)
    h = to_np(nvq.nvq_swiglu_forward(yg))
    dy1 = to_np(nvq.nvq_swiglu_backward(yg, to_gpu(dh)))
    y1f = _f(y1) if dtype == "bf16" else y1.astype(np.float64)
    href = oracle.swiglu_bf16(y1f)
    np.testing.assert_allclose(_f(h), _f(href), rtol=2 ** -7, atol=1e-30)
    _check_swiglu_bwd(dy1, oracle.swiglu_backward(y1, dh), y1f, dh, f"swiglu bwd {rows}x{I} {dtype}")


def _route(s):
    oids, ow = oracle.route(inputs.logits(s), s.topk)
    osp, ooff, opos = oracle.permute(oids, s.E)
    return oids, ow, osp, ooff, opos


@pytest.mark.parametrize("N", [64, 2048, 4104])
def test_combine_backward(N):
    import torch

    nvq = _nvq()
    s = inputs.small_moe(wid=104, T=133, E=7, topk=3)
    oids, ow, osp, ooff, opos = _route(s)
    g = np.random.default_rng(N)
    y = inputs.to_bf16_bits(g.standard_normal((s.P, N)).astype(np.float32))
    dout = inputs.to_bf16_bits(g.standard_normal((s.T, N)).astype(np.float32))
    dy, dw = nvq.nvq_moe_combine_backward(to_gpu(dout), to_gpu(opos), to_gpu(ow), s.P, y=to_gpu(y))
    dy_only, none = nvq.nvq_moe_combine_backward(to_gpu(dout), to_gpu(opos), to_gpu(ow), s.P,
                                                 want_dw=False)
    torch.cuda.synchronize()
    rdy, rdw = oracle.combine_backward(dout, y, opos, ow)
    assert_bits_equal(to_np(dy), rdy, "dy")
    assert_bits_equal(to_np(dy_only), rdy, "dy without dw")
    assert none is None
    D, Y = _f(dout), _f(y)
    den = np.linalg.norm(D, axis=1)[:, None] * np.linalg.norm(Y[opos.reshape(s.T, s.topk)], axis=2)
    err = np.abs(to_np(dw) - rdw) / np.maximum(den, 1e-30)
    log(f"[chain] combine bwd N={N}: dw max normalized err {err.max():.3e}")
    assert err.max() <= TOL


def _norm_err(got, ref, an, bn, what):
    err = np.abs(got.astype(np.float64) - ref) / np.maximum(np.outer(an, bn), 1e-30)
    log(f"[chain] {what}: max normalized err {err.max():.3e}")
    assert err.max() <= TOL, (what, err.max())


def test_chained_layer_backward_small():
    """Forward X -> Y1 = X W_gu^T -> H = swiglu(Y1) -> Y2 = H W_dn^T -> out =
    combine(Y2); backward from a seeded dOut through combine, down (input and
    weight gradients), SwiGLU, gate/up, and the token sum of the pair
    gradients.  The oracle runs the chain in fp64, rounding to bf16 where the
    GPU stores bf16; each GPU stage takes the oracle's input to that stage."""
    import torch

    nvq = _nvq()
    s = inputs.small_moe(wid=105, T=96, H=256, E=6, I=128, topk=2)
    oids, ow, osp, ooff, opos = _route(s)
    row_tok = (osp // s.topk).astype(np.int32)
    row_e = np.repeat(np.arange(s.E), np.diff(ooff)).astype(np.int32)
    g = np.random.default_rng(7)
    x = inputs.activations(s)
    dout = inputs.to_bf16_bits(g.standard_normal((s.T, s.H)).astype(np.float32))
    rec = {}
    for proj in ("gu", "dn"):
        wm = inputs.weights(s, proj)
        q = [oracle.quantize(wm[e]) for e in range(s.E)]
        rec[proj] = (np.stack([a[0] for a in q]), np.stack([a[1] for a in q]),
                     np.array([a[2] for a in q], np.float32))
    # the oracle's chain
    y1 = _bf(oracle.qat_fwd(x, row_tok, row_e, *rec["gu"]))
    h = oracle.swiglu_bf16(_f(y1))
    y2 = _bf(oracle.qat_fwd(h, np.arange(s.P), row_e, *rec["dn"]))
    dy2, dw = oracle.combine_backward(dout, y2, opos, ow)
    dh = _bf(oracle.qat_dgrad(dy2, np.arange(s.P), row_e, *rec["dn"]))
    dy1f = oracle.swiglu_backward(y1, dh)
    dy1 = _bf(dy1f)
    dxp = _bf(oracle.qat_dgrad(dy1, np.arange(s.P), row_e, *rec["gu"]))
    ones = np.ones((s.T, s.topk), np.float32)
    dx = oracle.combine_bf16(_f(dxp).astype(np.float32), opos, ones)
    # GPU stages on the oracle's inputs
    gq = {p: tuple(to_gpu(a) for a in rec[p]) for p in rec}
    off = to_gpu(ooff)
    h_g = nvq.nvq_swiglu_forward(to_gpu(y1))
    dy2_g, dw_g = nvq.nvq_moe_combine_backward(to_gpu(dout), to_gpu(opos), to_gpu(ow), s.P,
                                               y=to_gpu(y2))
    dh_g = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *gq["dn"], off, s.P, dy=to_gpu(dy2),
                                        want_f32=True)[1]
    dwdn_g = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *gq["dn"], off, s.P, x=to_gpu(h),
                                          dy=to_gpu(dy2))
    dy1_g = nvq.nvq_swiglu_backward(to_gpu(y1), to_gpu(dh))
    dxp_g = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *gq["gu"], off, s.P, dy=to_gpu(dy1),
                                         want_f32=True)[1]
    a_row = to_gpu(row_tok)
    dwgu_g = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *gq["gu"], off, s.P, x=to_gpu(x),
                                          dy=to_gpu(dy1), a_row=a_row)
    dx_g = nvq.nvq_moe_combine(to_gpu(dxp), to_gpu(opos), to_gpu(ones))
    torch.cuda.synchronize()
    np.testing.assert_allclose(_f(to_np(h_g)), _f(h), rtol=2 ** -7, atol=1e-30)
    assert_bits_equal(to_np(dy2_g), dy2, "dY2")
    D, Y2 = _f(dout), _f(y2)
    den = np.linalg.norm(D, axis=1)[:, None] * np.linalg.norm(Y2[opos.reshape(s.T, s.topk)], axis=2)
    assert (np.abs(to_np(dw_g) - dw) / np.maximum(den, 1e-30)).max() <= TOL
    _check_swiglu_bwd(to_np(dy1_g), dy1f, _f(y1), dh, "chain swiglu bwd")
    np.testing.assert_allclose(_f(to_np(dx_g)), _f(dx), rtol=2 ** -7, atol=1e-30)
    DY2, DY1, H, X = _f(dy2), _f(dy1), _f(h), _f(x)
    for e in range(s.E):
        rows = slice(ooff[e], ooff[e + 1])
        if ooff[e + 1] == ooff[e]:
            continue
        Wd = oracle.dequantize(rec["dn"][0][e], rec["dn"][1][e], rec["dn"][2][e]).astype(np.float64)
        Wg = oracle.dequantize(rec["gu"][0][e], rec["gu"][1][e], rec["gu"][2][e]).astype(np.float64)
        _norm_err(to_np(dh_g)[rows], oracle.qat_dgrad(dy2, np.arange(s.P), row_e, *rec["dn"])[rows],
                  np.linalg.norm(DY2[rows], axis=1), np.linalg.norm(Wd, axis=0), f"dH e={e}")
        _norm_err(to_np(dxp_g)[rows], oracle.qat_dgrad(dy1, np.arange(s.P), row_e, *rec["gu"])[rows],
                  np.linalg.norm(DY1[rows], axis=1), np.linalg.norm(Wg, axis=0), f"dXpairs e={e}")
        for name, dwg, dyb, ab, arow, N, K, a in (
                ("dW_dn", dwdn_g, dy2, h, np.arange(s.P), s.H, s.I, H),
                ("dW_gu", dwgu_g, dy1, x, row_tok, 2 * s.I, s.H, X)):
            nn, cc = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
            ref = oracle.qat_wgrad(dyb, ab, arow, ooff[e], ooff[e + 1], nn.ravel(), cc.ravel())
            _norm_err(to_np(dwg)[e], ref.reshape(N, K), np.linalg.norm(_f(dyb)[rows], axis=0),
                      np.linalg.norm(a[arow[rows]], axis=0), f"{name} e={e}")
    # the GPU's own chain end to end (reported; each stage is checked above)
    yg1 = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *gq["gu"], off, s.P, x=to_gpu(x), a_row=a_row)[0]
    hg = nvq.nvq_swiglu_forward(yg1)
    yg2 = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *gq["dn"], off, s.P, x=hg)[0]
    d2, _ = nvq.nvq_moe_combine_backward(to_gpu(dout), to_gpu(opos), to_gpu(ow), s.P, want_dw=False)
    dhh = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *gq["dn"], off, s.P, dy=d2)[0]
    d1 = nvq.nvq_swiglu_backward(yg1, dhh)
    dxx = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_DGRAD, *gq["gu"], off, s.P, dy=d1)[0]
    dxt = nvq.nvq_moe_combine(dxx, to_gpu(opos), to_gpu(ones))
    torch.cuda.synchronize()
    e2e = np.abs(_f(to_np(dxt)) - _f(dx)).max() / max(np.abs(_f(dx)).max(), 1e-30)
    log(f"[chain] GPU chain end to end: dX max |err| / max |dX| = {e2e:.3e}")
    assert e2e < 0.1


def test_glue_at_the_qat_layer_size_sampled():
    """SwiGLU forward/backward and the combine backward at the trainer layer's
    size (P = 131072 pairs, I = 1536, H = 4096) in the benchmark's launch
    configuration, checked on sampled rows and tokens."""
    import torch

    nvq = _nvq()
    s = inputs.QAT
    oids, ow, osp, ooff, opos = _route(s)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    y1 = (torch.randn(s.P, 2 * s.I, generator=g, device="cuda") * 2).to(torch.bfloat16)
    dh = torch.randn(s.P, s.I, generator=g, device="cuda").to(torch.bfloat16)
    y2 = torch.randn(s.P, s.H, generator=g, device="cuda").to(torch.bfloat16)
    dout = torch.randn(s.T, s.H, generator=g, device="cuda").to(torch.bfloat16)
    h = nvq.nvq_swiglu_forward(y1)
    dy1 = nvq.nvq_swiglu_backward(y1, dh)
    dy2, dw = nvq.nvq_moe_combine_backward(dout, to_gpu(opos), to_gpu(ow), s.P, y=y2)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, s.P, 1009), [s.P - 1]]))
    y1r, dhr = to_np(y1)[rows], to_np(dh)[rows]
    np.testing.assert_allclose(_f(to_np(h)[rows]), _f(oracle.swiglu_bf16(_f(y1r))), rtol=2 ** -7,
                               atol=1e-30)
    _check_swiglu_bwd(to_np(dy1)[rows], oracle.swiglu_backward(y1r, dhr), _f(y1r), dhr, "QAT-size")
    toks = np.unique(np.concatenate([np.arange(0, s.T, 331), [s.T - 1]]))
    pos2 = opos.reshape(s.T, s.topk)[toks]
    sub_pos = np.arange(toks.size * s.topk, dtype=np.int32)
    y2s = to_np(y2)[pos2.ravel()]
    rdy, rdw = oracle.combine_backward(to_np(dout)[toks], y2s, sub_pos, ow[toks])
    assert_bits_equal(to_np(dy2)[pos2.ravel()], rdy, "QAT-size dY2")
    D, Y = _f(to_np(dout)[toks]), _f(y2s).reshape(toks.size, s.topk, s.H)
    den = np.linalg.norm(D, axis=1)[:, None] * np.linalg.norm(Y, axis=2)
    assert (np.abs(to_np(dw)[toks] - rdw) / np.maximum(den, 1e-30)).max() <= TOL

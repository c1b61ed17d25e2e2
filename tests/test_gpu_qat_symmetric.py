"""The ablation variants of the QUADS explainer (§2.2-A asymmetric QAT against
its symmetric W4A4 alternative; §2.2-B compensation against naive W4A4), built
from the library's kernels and checked against the oracle:
  symmetric W4A4 QAT forward  Y = deq(q(X)) deq(qW)^T: NVFP4-quantized trainer
      activations through the W4A4 grouped GEMM with no compensation (k = 0);
  its weight gradient  dW = dY^T Xhat with Xhat = bf16(deq(q(X))) (identity
      straight-through estimator); the input gradient is the asymmetric one.
Tolerance |err| / (||a||_2 ||b||_2) <= 2e-3 as for every GEMM here, with a the
pre-quantization activation row for the forward."""
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
    log(f"[sym] {what}: max normalized err {worst:.3e} over {err.size} outputs")
    assert worst <= TOL, (what, worst)


@pytest.mark.parametrize("proj", ["gu", "dn"])
def test_symmetric_w4a4_qat_forward_and_weight_gradient(proj):
    import torch

    nvq = _nvq()
    s = inputs.small_moe(wid=103, T=150, H=256, E=5, I=128, topk=2)
    ids, _ = nvq.nvq_moe_route(to_gpu(inputs.logits(s)), s.topk)
    sp, off, _, _ = nvq.nvq_moe_permute(ids, s.E)
    K, N = (s.H, 2 * s.I) if proj == "gu" else (s.I, s.H)
    g = np.random.default_rng(77 + K)
    x = inputs.to_bf16_bits(g.standard_normal((s.T if proj == "gu" else s.P, K)).astype(np.float32))
    dy = inputs.to_bf16_bits(g.standard_normal((s.P, N)).astype(np.float32))
    wm = inputs.weights(s, proj)
    xg, dyg = to_gpu(x), to_gpu(dy)
    qw = nvq.nvfp4_quantize(to_gpu(wm))
    qx = nvq.nvfp4_quantize(xg)
    a_row = (sp // s.topk).to(torch.int32).contiguous() if proj == "gu" else None
    _, yf = nvq.moe_grouped_gemm_w4a4_comp(qx[0], qx[1], qx[2], qw[0], qw[1], qw[2], off, rows=s.P,
                                           a_row=a_row, want_bf16=False, want_f32=True)
    xhat = nvq.nvfp4_dequantize(qx[0], qx[1], qx[2], out_dtype=torch.bfloat16)
    dw = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *qw[:3], off, s.P, x=xhat, dy=dyg,
                                      a_row=a_row)
    torch.cuda.synchronize()
    # oracle: its own quantization of X and W, its own dequantized Xhat
    oqx = oracle.quantize(x)
    assert_bits_equal(to_np(qx[0]), oqx[0], "q(X) codes")
    oxhat = oracle.dequantize(*oqx, out="bf16")
    assert_bits_equal(to_np(xhat), oxhat, "Xhat")
    wq = [oracle.quantize(wm[e]) for e in range(s.E)]
    wc, wsc = np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq])
    wst = np.array([q[2] for q in wq], np.float32)
    offn = to_np(off)
    row_e = np.repeat(np.arange(s.E), np.diff(offn)).astype(np.int32)
    row_tok = to_np(sp) // s.topk if proj == "gu" else np.arange(s.P)
    ref_y = oracle.moe_gemm_w4a4(*oqx, x, None, wc, wsc, wst, row_tok, row_e)
    X = inputs.bf16_bits_to_f32(x).astype(np.float64)
    Xh = inputs.bf16_bits_to_f32(oxhat).astype(np.float64)
    DY = inputs.bf16_bits_to_f32(dy).astype(np.float64)
    y, dwn = to_np(yf), to_np(dw)
    for e in range(s.E):
        rows = slice(offn[e], offn[e + 1])
        if offn[e + 1] == offn[e]:
            continue
        W = oracle.dequantize(wc[e], wsc[e], wst[e]).astype(np.float64)
        _norm_err(y[rows], ref_y[rows], np.linalg.norm(X[row_tok[rows]], axis=1),
                  np.linalg.norm(W, axis=1), f"{proj} sym fwd e={e}")
        nn, cc = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
        ref_w = oracle.qat_wgrad(dy, oxhat, row_tok, offn[e], offn[e + 1], nn.ravel(), cc.ravel())
        _norm_err(dwn[e], ref_w.reshape(N, K), np.linalg.norm(DY[rows], axis=0),
                  np.linalg.norm(Xh[row_tok[rows]], axis=0), f"{proj} sym wgrad e={e}")
    # the asymmetric forward on the same X differs from the symmetric one by the
    # activation quantization error (the ablation's point), not by rounding
    yb_asym, yf_asym = nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_FWD, *qw[:3], off, s.P, x=xg,
                                                    a_row=a_row, want_f32=True)
    torch.cuda.synchronize()
    gap = np.abs(to_np(yf_asym).astype(np.float64) - y).max()
    assert gap > 1e-3, gap

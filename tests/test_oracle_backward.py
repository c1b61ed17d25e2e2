"""Pins of the oracle's backward glue for the chained QAT backward of the MoE
layer (QUADS explainer §2.2-A: the trainer's identity straight-through
backward through the layer): SwiGLU backward against finite differences of the
forward and its closed-form special cases; combine backward against numpy's
fp32 product and torch's bf16 rounding, brute force and the adjoint identity."""
import numpy as np
import torch

import oracle
from qat_nvfp4_quantize_amd import inputs


def _silu_u(g, u):
    return g / (1.0 + np.exp(-g)) * u


def test_swiglu_backward_matches_finite_differences():
    g = np.random.default_rng(0)
    rows, I = 16, 40
    y1 = (g.standard_normal((rows, 2 * I)) * 3).astype(np.float32)
    dh = inputs.to_bf16_bits(g.standard_normal((rows, I)).astype(np.float32))
    got = oracle.swiglu_backward(y1, dh)
    G = y1[:, :I].astype(np.float64)
    U = y1[:, I:].astype(np.float64)
    D = inputs.bf16_bits_to_f32(dh).astype(np.float64)
    eg = 1e-6 * np.maximum(1.0, np.abs(G))
    eu = 1e-6 * np.maximum(1.0, np.abs(U))
    fd_g = (_silu_u(G + eg, U) - _silu_u(G - eg, U)) / (2 * eg) * D
    fd_u = (_silu_u(G, U + eu) - _silu_u(G, U - eu)) / (2 * eu) * D
    scale = np.abs(D) * (np.abs(U) + np.abs(G) + 1)
    assert np.all(np.abs(got[:, :I] - fd_g) <= 1e-7 * scale)
    assert np.all(np.abs(got[:, I:] - fd_u) <= 1e-7 * scale)


def test_swiglu_backward_special_values_and_bf16_input():
    # g = 0: silu'(0) = 1/2 and silu(0) = 0; g -> +inf: silu' -> 1, silu(g) -> g;
    # g -> -inf: both -> 0
    y1 = np.array([[0.0, 40.0, -40.0, 5.0, 3.0, 2.0]], np.float32)
    dh = inputs.to_bf16_bits(np.array([[2.0, 1.0, 1.0]], np.float32))
    d = oracle.swiglu_backward(y1, dh)
    assert d[0, 0] == 2.0 * 5.0 * 0.5 and d[0, 3] == 0.0
    assert abs(d[0, 1] - 3.0) < 1e-12 and abs(d[0, 4] - 40.0) < 1e-12
    assert abs(d[0, 2]) < 1e-14 and abs(d[0, 5]) < 1e-14
    # a bf16 pre-activation gives the same as its fp32 widening
    yb = inputs.to_bf16_bits(np.random.default_rng(1).standard_normal((4, 32)).astype(np.float32))
    dhb = inputs.to_bf16_bits(np.ones((4, 16), np.float32))
    np.testing.assert_array_equal(oracle.swiglu_backward(yb, dhb),
                                  oracle.swiglu_backward(inputs.bf16_bits_to_f32(yb), dhb))


def _combine_case(seed, T=9, topk=3, E=4, N=24):
    g = np.random.default_rng(seed)
    ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    _, _, pos = oracle.permute(ids, E)
    w = g.dirichlet(np.ones(topk), T).astype(np.float32)
    y = inputs.to_bf16_bits(g.standard_normal((T * topk, N)).astype(np.float32))
    dout = inputs.to_bf16_bits(g.standard_normal((T, N)).astype(np.float32))
    return pos.astype(np.int32), w, y, dout


def test_combine_backward_rounding_brute_force_and_adjoint():
    pos, w, y, dout = _combine_case(0)
    T, topk = w.shape
    N = dout.shape[1]
    dy, dw = oracle.combine_backward(dout, y, pos, w)
    D = inputs.bf16_bits_to_f32(dout)
    Y = inputs.bf16_bits_to_f32(y)
    # dy: numpy's correctly rounded fp32 product, then torch's bf16 rounding
    ref = np.zeros_like(dy)
    for t in range(T):
        for j in range(topk):
            prod = np.float32(w[t, j]) * D[t]  # fp32 * fp32 -> fp32, correctly rounded
            ref[pos[t * topk + j]] = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(dy, ref)
    # dw: brute force
    for t in range(T):
        for j in range(topk):
            p = pos[t * topk + j]
            assert dw[t, j] == sum(float(D[t, n]) * float(Y[p, n]) for n in range(N))
    # adjoint: <dout, sum_j w y[pos]> = sum w dw
    lhs = sum(float(np.dot(D[t].astype(np.float64),
                           sum(np.float64(w[t, j]) * Y[pos[t * topk + j]].astype(np.float64)
                               for j in range(topk)))) for t in range(T))
    assert abs(lhs - float((w.astype(np.float64) * dw).sum())) <= 1e-9 * max(1.0, abs(lhs))


def test_combine_backward_skips_dropped_pairs():
    pos, w, y, dout = _combine_case(1)
    pos = pos.copy()
    pos[4] = -1
    dy, dw = oracle.combine_backward(dout, y, pos, w)
    assert dw.ravel()[4] == 0.0

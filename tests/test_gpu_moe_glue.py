"""GPU parity of the MoE glue: routing (bit-exact expert ids, softmax weights
within fp32 rounding), the stable permutation (bit-exact) and the combine."""
import numpy as np
import pytest

import oracle
from helpers import assert_bits_equal, log, to_gpu, to_np
from qat_nvfp4_quantize_amd import inputs

pytestmark = pytest.mark.gpu


def _nvq():
    from qat_nvfp4_quantize_amd import nvq

    return nvq


@pytest.mark.parametrize("shape", ["small", "decode", "prefill"])
def test_route_and_permute(shape):
    import torch

    nvq = _nvq()
    s = {"small": inputs.small_moe(), "decode": inputs.DECODE, "prefill": inputs.PREFILL}[shape]
    log(f"[route] {shape} T={s.T} E={s.E} topk={s.topk}")
    logits = inputs.logits(s)
    ids, w = nvq.nvq_moe_route(to_gpu(logits), s.topk)
    oids, ow = oracle.route(logits, s.topk)
    assert_bits_equal(to_np(ids), oids, "ids")
    np.testing.assert_allclose(to_np(w), ow, rtol=4e-7, atol=0)
    sp, off, pos, ws = nvq.nvq_moe_permute(ids, s.E)
    torch.cuda.synchronize()
    osp, ooff, opos = oracle.permute(oids, s.E)
    assert_bits_equal(to_np(off), ooff, "offsets")
    assert_bits_equal(to_np(sp), osp, "sorted_pair")
    assert_bits_equal(to_np(pos), opos, "pos")
    assert nvq.device_status(ws) == 0


@pytest.mark.parametrize("T,topk,E", [(5000, 4, 300), (8192, 8, 1024), (16384, 4, 128), (16385, 4, 128),
                                     (1, 1, 7), (20000, 4, 300), (9000, 8, 1024), (33000, 2, 7)])
def test_permute_chunk_counts_and_wide_expert_sets(T, topk, E):
    """The permutation with the scatter deriving its own bases (at most 64
    chunks of 1024 pairs) and with the scan kernel (65 chunks and more):
    expert counts above one per thread (E = 300, 1024), the 64 / 65 chunk
    boundary, a single pair; the scan with expert counts that do not divide
    its 1024 threads (E = 300, 7) and with one thread per expert (E = 1024);
    skewed ids leave experts empty."""
    nvq = _nvq()
    g = np.random.default_rng(T + E)
    ids = np.minimum(g.zipf(1.3, (T, topk)) - 1, E - 1).astype(np.int32)
    log(f"[permute] T={T} topk={topk} E={E} chunks={(T * topk + 1023) // 1024}")
    sp, off, pos, ws = nvq.nvq_moe_permute(to_gpu(ids), E)
    osp, ooff, opos = oracle.permute(ids, E)
    assert_bits_equal(to_np(off), ooff, "offsets")
    assert_bits_equal(to_np(sp), osp, "sorted_pair")
    assert_bits_equal(to_np(pos), opos, "pos")
    assert nvq.device_status(ws) == 0


def test_route_ties_and_negative_zero():
    nvq = _nvq()
    g = np.random.default_rng(3)
    logits = np.round(g.standard_normal((300, 64))).astype(np.float32)
    logits[:, 5] = -0.0
    logits[:, 9] = 0.0
    ids, w = nvq.nvq_moe_route(to_gpu(logits), 8)
    oids, ow = oracle.route(logits, 8)
    assert_bits_equal(to_np(ids), oids, "ids with ties")
    np.testing.assert_allclose(to_np(w), ow, rtol=4e-7, atol=0)


def test_permute_empty_experts_and_bad_ids():
    nvq = _nvq()
    g = np.random.default_rng(4)
    T, topk, E = 777, 3, 40
    ids = g.integers(0, 10, (T, topk)).astype(np.int32)  # experts 10..39 empty
    sp, off, pos, ws = nvq.nvq_moe_permute(to_gpu(ids), E)
    osp, ooff, opos = oracle.permute(ids, E)
    assert_bits_equal(to_np(off), ooff, "offsets")
    assert_bits_equal(to_np(sp), osp, "sorted_pair")
    assert_bits_equal(to_np(pos), opos, "pos")
    bad = ids.copy()
    bad[5, 1] = E + 3
    _, _, pos2, ws2 = nvq.nvq_moe_permute(to_gpu(bad), E)
    assert nvq.device_status(ws2) & nvq.NVQ_STATUS_BAD_EXPERT
    assert to_np(pos2)[5 * topk + 1] == -1


def test_combine_matches_oracle():
    nvq = _nvq()
    s = inputs.small_moe()
    logits = inputs.logits(s)
    oids, ow = oracle.route(logits, s.topk)
    _, _, opos = oracle.permute(oids, s.E)
    g = np.random.default_rng(5)
    y = inputs.to_bf16_bits(g.standard_normal((s.P, 64)).astype(np.float32))
    out = nvq.nvq_moe_combine(to_gpu(y), to_gpu(opos), to_gpu(ow))
    ref = oracle.combine_bf16(inputs.bf16_bits_to_f32(y), opos, ow)
    got = inputs.bf16_bits_to_f32(to_np(out))
    np.testing.assert_allclose(got, inputs.bf16_bits_to_f32(ref), rtol=2 ** -7, atol=1e-6)


def test_no_tokens():
    """T = 0: routing and combine do nothing, the permutation writes all-zero
    expert offsets."""
    import torch

    nvq = _nvq()
    E, topk, H = 16, 4, 64
    ids, w = nvq.nvq_moe_route(torch.empty(0, E, dtype=torch.float32, device="cuda"), topk)
    sp, off, pos, _ = nvq.nvq_moe_permute(ids, E)
    out = nvq.nvq_moe_combine(torch.empty(0, H, dtype=torch.bfloat16, device="cuda"), pos, w)
    torch.cuda.synchronize()
    assert ids.shape == (0, topk) and sp.numel() == 0 and out.shape[0] == 0
    assert_bits_equal(to_np(off), np.zeros(E + 1, np.int32), "offsets of no tokens")


@pytest.mark.parametrize("topk,N", [(3, 64), (8, 4096), (9, 72)])
def test_combine_with_dropped_pairs(topk, N):
    """Pairs the permutation dropped (pos = -1) are left out of the combine,
    through the all-loads-first kernel (topk <= 8) and the general one."""
    nvq = _nvq()
    g = np.random.default_rng(topk * 1000 + N)
    T, E = 300, 16
    ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    ids[g.random((T, topk)) < 0.05] = E + 1  # dropped
    sp, off, pos, _ = nvq.nvq_moe_permute(to_gpu(ids), E)
    opos = to_np(pos)
    assert (opos < 0).any()
    P = int(to_np(off)[-1])
    y = inputs.to_bf16_bits(g.standard_normal((P, N)).astype(np.float32))
    w = g.random((T, topk)).astype(np.float32)
    out = nvq.nvq_moe_combine(to_gpu(y), pos, to_gpu(w))
    ref = oracle.combine_bf16(inputs.bf16_bits_to_f32(y), opos, w)
    np.testing.assert_allclose(inputs.bf16_bits_to_f32(to_np(out)), inputs.bf16_bits_to_f32(ref),
                               rtol=2 ** -7, atol=1e-6)


@pytest.mark.parametrize("topk,N,T", [(8, 2048, 333), (9, 80, 50), (2, 16, 1)])
def test_combine_records_the_amax_of_its_output(topk, N, T):
    """out_amax = max |out| over the stored bf16 output (both combine
    kernels, ragged last vectors), and quantizing out with it as amax_in gives
    the same record and scores as quantizing with its own amax pass."""
    import torch

    nvq = _nvq()
    g = np.random.default_rng(topk * 7 + N + T)
    E = 16
    ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    sp, off, pos, _ = nvq.nvq_moe_permute(to_gpu(ids), E)
    P = int(to_np(off)[-1])
    y = inputs.to_bf16_bits((g.standard_t(3, (P, N)) * 3).astype(np.float32))
    w = g.random((T, topk)).astype(np.float32)
    amax = torch.full((1,), 123.0, dtype=torch.float32, device="cuda")  # overwritten
    out = nvq.nvq_moe_combine(to_gpu(y), pos, to_gpu(w), out_amax=amax)
    q_own = nvq.nvfp4_quantize(out, score=True)
    q_in = nvq.nvfp4_quantize(out, amax_in=amax, score=True)
    torch.cuda.synchronize()
    outf = inputs.bf16_bits_to_f32(to_np(out))
    assert float(to_np(amax)[0]) == float(np.abs(outf).max())
    for a, b, what in zip(q_own[:4], q_in[:4], ("codes", "scales", "s_t", "scores")):
        assert_bits_equal(to_np(b), to_np(a), f"quantize with the combine's amax: {what}")
    # no tokens: the maximum of nothing is 0
    empty = nvq.nvq_moe_combine(torch.empty(0, N, dtype=torch.bfloat16, device="cuda"),
                                torch.empty(0, dtype=torch.int32, device="cuda"),
                                torch.empty(0, topk, dtype=torch.float32, device="cuda"),
                                out_amax=amax)
    torch.cuda.synchronize()
    assert empty.shape == (0, N) and float(to_np(amax)[0]) == 0.0

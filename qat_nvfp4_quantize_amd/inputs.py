"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
quantization, routing or GEMM arithmetic.  Every tensor comes from its own
numpy ``Generator(PCG64(SeedSequence([seed, workload_id, tensor_id, ...])))``
stream, so any tensor (or any single expert's weights) can be regenerated
alone.  bf16 tensors are returned as uint16 bit patterns: fp32 draws rounded
to nearest even by torch's CPU conversion.

Workloads (MoE shapes stand in for the 25B/2.8B-active MoE of the QUADS
explainer §4 and the MoE models of the TRACE post; the pages give no layer
shapes):
  1 dense    X 64x256 f32 N(0,1) with 4 seeded outlier columns x20;
             W [K=256, N=128] f32 N(0, 0.02^2), stored transposed [N, K]; k = 8.
  2 quant    X 8192x7168 bf16, Student-t (nu = 4), 36 (0.5%) seeded
             channels x50.
  3 decode   T=4096, H=2048, E=128, I=768, top-8, N(0,1) logits, X bf16 N(0,1),
             W_gu [E, 2I, H], W_dn [E, H, I] bf16 N(0, 0.02^2); k = 64.
  4 prefill  T=32768, H=4096, E=128, I=1536, top-8, k = 128; Zipf(1.1) expert
             popularity via logits = log p_e + Gumbel(0,1), p_e ~ (e+1)^-1.1;
             weights N(0, 0.02^2) with 1% of each expert's K-channels x10.
  5 qat      T=16384, H=4096, E=128, I=1536, top-8, N(0,1) logits; bf16 master
             weights N(0, 0.02^2); X and per-projection dY bf16 N(0,1).
             Drifted masters for the rollout-guided rounding (TRACE post): the
             bf16 master plus an independent N(0, 0.002^2) draw (a tenth of the
             weights' spread; the pages give no step size), rounded to bf16.
  6 kv       FP4 KV cache of one attention layer (TRACE post: FP4 KV cache in
             the rollout): K and V [B * Hkv * S, D] with B=64 sequences, Hkv=8
             KV heads, S=4096 positions, D=128 (16-element blocks along the head
             dimension), bf16 N(0,1), K with 2 seeded head-dim channels x10;
             a decode step appends B * Hkv rows per tensor, N(0, 1.5^2) with 1%
             of the elements x30.  The
             cache keeps a static tensor scale: amax 42 = 2688 * 2^-6.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BASE_SEED = 0


def rng(*ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *ids])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 draws -> bf16 bit patterns (round to nearest even, torch CPU)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class MoEShape:
    wid: int
    T: int
    H: int
    E: int
    I: int
    topk: int
    k: int

    @property
    def P(self) -> int:
        return self.T * self.topk


DECODE = MoEShape(wid=3, T=4096, H=2048, E=128, I=768, topk=8, k=64)
PREFILL = MoEShape(wid=4, T=32768, H=4096, E=128, I=1536, topk=8, k=128)
QAT = MoEShape(wid=5, T=16384, H=4096, E=128, I=1536, topk=8, k=0)

# tensor ids within a workload
_X, _W, _OUTLIER, _LOGITS, _WGU, _WDN, _DYGU, _DYDN, _WOUT, _HID, _DRIFT = range(11)

DRIFT_STD = 0.002


# ------------------------------------------------------------- workload 1 --
def dense_check(M=64, K=256, N=128, n_outlier=4, outlier_scale=20.0, w_std=0.02, wid=1):
    """Returns (x f32 [M, K], w f32 [N, K] (the [K, N] draw transposed), k)."""
    x = rng(wid, _X).standard_normal((M, K), dtype=np.float32)
    cols = rng(wid, _OUTLIER).permutation(K)[:n_outlier]
    x[:, cols] *= np.float32(outlier_scale)
    w_kn = (rng(wid, _W).standard_normal((K, N), dtype=np.float32) * np.float32(w_std))
    return x, np.ascontiguousarray(w_kn.T), 8


# ------------------------------------------------------------- workload 2 --
def quant_sweep(M=8192, K=7168, frac=0.005, scale=50.0, nu=4.0, wid=2):
    """bf16 bits [M, K]: Student-t draws, round(frac*K) seeded channels x scale."""
    x = rng(wid, _X).standard_t(nu, size=(M, K)).astype(np.float32)
    n = int(round(frac * K))
    cols = rng(wid, _OUTLIER).permutation(K)[:n]
    x[:, cols] *= np.float32(scale)
    return to_bf16_bits(x)


# ---------------------------------------------------------- MoE workloads --
def logits(s: MoEShape) -> np.ndarray:
    g = rng(s.wid, _LOGITS)
    if s.wid == PREFILL.wid:
        p = (np.arange(1, s.E + 1, dtype=np.float64)) ** -1.1
        p /= p.sum()
        gumbel = g.gumbel(0.0, 1.0, size=(s.T, s.E))
        return (np.log(p)[None, :] + gumbel).astype(np.float32)
    return g.standard_normal((s.T, s.E), dtype=np.float32)


def activations(s: MoEShape) -> np.ndarray:
    """bf16 bits [T, H], N(0,1)."""
    return to_bf16_bits(rng(s.wid, _X).standard_normal((s.T, s.H), dtype=np.float32))


def expert_weight_f32(s: MoEShape, proj: str, e: int) -> np.ndarray:
    """fp32 draw of one expert's weight, [N, K] with K contiguous.

    proj 'gu': [2I, H] (gate rows first, then up); 'dn': [H, I]."""
    tid = _WGU if proj == "gu" else _WDN
    N, K = (2 * s.I, s.H) if proj == "gu" else (s.H, s.I)
    w = rng(s.wid, tid, e).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    if s.wid == PREFILL.wid:
        n_out = max(1, int(round(0.01 * K)))
        cols = rng(s.wid, _WOUT, tid, e).permutation(K)[:n_out]
        w[:, cols] *= np.float32(10.0)
    return w


def expert_weight(s: MoEShape, proj: str, e: int) -> np.ndarray:
    """bf16 bits of one expert's weight [N, K]."""
    return to_bf16_bits(expert_weight_f32(s, proj, e))


def weights(s: MoEShape, proj: str, experts=None) -> np.ndarray:
    """bf16 bits [len(experts), N, K] (all experts by default)."""
    experts = range(s.E) if experts is None else experts
    return np.stack([expert_weight(s, proj, e) for e in experts])


def grad_out(s: MoEShape, proj: str) -> np.ndarray:
    """bf16 bits [P, N] upstream gradient of one projection, sorted-pair rows."""
    tid = _DYGU if proj == "gu" else _DYDN
    N = 2 * s.I if proj == "gu" else s.H
    return to_bf16_bits(rng(s.wid, tid).standard_normal((s.P, N), dtype=np.float32))


def hidden(s: MoEShape) -> np.ndarray:
    """bf16 bits [P, I]: a stand-in for the down projection's input (the SwiGLU
    output), drawn independently of the gate/up path: N(0,1) with 1% of the
    channels x8."""
    g = rng(s.wid, _HID)
    h = g.standard_normal((s.P, s.I), dtype=np.float32)
    cols = g.permutation(s.I)[: max(1, int(round(0.01 * s.I)))]
    h[:, cols] *= np.float32(8.0)
    return to_bf16_bits(h)


def small_moe(wid=100, T=96, H=256, E=8, I=128, topk=2, k=16) -> MoEShape:
    """A reduced MoE shape for fast parity tests (several tiles plus ragged tails)."""
    return MoEShape(wid=wid, T=T, H=H, E=E, I=I, topk=topk, k=k)


def weights_device(s: MoEShape, proj: str, device="cuda"):
    """bf16 [E, N, K] expert weights drawn on the GPU (torch Philox generator,
    seeded per workload and tensor): same recipe as expert_weight_f32, another
    random stream, for the full-size layers (the parity tests copy the sampled
    experts to the host for the oracle)."""
    import torch

    tid = _WGU if proj == "gu" else _WDN
    N, K = (2 * s.I, s.H) if proj == "gu" else (s.H, s.I)
    g = torch.Generator(device=device)
    g.manual_seed(BASE_SEED * 1_000_003 + s.wid * 1009 + tid)
    w = torch.empty(s.E, N, K, dtype=torch.bfloat16, device=device)
    for e in range(s.E):
        we = torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * 0.02
        if s.wid == PREFILL.wid:
            n_out = max(1, int(round(0.01 * K)))
            cols = torch.randperm(K, generator=g, device=device)[:n_out]
            we[:, cols] *= 10.0
        w[e] = we.to(torch.bfloat16)
    return w


def drifted_expert_weight(s: MoEShape, proj: str, e: int) -> np.ndarray:
    """bf16 bits [N, K]: expert e's bf16 master plus its own N(0, DRIFT_STD^2)
    draw, rounded to bf16 (the master after the trainer's update)."""
    tid = _WGU if proj == "gu" else _WDN
    w = bf16_bits_to_f32(expert_weight(s, proj, e))
    d = rng(s.wid, _DRIFT, tid, e).standard_normal(w.shape, dtype=np.float32)
    return to_bf16_bits(w + d * np.float32(DRIFT_STD))


def drift_device(w, s: MoEShape, proj: str):
    """bf16 [E, N, K]: the GPU-drawn masters w plus a seeded N(0, DRIFT_STD^2)
    draw (torch Philox stream of its own), rounded to bf16."""
    import torch

    tid = _WGU if proj == "gu" else _WDN
    g = torch.Generator(device=w.device)
    g.manual_seed(BASE_SEED * 1_000_003 + s.wid * 1009 + 100 + tid)
    out = torch.empty_like(w)
    for e in range(w.shape[0]):
        d = torch.randn(w.shape[1:], generator=g, device=w.device, dtype=torch.float32)
        out[e] = (w[e].float() + d * DRIFT_STD).to(torch.bfloat16)
    return out


KV_SHAPE = dict(B=64, Hkv=8, S=4096, D=128)
KV_STATIC_AMAX = 42.0  # 2688 * 2^-6: tensor scale 2^-6 exactly
_KV_K, _KV_V, _KV_OUT, _KV_NEW = range(4)


def kv_cache(B=64, Hkv=8, S=4096, D=128, wid=6, device=None):
    """bf16 [2, B*Hkv*S, D]: the K (item 0) and V (item 1) caches.  numpy bits
    on the host, or a torch bf16 tensor drawn on `device` (torch Philox
    stream seeded per workload; same recipe, another stream)."""
    rows = B * Hkv * S
    cols = rng(wid, _KV_OUT).permutation(D)[:2]
    if device is None:
        k = rng(wid, _KV_K).standard_normal((rows, D), dtype=np.float32)
        k[:, cols] *= np.float32(10.0)
        v = rng(wid, _KV_V).standard_normal((rows, D), dtype=np.float32)
        return np.stack([to_bf16_bits(k), to_bf16_bits(v)])
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(BASE_SEED * 1_000_003 + wid * 1009)
    out = torch.empty(2, rows, D, dtype=torch.bfloat16, device=device)
    for i in range(2):
        t = torch.randn(rows, D, generator=g, device=device, dtype=torch.float32)
        if i == 0:
            t[:, torch.from_numpy(cols).to(device)] *= 10.0
        out[i] = t.to(torch.bfloat16)
    return out


def kv_append(B=64, Hkv=8, D=128, wid=6, step=0):
    """bf16 bits [2, B*Hkv, D]: one decode step's new K and V rows, N(0, 1.5^2),
    with 1% of the elements x30 (some beyond the cache's static amax)."""
    g = rng(wid, _KV_NEW, step)
    x = g.standard_normal((2, B * Hkv, D), dtype=np.float32) * np.float32(1.5)
    x[g.random(x.shape) < 0.01] *= np.float32(30.0)
    return to_bf16_bits(x)

#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

One step = one pass of every measured leg over its seeded synthetic workload
(inputs already resident in HBM):
  quant   NVFP4 quantize of the 8192x7168 bf16 activation sweep (Student-t,
          0.5% outlier channels): amax, codes, E4M3 scales, tensor scale and
          per-channel residual sums, then the top-64 residual channels.
  moe     (when built) the MoE rollout layer with W4A4 grouped GEMMs and
          residual compensation.
  qat     (when built) the asymmetric W4A16 QAT layer forward + backward.

Prints ONE JSON line.  `value` is the quantizer's algorithmic GB/s (x read
once, codes + scales + scores written); the GEMM legs report TFLOP/s in
their own fields.  Kernel durations come from HIP events on the stream the
library launches on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16/fp16 MFMA
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--legs", default="quant,moe,qat")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


class EventTimer:
    """Accumulates event-timed durations per label on the current stream."""

    def __init__(self):
        import torch

        self.torch = torch
        self.pending = []
        self.total = {}
        self.count = {}

    def __call__(self, label, fn):
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        out = fn()
        b.record()
        self.pending.append((label, a, b))
        return out

    def collect(self):
        self.torch.cuda.synchronize()
        for label, a, b in self.pending:
            self.total[label] = self.total.get(label, 0.0) + a.elapsed_time(b)
            self.count[label] = self.count.get(label, 0) + 1
        self.pending = []

    def avg_ms(self, label):
        return self.total[label] / self.count[label]

    def reset(self):
        self.pending, self.total, self.count = [], {}, {}


# ------------------------------------------------------------------ legs --
class QuantLeg:
    name = "quant"

    def __init__(self):
        import torch

        from qat_nvfp4_quantize_amd import inputs, nvq

        self.nvq = nvq
        self.x_np = inputs.quant_sweep()
        M, K = self.x_np.shape
        self.M, self.K, self.k = M, K, 64
        self.x = torch.from_numpy(self.x_np.view(np.int16)).view(torch.bfloat16).cuda()
        dev = self.x.device
        self.out = (torch.empty(M, K // 2, dtype=torch.uint8, device=dev),
                    torch.empty(M, K // 16, dtype=torch.uint8, device=dev),
                    torch.empty(1, dtype=torch.float32, device=dev),
                    torch.empty(K, dtype=torch.float32, device=dev))
        L = nvq.load()
        self.ws = nvq.workspace(L.nvfp4_quantize_workspace_bytes(1, M, K), dev)
        self.ws2 = nvq.workspace(L.residual_topk_workspace_bytes(M, K, self.k), dev)
        # algorithmic bytes: read x once; write codes, scales, scores, s_t
        self.bytes = M * K * 2 + M * K // 2 + M * K // 16 + K * 4 + 4

    def step(self, timer):
        nvq = self.nvq
        codes, scales, st, score = self.out
        timer("quantize", lambda: nvq.nvfp4_quantize(self.x, score=True, ws=self.ws, out=self.out))
        timer("topk", lambda: nvq.residual_topk_channels(self.x, codes, scales, st, self.k,
                                                         scores=score, want_resid=False,
                                                         ws=self.ws2))

    def cpu_baseline(self):
        import oracle

        x = self.x_np
        t0 = time.perf_counter()
        oracle.quantize(x[:256])
        t0 = time.perf_counter()
        c, s, st = oracle.quantize(x)
        oracle.residual_scores(x, c, s, st)
        dt = time.perf_counter() - t0
        return {"value": round(self.bytes / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
                "kind": "oracle",
                "sample": "full 8192x7168 bf16 sweep tensor, one timed run of the fp64 "
                          "exhaustive-search quantizer + residual scores (%.1f s)" % dt}


class CopyLeg:
    """Plain elementwise copy of a known size: calibrates the FETCH_SIZE /
    WRITE_SIZE counters (and measures achievable HBM bandwidth)."""

    name = "copy"

    def __init__(self, nbytes=256 << 20):
        import torch

        self.src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.bytes = 2 * nbytes

    def step(self, timer):
        import torch

        timer("copy", lambda: torch.mul(self.src, 1.0, out=self.dst))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    os.environ.setdefault("ORACLE_THREADS", "16")
    legs = []
    wanted = args.legs.split(",")
    if "quant" in wanted:
        legs.append(QuantLeg())
    if "copy" in wanted:
        legs.append(CopyLeg())
    timer = EventTimer()
    for _ in range(args.warmup):
        for leg in legs:
            leg.step(timer)
    timer.collect()
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for leg in legs:
            leg.step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect()
    ms_step = wall * 1e3 / args.steps

    q = next(l for l in legs if l.name == "quant")
    q_ms = timer.avg_ms("quantize")
    gbs = q.bytes / (q_ms * 1e-3) / 1e9
    result = {
        "metric": "NVFP4 quantize GB/s + W4A4 MoE grouped-GEMM TFLOP/s (% of MI355X peak)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, e2m1/e4m3 out",
        "data": "synthetic",
        "config": {"workload": "quantizer sweep: bf16 activation 8192x7168, Student-t nu=4, "
                               "36 outlier channels x50; codes+scales+tensor scale+residual sums, "
                               "then top-64 channels"},
        "legs": {"quant": {"quantize_ms": round(q_ms, 5), "topk_ms": round(timer.avg_ms("topk"), 5),
                           "algorithmic_bytes": q.bytes}},
        "roofline": {"kernel": "nvfp4_quantize (amax + quantize + score-reduce kernels)",
                     "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if any(l.name == "copy" for l in legs):
        c = next(l for l in legs if l.name == "copy")
        result["legs"]["copy"] = {"ms": round(timer.avg_ms("copy"), 5), "bytes": c.bytes,
                                  "GBps": round(c.bytes / timer.avg_ms("copy") / 1e6, 1)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = q.cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

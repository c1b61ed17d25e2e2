#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

One step = one pass of every measured leg over its seeded synthetic workload
(inputs already resident in HBM):
  quant   NVFP4 quantize of the 8192x7168 bf16 activation sweep (Student-t,
          0.5% outlier channels): amax, codes, E4M3 scales, tensor scale and
          per-channel residual sums, then the top-64 residual channels.
  moe     (when built) the MoE rollout layer with W4A4 grouped GEMMs and
          residual compensation.
  qat     (when built) the asymmetric W4A16 QAT layer: codes of the drifted
          master weights rebuilt from the rollout's guidance record, then
          forward + backward.
  kv      FP4 KV cache: K/V caches of one attention layer quantized with a
          static tensor scale, dequantized to bf16, one decode step appended.

Prints ONE JSON line.  `value` is the quantizer's algorithmic GB/s (x read
once, codes + scales + scores written); the GEMM legs report TFLOP/s in
their own fields.  Kernel durations come from HIP events on the stream the
library launches on.
"""
from __future__ import annotations

import argparse
import json
import re
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


def host_cpu_info():
    """CPU model (from /proc/cpuinfo) and the CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        ncpu = os.cpu_count() or 1
    return model, ncpu


def oracle_thread_count():
    """Threads for the CPU baseline: ORACLE_THREADS if set, else the host's CPU
    share as the job environment states it (OMP_NUM_THREADS), else every CPU
    this process may run on."""
    for var in ("ORACLE_THREADS", "OMP_NUM_THREADS"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return int(v)
    return host_cpu_info()[1]


def timed_median(fn, runs=3, warm=None):
    """One warm-up call (of `warm` if given: a smaller call of the same code),
    then the median wall time of `runs` calls of fn."""
    (warm or fn)()
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2], sum(ts)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--legs", default="quant,moe,qat,kv")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quant-shape", default="8192x7168",
                   help="rows x K of the quantizer leg (the headline workload is 8192x7168; "
                        "other shapes are for tile-count studies)")
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

    def __init__(self, M=8192, K=7168):
        import torch

        from qat_nvfp4_quantize_amd import inputs, nvq

        self.nvq = nvq
        self.x_np = inputs.quant_sweep(M, K)
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
        oracle.quantize(x[:256])  # warm-up (library load, page-in)
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            c, s, st = oracle.quantize(x)
            oracle.residual_scores(x, c, s, st)
            runs.append(time.perf_counter() - t0)
        dt = sorted(runs)[1]
        model, ncpu = host_cpu_info()
        return {"value": round(self.bytes / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
                "kind": "oracle", "cpu_model": model, "host_cpus": ncpu,
                "sample": f"full {self.M}x{self.K} bf16 sweep tensor: fp64 exhaustive-search quantizer + "
                          "residual scores, median of 3 runs (%.2f s each, %.1f s in all)"
                          % (dt, sum(runs))}


class MoeLeg:
    """One W4A4 MoE layer with residual compensation: route, permute, quantize X
    (+ residual scores), top-k channels + residual columns, gate/up grouped GEMM
    with SwiGLU epilogue (which also records max |h|), quantize H with that
    amax (+ scores), top-k + residuals, down grouped
    GEMM, combine.  Expert weights are quantized (and their channel-major copy
    made) once outside the timed step
    (they are static during a rollout)."""

    def __init__(self, shape):
        import torch

        from qat_nvfp4_quantize_amd import inputs, nvq

        self.nvq = nvq
        s = self.s = shape
        self.name = "moe_%s" % ("decode" if s.wid == inputs.DECODE.wid else "prefill")
        dev = torch.device("cuda")
        log(f"[bench] {self.name}: generating inputs")
        self.logits = torch.from_numpy(inputs.logits(s)).to(dev)
        self.x = torch.from_numpy(inputs.activations(s).view(np.int16)).view(torch.bfloat16).to(dev)
        self.qw, self.wcm = {}, {}
        for proj in ("gu", "dn"):
            w = inputs.weights_device(s, proj, dev)
            codes, scales, st, _, _ = nvq.nvfp4_quantize(w)
            self.qw[proj] = (codes, scales, st)
            # channel-major copy for the compensation gather, made with the record
            self.wcm[proj] = nvq.nvfp4_channel_major(codes, scales)
            del w
        torch.cuda.synchronize()
        P, H, I, k = s.P, s.H, s.I, s.k
        u8, i32, f32, bf = torch.uint8, torch.int32, torch.float32, torch.bfloat16
        self.ids = torch.empty(s.T, s.topk, dtype=i32, device=dev)
        L = nvq.load()
        self.ws_perm = nvq.workspace(L.nvq_moe_permute_workspace_bytes(s.T, s.topk, s.E), dev)
        self.ws_q1 = nvq.workspace(L.nvfp4_quantize_workspace_bytes(1, s.T, H), dev)
        self.ws_q2 = nvq.workspace(L.nvfp4_quantize_workspace_bytes(1, P, I), dev)
        self.ws_t1 = nvq.workspace(L.residual_topk_workspace_bytes(s.T, H, k), dev)
        self.ws_t2 = nvq.workspace(L.residual_topk_workspace_bytes(P, I, k), dev)
        self.ws_g = nvq.workspace(max(L.moe_gemm_workspace_bytes(P, s.E, 2 * I, k),
                                      L.moe_gemm_workspace_bytes(P, s.E, H, k)), dev)
        self.qx = (torch.empty(s.T, H // 2, dtype=u8, device=dev), torch.empty(s.T, H // 16, dtype=u8, device=dev),
                   torch.empty(1, dtype=f32, device=dev), torch.empty(H, dtype=f32, device=dev))
        self.qh = (torch.empty(P, I // 2, dtype=u8, device=dev), torch.empty(P, I // 16, dtype=u8, device=dev),
                   torch.empty(1, dtype=f32, device=dev), torch.empty(I, dtype=f32, device=dev))
        self.h = torch.empty(P, I, dtype=bf, device=dev)
        # max |h|, produced by the gate/up epilogue and consumed as amax_in by
        # the quantization of h (which then skips its own amax pass)
        self.h_amax = torch.zeros(1, dtype=f32, device=dev)
        self.y2 = torch.empty(P, H, dtype=bf, device=dev)
        # the layer output (the next layer's input) and its max |x|, recorded
        # by the combine for that input's quantization
        self.out = torch.empty(s.T, H, dtype=bf, device=dev)
        self.out_amax = torch.zeros(1, dtype=f32, device=dev)
        self.qnext = (torch.empty(s.T, H // 2, dtype=u8, device=dev),
                      torch.empty(s.T, H // 16, dtype=u8, device=dev),
                      torch.empty(1, dtype=f32, device=dev), torch.empty(H, dtype=f32, device=dev))
        self.flops_gu = 2.0 * P * H * 2 * I
        self.flops_dn = 2.0 * P * I * H
        self.flops_comp = 2.0 * P * k * 2 * I + 2.0 * P * k * H

    def gemm(self, proj, a, rows, a_row, resid, idx, out, epi, comp=True, path=0):
        nvq = self.nvq
        codes, scales, st = self.qw[proj]
        return nvq.moe_grouped_gemm_w4a4_comp(
            a[0], a[1], a[2], codes, scales, st, self.off, rows=rows, a_row=a_row,
            a_resid=resid if comp else None, comp_idx=idx if comp else None, epilogue=epi,
            ws=self.ws_g, a_row_div=self.s.topk if a_row is not None else 0, out=out, path=path,
            w_cm=self.wcm[proj], h_amax=self.h_amax if epi == nvq.NVQ_EPI_SWIGLU else None)

    def step(self, timer_, comp=True, path=0, tag=""):
        """path 0: the library's choice (exact fp16 dequantization, 128-row
        tiles); 2: the FP8 block-product path; 3: the 256-row tiles; 2 and 3
        are timed separately for the comparison.  tag: a suffix for the GEMM
        timer labels of this call (k = 0 and the paths add their own)."""
        nvq, s = self.nvq, self.s
        tag = tag + ("" if comp else "_k0") + {nvq.NVQ_GEMM_FP8_BLOCK: "_fp8blk",
                                                nvq.NVQ_GEMM_DEQ16_WIDE: "_wide"}.get(path, "")
        timer = lambda label, fn: timer_(self.name + "/" + label, fn)
        r = timer("route", lambda: nvq.nvq_moe_route(self.logits, s.topk))
        self.ids, self.w = r
        self.sp, self.off, self.pos, _ = timer("permute", lambda: nvq.nvq_moe_permute(self.ids, s.E, ws=self.ws_perm))
        timer("quant_x", lambda: nvq.nvfp4_quantize(self.x, score=True, ws=self.ws_q1, out=self.qx))
        idx1, r1, _ = timer("topk_x", lambda: nvq.residual_topk_channels(
            self.x, self.qx[0], self.qx[1], self.qx[2], s.k, scores=self.qx[3], ws=self.ws_t1))
        timer("gemm_gu" + tag, lambda: self.gemm("gu", self.qx, s.P, self.sp, r1, idx1, (self.h, None),
                                                  nvq.NVQ_EPI_SWIGLU, comp, path))
        timer("quant_h", lambda: nvq.nvfp4_quantize(self.h, amax_in=self.h_amax, score=True,
                                                    ws=self.ws_q2, out=self.qh))
        idx2, r2, _ = timer("topk_h", lambda: nvq.residual_topk_channels(
            self.h, self.qh[0], self.qh[1], self.qh[2], s.k, scores=self.qh[3], ws=self.ws_t2))
        timer("gemm_dn" + tag, lambda: self.gemm("dn", self.qh, s.P, None, r2, idx2, (self.y2, None),
                                                  nvq.NVQ_EPI_NONE, comp, path))
        timer("combine", lambda: nvq.nvq_moe_combine(self.y2, self.pos, self.w, out=self.out))

    def fused_combine(self, timer_):
        """The down projection with the layer's combine fused into its
        epilogue (outside the timed steps; same inputs as the step's down
        projection), against the step's separate down GEMM + combine."""
        nvq, s = self.nvq, self.s
        timer = lambda label, fn: timer_(self.name + "/" + label, fn)
        if not hasattr(self, "ws_comb"):
            L = nvq.load()
            self.ws_comb = nvq.workspace(L.moe_gemm_workspace_bytes_comb(s.P, s.E, s.H, s.k, s.T),
                                         self.y2.device)
        idx2, r2, _ = nvq.residual_topk_channels(self.h, self.qh[0], self.qh[1], self.qh[2], s.k,
                                                 scores=self.qh[3], ws=self.ws_t2)
        codes, scales, st = self.qw["dn"]
        timer("gemm_dn_fused_combine", lambda: nvq.moe_grouped_gemm_w4a4_comp(
            self.qh[0], self.qh[1], self.qh[2], codes, scales, st, self.off, rows=s.P,
            a_resid=r2, comp_idx=idx2, ws=self.ws_comb, out=(self.y2, None), w_cm=self.wcm["dn"],
            comb=(self.sp, self.pos, self.w, self.out)))

    def next_input(self, timer_):
        """The layer output quantized as the next layer's input (outside the
        timed steps), two ways: the combine records max |x| and the
        quantization takes it as amax_in (one pass fewer over x), or the plain
        combine and the quantization's own amax pass.  Same record."""
        nvq = self.nvq
        timer = lambda label, fn: timer_(self.name + "/" + label, fn)
        timer("combine_with_amax", lambda: nvq.nvq_moe_combine(self.y2, self.pos, self.w, out=self.out,
                                                               out_amax=self.out_amax))
        timer("quant_next_x_combine_amax", lambda: nvq.nvfp4_quantize(
            self.out, amax_in=self.out_amax, score=True, ws=self.ws_q1, out=self.qnext))
        timer("quant_next_x_own_amax", lambda: nvq.nvfp4_quantize(
            self.out, score=True, ws=self.ws_q1, out=self.qnext))

    def cpu_baseline(self, max_rows=64):
        """The oracle's W4A4 grouped GEMM with compensation (fp64, exhaustive
        dequantization) on the first `max_rows` rows of one expert, gate/up
        then down, timed on the host: a fixed, labelled subset of the layer,
        reported as GFLOP/s of the algorithmic 2 rows K N (the compensation's
        2 rows k N comes on top and is not counted)."""
        import oracle
        from qat_nvfp4_quantize_amd import inputs

        s = self.s
        e = 0 if self.name == "moe_decode" else s.E - 1
        ids, _ = oracle.route(inputs.logits(s), s.topk)
        sp, off, _ = oracle.permute(ids, s.E)
        n_e = int(off[e + 1] - off[e])
        toks = sp[off[e]:off[e + 1]][:max_rows] // s.topk
        rows = toks.size
        xe = inputs.activations(s)[toks]
        he = inputs.to_bf16_bits(np.random.default_rng([0, s.wid, 991]).standard_normal(
            (rows, s.I), dtype=np.float32))
        legs = []
        for proj, a in (("gu", xe), ("dn", he)):
            ac, asc, ast = oracle.quantize(a)
            idx = oracle.topk(oracle.residual_scores(a, ac, asc, ast), s.k)
            wc, wsc, wst = oracle.quantize(inputs.expert_weight(s, proj, e))
            args = (ac, asc, ast, a, idx, wc, wsc, wst, np.arange(rows, dtype=np.int32),
                    np.zeros(rows, np.int32))
            legs.append((oracle.moe_gemm_w4a4, args))
        t = 0.0
        total = 0.0
        for fn, args in legs:
            warm = args[:8] + (args[8][:2], args[9][:2])
            dt, tot = timed_median(lambda: fn(*args), warm=lambda: fn(*warm))
            t += dt
            total += tot
        flops = 2.0 * rows * s.H * 2 * s.I + 2.0 * rows * s.I * s.H
        return {"value": round(flops / t / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.threads(),
                "kind": "oracle",
                "sample": f"first {rows} of expert {e}'s {n_e} rows ({s.P} in the layer): gate/up "
                          f"K={s.H} N={2 * s.I} and down K={s.I} N={s.H} with k={s.k} compensation "
                          "(its own inputs: those rows' tokens of X and a seeded N(0,1) H block), "
                          "median of 3 runs after a 2-row warm-up (%.2f s per subset, %.1f s in all)"
                          % (t, total)}

    def time_graph(self, reps=20):
        """The same layer step captured once into a HIP graph and replayed:
        every kernel and its inputs as in the eager step, without the
        per-launch host overhead between the small kernels."""
        import torch

        passthrough = lambda label, fn: fn()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step(passthrough)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(passthrough)
        for _ in range(3):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        self.graph_ms = a.elapsed_time(b) / reps
        del g

    def report(self, timer_):
        class _T:
            total = {k.split("/", 1)[1]: v for k, v in timer_.total.items() if k.startswith(self.name + "/")}

            @staticmethod
            def avg_ms(label):
                return timer_.avg_ms(self.name + "/" + label)
        timer = _T
        gu, dn = timer.avg_ms("gemm_gu"), timer.avg_ms("gemm_dn")
        layer = sum(timer.avg_ms(k) for k in ("route", "permute", "quant_x", "topk_x", "gemm_gu",
                                                  "quant_h", "topk_h", "gemm_dn", "combine"))
        tf = (self.flops_gu + self.flops_dn) / ((gu + dn) * 1e-3) / 1e12
        out = {"layer_ms": round(layer, 4), "gemm_gu_ms": round(gu, 4), "gemm_dn_ms": round(dn, 4),
               "gemm_tflops": round(tf, 1),
               "gemm_gu_tflops": round(self.flops_gu / (gu * 1e-3) / 1e12, 1),
               "gemm_dn_tflops": round(self.flops_dn / (dn * 1e-3) / 1e12, 1),
               "gemm_frac_fp16_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4),
               "gemm_frac_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4),
               "algorithmic_gflop": round((self.flops_gu + self.flops_dn) / 1e9, 1),
               "comp_gflop": round(self.flops_comp / 1e9, 1),
               "stages_ms": {k: round(timer.avg_ms(k), 4) for k in
                             ("route", "permute", "quant_x", "topk_x", "quant_h", "topk_h", "combine")}}
        if "gemm_gu_k0" in timer.total and "gemm_gu_pair" in timer.total:
            # k > 0 and k = 0 layer steps alternating, each after a step of
            # the same layer, so both find the caches in the same state
            k0 = timer.avg_ms("gemm_gu_k0") + timer.avg_ms("gemm_dn_k0")
            kp = timer.avg_ms("gemm_gu_pair") + timer.avg_ms("gemm_dn_pair")
            out["comp_overhead_vs_k0"] = round(kp / k0 - 1.0, 4)
        if "gemm_gu_fp8blk" in timer.total:
            g8, d8 = timer.avg_ms("gemm_gu_fp8blk"), timer.avg_ms("gemm_dn_fp8blk")
            tf8 = (self.flops_gu + self.flops_dn) / ((g8 + d8) * 1e-3) / 1e12
            out["path_fp8_block"] = {"gemm_gu_ms": round(g8, 4), "gemm_dn_ms": round(d8, 4),
                                     "gemm_tflops": round(tf8, 1),
                                     "frac_fp8_mfma_peak": round(tf8 / FP8_PEAK_TFLOPS, 4),
                                     "time_vs_chosen_path": round((g8 + d8) / (gu + dn), 3)}
        if "gemm_gu_wide" in timer.total:
            gw, dw_ = timer.avg_ms("gemm_gu_wide"), timer.avg_ms("gemm_dn_wide")
            tfw = (self.flops_gu + self.flops_dn) / ((gw + dw_) * 1e-3) / 1e12
            out["path_deq16_wide"] = {"gemm_gu_ms": round(gw, 4), "gemm_dn_ms": round(dw_, 4),
                                      "gemm_tflops": round(tfw, 1),
                                      "time_vs_chosen_path": round((gw + dw_) / (gu + dn), 3)}
        if "gemm_dn_fused_combine" in timer.total:
            fz = timer.avg_ms("gemm_dn_fused_combine")
            out["fused_combine"] = {"gemm_dn_with_combine_ms": round(fz, 4),
                                    "separate_gemm_dn_plus_combine_ms": round(dn + timer.avg_ms("combine"), 4),
                                    "time_vs_separate": round(fz / (dn + timer.avg_ms("combine")), 3)}
        if "quant_next_x_combine_amax" in timer.total:
            ca, qa = timer.avg_ms("combine_with_amax"), timer.avg_ms("quant_next_x_combine_amax")
            c0, q0 = timer.avg_ms("combine"), timer.avg_ms("quant_next_x_own_amax")
            out["next_input_amax"] = {"combine_with_amax_ms": round(ca, 4), "quant_with_amax_in_ms": round(qa, 4),
                                      "combine_ms": round(c0, 4), "quant_own_amax_ms": round(q0, 4),
                                      "pair_vs_plain": round((ca + qa) / (c0 + q0), 3)}
        if hasattr(self, "graph_ms"):
            out["layer_ms_graph"] = round(self.graph_ms, 4)
        return out


class QatLeg:
    """Trainer-side asymmetric W4A16 QAT layer on the cached NVFP4 weight
    record: forward, input gradient and weight gradient of the gate/up and
    down projections (upstream gradients and the down projection's input are
    seeded independently; the SwiGLU backward is not on this path)."""

    name = "qat"

    def __init__(self):
        import torch

        from qat_nvfp4_quantize_amd import inputs, nvq

        self.nvq = nvq
        s = self.s = inputs.QAT
        dev = torch.device("cuda")
        log("[bench] qat: generating inputs")
        ids, self.w = nvq.nvq_moe_route(torch.from_numpy(inputs.logits(s)).to(dev), s.topk)
        self.sp, self.off, self.pos, _ = nvq.nvq_moe_permute(ids, s.E)
        self.ones = torch.ones_like(self.w)
        self.a_row = (self.sp // s.topk).to(torch.int32).contiguous()
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        bf = torch.bfloat16
        self.x = torch.randn(s.T, s.H, generator=g, device=dev).to(bf)
        self.hin = torch.randn(s.P, s.I, generator=g, device=dev).to(bf)
        self.dy_gu = torch.randn(s.P, 2 * s.I, generator=g, device=dev).to(bf)
        self.dy_dn = torch.randn(s.P, s.H, generator=g, device=dev).to(bf)
        self.dout = torch.randn(s.T, s.H, generator=g, device=dev).to(bf)  # gradient of the layer output
        self.out = torch.empty(s.T, s.H, dtype=bf, device=dev)
        self.dx_tok = torch.empty(s.T, s.H, dtype=bf, device=dev)
        self.dw_route = torch.empty(s.T, s.topk, dtype=torch.float32, device=dev)
        # The rollout's record of each projection (codes, scales, s_t) and its
        # compact guidance record (mantissa bits); the trainer's masters have
        # drifted since, and each step rebuilds their codes from the record.
        self.q, self.rec, self.wd, self.gcodes = {}, {}, {}, {}
        for proj in ("gu", "dn"):
            w = inputs.weights_device(s, proj, dev)
            self.q[proj] = nvq.nvfp4_quantize(w)[:3]
            self.rec[proj] = nvq.nvfp4_guidance_record(self.q[proj][0], nvq.NVQ_GUIDE_MANTISSA)
            self.wd[proj] = inputs.drift_device(w, s, proj)
            self.gcodes[proj] = torch.empty_like(self.q[proj][0])
            del w
        n_gu, n_dn = self.wd["gu"].numel(), self.wd["dn"].numel()
        # read w (bf16) + bits + scales, write codes: 2 + 1/8 + 1/16 + 1/2 B/elem
        self.guide_bytes = {"gu": n_gu * 43 // 16, "dn": n_dn * 43 // 16}
        P = s.P
        self.y_gu = torch.empty(P, 2 * s.I, dtype=bf, device=dev)
        self.y_dn = torch.empty(P, s.H, dtype=bf, device=dev)
        self.dx = torch.empty(P, s.H, dtype=bf, device=dev)
        self.dh = torch.empty(P, s.I, dtype=bf, device=dev)
        self.dw_gu = torch.empty(s.E, 2 * s.I, s.H, dtype=torch.float32, device=dev)
        self.dw_dn = torch.empty(s.E, s.H, s.I, dtype=torch.float32, device=dev)
        L = nvq.load()
        self.ws = nvq.workspace(L.qat_gemm_workspace_bytes(P, s.E), dev)
        f_gu = 2.0 * P * s.H * 2 * s.I
        f_dn = 2.0 * P * s.I * s.H
        self.flops = {"fwd_gu": f_gu, "dgrad_gu": f_gu, "wgrad_gu": f_gu,
                      "fwd_dn": f_dn, "dgrad_dn": f_dn, "wgrad_dn": f_dn}

    def step(self, timer_):
        nvq, s = self.nvq, self.s
        timer = lambda label, fn: timer_("qat/" + label, fn)
        F, D, W = nvq.NVQ_QAT_FWD, nvq.NVQ_QAT_DGRAD, nvq.NVQ_QAT_WGRAD
        for proj in ("gu", "dn"):
            # rollout side: export the compact record of its weight codes
            timer("record_" + proj, lambda proj=proj: nvq.nvfp4_guidance_record(
                self.q[proj][0], nvq.NVQ_GUIDE_MANTISSA, out=self.rec[proj]))
        for proj in ("gu", "dn"):
            _, sc, st = self.q[proj]
            timer("guide_" + proj, lambda proj=proj, sc=sc, st=st: nvq.nvfp4_guided_quantize(
                self.wd[proj], self.rec[proj], sc, st, nvq.NVQ_GUIDE_MANTISSA,
                out=self.gcodes[proj]))
        qg = (self.gcodes["gu"], *self.q["gu"][1:])
        qd = (self.gcodes["dn"], *self.q["dn"][1:])
        call = nvq.qat_fakequant_gemm_w4a16
        # forward through the layer
        timer("fwd_gu", lambda: call(F, *qg, self.off, s.P, x=self.x, a_row=self.a_row, ws=self.ws,
                                     out=(self.y_gu, None)))
        timer("swiglu_fwd", lambda: nvq.nvq_swiglu_forward(self.y_gu, out=self.hin))
        timer("fwd_dn", lambda: call(F, *qd, self.off, s.P, x=self.hin, ws=self.ws, out=(self.y_dn, None)))
        timer("combine", lambda: nvq.nvq_moe_combine(self.y_dn, self.pos, self.w, out=self.out))
        # chained backward from the output gradient (identity straight-through)
        timer("combine_bwd", lambda: nvq.nvq_moe_combine_backward(
            self.dout, self.pos, self.w, s.P, y=self.y_dn, out=(self.dy_dn, self.dw_route)))
        timer("dgrad_dn", lambda: call(D, *qd, self.off, s.P, dy=self.dy_dn, ws=self.ws, out=(self.dh, None)))
        timer("wgrad_dn", lambda: call(W, *qd, self.off, s.P, x=self.hin, dy=self.dy_dn, dw=self.dw_dn,
                                       ws=self.ws))
        timer("swiglu_bwd", lambda: nvq.nvq_swiglu_backward(self.y_gu, self.dh, out=self.dy_gu))
        timer("dgrad_gu", lambda: call(D, *qg, self.off, s.P, dy=self.dy_gu, ws=self.ws, out=(self.dx, None)))
        timer("wgrad_gu", lambda: call(W, *qg, self.off, s.P, x=self.x, dy=self.dy_gu, a_row=self.a_row,
                                       dw=self.dw_gu, ws=self.ws))
        timer("token_sum", lambda: nvq.nvq_moe_combine(self.dx, self.pos, self.ones, out=self.dx_tok))

    def cpu_baseline(self, rows=32):
        """The oracle's QAT forward, input gradient and weight gradient (fp64,
        exhaustive dequantization of the cached record) on the first `rows`
        rows of expert 0, both projections: GFLOP/s of the algorithmic
        2 rows K N per GEMM."""
        import oracle
        from qat_nvfp4_quantize_amd import inputs

        s = self.s
        g = np.random.default_rng([0, s.wid, 992])
        legs, flops = [], 0.0
        for proj in ("gu", "dn"):
            K, N = (s.H, 2 * s.I) if proj == "gu" else (s.I, s.H)
            x = inputs.to_bf16_bits(g.standard_normal((rows, K), dtype=np.float32))
            dy = inputs.to_bf16_bits(g.standard_normal((rows, N), dtype=np.float32))
            wc, wsc, wst = oracle.quantize(inputs.expert_weight(s, proj, 0))
            r = np.arange(rows, dtype=np.int32)
            z = np.zeros(rows, np.int32)
            nn, cc = np.meshgrid(np.arange(N, dtype=np.int32), np.arange(K, dtype=np.int32),
                                 indexing="ij")
            legs += [(oracle.qat_fwd, (x, r, z, wc, wsc, wst), (x, r[:2], z[:2], wc, wsc, wst)),
                     (oracle.qat_dgrad, (dy, r, z, wc, wsc, wst), (dy, r[:2], z[:2], wc, wsc, wst)),
                     (oracle.qat_wgrad, (dy, x, r, 0, rows, nn.ravel(), cc.ravel()),
                      (dy, x, r, 0, 2, nn.ravel()[:4096], cc.ravel()[:4096]))]
            flops += 3 * 2.0 * rows * K * N
        t = total = 0.0
        for fn, args, warm in legs:
            dt, tot = timed_median(lambda: fn(*args), warm=lambda: fn(*warm))
            t += dt
            total += tot
        return {"value": round(flops / t / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.threads(),
                "kind": "oracle",
                "sample": f"expert 0, first {rows} rows: forward, input gradient and weight gradient "
                          f"of gate/up (K={s.H}, N={2 * s.I}) and down (K={s.I}, N={s.H}) on seeded "
                          "N(0,1) inputs, median of 3 runs after a 2-row warm-up (%.2f s per "
                          "subset, %.1f s in all)" % (t, total)}

    def direction_mode(self, timer_):
        """The up/down-bit reading of the guidance record (outside the timed
        steps): direction record of the gate/up weights from the rollout's
        codes and its masters, then the guided requantization of the drifted
        masters in direction mode."""
        import torch

        nvq = self.nvq
        timer = lambda label, fn: timer_("qat_dir/" + label, fn)
        if not hasattr(self, "dir_bits"):
            from qat_nvfp4_quantize_amd import inputs

            self.w_master_gu = inputs.weights_device(self.s, "gu")
            self.dir_bits = torch.empty_like(self.rec["gu"])
        codes, sc, st = self.q["gu"]
        timer("record", lambda: nvq.nvfp4_guidance_record(
            codes, nvq.NVQ_GUIDE_DIRECTION, x=self.w_master_gu, scales=sc, tensor_scale=st,
            out=self.dir_bits))
        timer("guide", lambda: nvq.nvfp4_guided_quantize(
            self.wd["gu"], self.dir_bits, sc, st, nvq.NVQ_GUIDE_DIRECTION, out=self.gcodes["gu"]))

    def symmetric(self, timer_):
        """Ablation (outside the timed steps): symmetric W4A4 QAT, i.e. the
        trainer's activations NVFP4-quantized too.  Forward = quantize X +
        W4A4 grouped GEMM without compensation; weight gradient on the
        dequantized activations."""
        import torch

        nvq, s = self.nvq, self.s
        timer = lambda label, fn: timer_("qat_sym/" + label, fn)
        if not hasattr(self, "sym_ws"):
            L = nvq.load()
            self.sym_ws = nvq.workspace(max(L.moe_gemm_workspace_bytes(s.P, s.E, 2 * s.I, 0),
                                            L.moe_gemm_workspace_bytes(s.P, s.E, s.H, 0)), "cuda")
            self.xhat = {"gu": torch.empty_like(self.x), "dn": torch.empty_like(self.hin)}
        for proj, xin, y, a_row, dy, dw in (("gu", self.x, self.y_gu, self.a_row, self.dy_gu, self.dw_gu),
                                            ("dn", self.hin, self.y_dn, None, self.dy_dn, self.dw_dn)):
            qw = (self.gcodes[proj], *self.q[proj][1:])
            qx = timer("quant_" + proj, lambda xin=xin: nvq.nvfp4_quantize(xin))
            timer("fwd_" + proj, lambda qx=qx, qw=qw, y=y, a_row=a_row: nvq.moe_grouped_gemm_w4a4_comp(
                qx[0], qx[1], qx[2], *qw, self.off, rows=s.P, a_row=a_row, ws=self.sym_ws,
                out=(y, None)))
            timer("dequant_" + proj, lambda qx=qx, proj=proj: nvq.nvfp4_dequantize(
                qx[0], qx[1], qx[2], out=self.xhat[proj]))
            timer("wgrad_" + proj, lambda qw=qw, proj=proj, a_row=a_row, dy=dy, dw=dw:
                  nvq.qat_fakequant_gemm_w4a16(nvq.NVQ_QAT_WGRAD, *qw, self.off, s.P,
                                               x=self.xhat[proj], dy=dy, a_row=a_row, dw=dw,
                                               ws=self.ws))

    def report(self, timer):
        out = {}
        tot_ms, tot_f = 0.0, 0.0
        for k, f in self.flops.items():
            ms = timer.avg_ms("qat/" + k)
            out[k + "_ms"] = round(ms, 4)
            out[k + "_tflops"] = round(f / (ms * 1e-3) / 1e12, 1)
            tot_ms += ms
            tot_f += f
        out["total_ms"] = round(tot_ms, 4)
        out["tflops"] = round(tot_f / (tot_ms * 1e-3) / 1e12, 1)
        glue = {k: round(timer.avg_ms("qat/" + k), 4)
                for k in ("swiglu_fwd", "combine", "combine_bwd", "swiglu_bwd", "token_sum")}
        out["glue_ms"] = glue
        out["layer_ms"] = round(tot_ms + sum(glue.values()), 4)
        out["frac_bf16_mfma_peak"] = round(out["tflops"] / BF16_PEAK_TFLOPS, 4)
        out["algorithmic_tflop"] = round(tot_f / 1e12, 3)
        g = {}
        for proj in ("gu", "dn"):
            ms = timer.avg_ms("qat/guide_" + proj)
            g[proj + "_ms"] = round(ms, 4)
            g[proj + "_GBps"] = round(self.guide_bytes[proj] / (ms * 1e-3) / 1e9, 1)
        tot = sum(self.guide_bytes.values()) / ((g["gu_ms"] + g["dn_ms"]) * 1e-3) / 1e9
        g["GBps"] = round(tot, 1)
        g["frac_hbm_peak"] = round(tot / HBM_PEAK_GBS, 4)
        g["algorithmic_bytes"] = sum(self.guide_bytes.values())
        # record: read codes (1/2 B/elem), write bits (1/8 B/elem)
        rb = (self.wd["gu"].numel() + self.wd["dn"].numel()) * 5 // 8
        rms = timer.avg_ms("qat/record_gu") + timer.avg_ms("qat/record_dn")
        g["record_ms"] = round(rms, 4)
        g["record_GBps"] = round(rb / (rms * 1e-3) / 1e9, 1)
        if "qat_dir/guide" in timer.total:
            n = self.wd["gu"].numel()
            rms, gms = timer.avg_ms("qat_dir/record"), timer.avg_ms("qat_dir/guide")
            # direction record reads the master (2), codes (1/2), scales (1/16), writes bits (1/8)
            g["direction_mode_gu"] = {
                "record_ms": round(rms, 4), "record_GBps": round(n * 43 / 16 / (rms * 1e-3) / 1e9, 1),
                "guide_ms": round(gms, 4), "guide_GBps": round(self.guide_bytes["gu"] / (gms * 1e-3) / 1e9, 1)}
        out["guided_requantize"] = g
        if "qat_sym/fwd_gu" in timer.total:
            sym = {}
            for proj in ("gu", "dn"):
                f = self.flops["fwd_" + proj]
                q = timer.avg_ms("qat_sym/quant_" + proj)
                fw = timer.avg_ms("qat_sym/fwd_" + proj)
                sym[proj + "_quant_ms"] = round(q, 4)
                sym[proj + "_fwd_w4a4_k0_ms"] = round(fw, 4)
                sym[proj + "_fwd_w4a4_k0_tflops"] = round(f / (fw * 1e-3) / 1e12, 1)
                sym[proj + "_dequant_ms"] = round(timer.avg_ms("qat_sym/dequant_" + proj), 4)
                sym[proj + "_wgrad_ms"] = round(timer.avg_ms("qat_sym/wgrad_" + proj), 4)
                sym[proj + "_fwd_vs_asymmetric"] = round((q + fw) / out["fwd_" + proj + "_ms"], 3)
            out["symmetric_w4a4_ablation"] = sym
        return out


class KvLeg:
    """FP4 KV cache of one attention layer: quantize the K and V caches
    (2 x [64*8*4096, 128] bf16, static tensor scale), dequantize them to bf16
    (what attention reads), and quantize one decode step's appended rows."""

    name = "kv"

    def __init__(self):
        import torch

        from qat_nvfp4_quantize_amd import inputs, nvq

        self.nvq = nvq
        log("[bench] kv: generating inputs")
        self.kv = inputs.kv_cache(device="cuda")
        self.new = torch.from_numpy(inputs.kv_append().view(np.int16)).view(torch.bfloat16).cuda()
        self.amax = torch.full((2,), inputs.KV_STATIC_AMAX, dtype=torch.float32, device="cuda")
        _, rows, D = self.kv.shape
        dev = self.kv.device
        self.out = (torch.empty(2, rows, D // 2, dtype=torch.uint8, device=dev),
                    torch.empty(2, rows, D // 16, dtype=torch.uint8, device=dev),
                    torch.empty(2, dtype=torch.float32, device=dev), None)
        self.deq = torch.empty_like(self.kv)
        n_new = self.new.shape[1]
        self.out_new = (torch.empty(2, n_new, D // 2, dtype=torch.uint8, device=dev),
                        torch.empty(2, n_new, D // 16, dtype=torch.uint8, device=dev),
                        torch.empty(2, dtype=torch.float32, device=dev), None)
        L = nvq.load()
        self.ws = nvq.workspace(L.nvfp4_quantize_workspace_bytes(2, rows, D), dev)
        self.ws_new = nvq.workspace(L.nvfp4_quantize_workspace_bytes(2, n_new, D), dev)
        n = 2 * rows * D
        self.q_bytes = n * 2 + n // 2 + n // 16 + 8      # read bf16; write codes, scales, s_t
        self.d_bytes = n // 2 + n // 16 + n * 2           # read codes, scales; write bf16

    def step(self, timer_):
        nvq = self.nvq
        timer = lambda label, fn: timer_("kv/" + label, fn)
        timer("quantize", lambda: nvq.nvfp4_quantize(self.kv, amax_in=self.amax, ws=self.ws,
                                                     out=self.out))
        timer("dequantize", lambda: nvq.nvfp4_dequantize(*self.out[:3], out=self.deq))
        timer("append", lambda: nvq.nvfp4_quantize(self.new, amax_in=self.amax, ws=self.ws_new,
                                                   out=self.out_new))

    def report(self, timer):
        q, d = timer.avg_ms("kv/quantize"), timer.avg_ms("kv/dequantize")
        return {"quantize_ms": round(q, 4), "quantize_GBps": round(self.q_bytes / (q * 1e-3) / 1e9, 1),
                "quantize_frac_hbm_peak": round(self.q_bytes / (q * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "dequantize_ms": round(d, 4),
                "dequantize_GBps": round(self.d_bytes / (d * 1e-3) / 1e9, 1),
                "dequantize_frac_hbm_peak": round(self.d_bytes / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "append_ms": round(timer.avg_ms("kv/append"), 4)}


def profiled_traffic(profile="quantize_sweep_8192x7168_bf16.txt",
                     sources=("quantize.hip", "nvq_device.h", "nvq_internal.h")):
    """HBM bytes per call from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (copy-calibrated), when the kernel sources still hash to the value
    recorded there; else None (the figure is stale once the kernel changes)."""
    import hashlib

    here = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(here, "profiles", profile)).read()
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_call: (\d+)", text, re.M)
    m_h = re.search(r"^source_sha1 \(.*\): ([0-9a-f]{40})", text, re.M)
    if not (m_b and m_h):
        return None
    h = hashlib.sha1()
    for fn in sources:
        with open(os.path.join(here, "qat_nvfp4_quantize_amd", "csrc", fn), "rb") as fh:
            h.update(fh.read())
    return int(m_b.group(1)) if h.hexdigest() == m_h.group(1) else None


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
    os.environ["ORACLE_THREADS"] = str(oracle_thread_count())
    legs = []
    wanted = args.legs.split(",")
    if "quant" not in wanted:
        wanted.append("quant")  # the headline value is the quantizer's
    # Step order: the decode layer, then the quantizer (as in the rollout
    # loop, where the next layer's activations are quantized right after a
    # decode layer), then the rest.  Right after the QAT leg's 9.7 GB of
    # writes the quantizer's first pass pays for evicting them.
    from qat_nvfp4_quantize_amd import inputs as _inputs
    if "moe" in wanted or "decode" in wanted:
        legs.append(MoeLeg(_inputs.DECODE))
    qM, qK = (int(v) for v in args.quant_shape.lower().split("x"))
    if "quant" in wanted:
        legs.append(QuantLeg(qM, qK))
    if "copy" in wanted:
        legs.append(CopyLeg())
    if "moe" in wanted or "prefill" in wanted:
        legs.append(MoeLeg(_inputs.PREFILL))
    if "qat" in wanted:
        legs.append(QatLeg())
    if "kv" in wanted:
        legs.append(KvLeg())
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
    # k = 0 reference runs of the MoE legs (outside the timed steps): the
    # compensation overhead is the GEMM time at k > 0 over the time at k = 0,
    # from steps that alternate k > 0 and k = 0 after one untimed pair (every
    # timed one then follows a step of the same layer); and the FP8
    # block-product path, the evaluated alternative to exact fp16
    # dequantization, on the same layers
    from qat_nvfp4_quantize_amd import nvq as _nvq
    untimed = lambda label, fn: fn()
    for leg in legs:
        if leg.name.startswith("moe"):
            leg.step(untimed)
            leg.step(untimed, comp=False)
            for _ in range(3):
                leg.step(timer, tag="_pair")
                leg.step(timer, comp=False)
            for _ in range(2):
                leg.step(timer, path=_nvq.NVQ_GEMM_FP8_BLOCK)
            if leg.name == "moe_prefill":
                for _ in range(2):
                    leg.step(timer, path=_nvq.NVQ_GEMM_DEQ16_WIDE)
            for _ in range(5):
                leg.next_input(timer)
            for _ in range(3):
                leg.fused_combine(timer)
        if leg.name == "qat":
            for _ in range(3):
                leg.symmetric(timer)
            for _ in range(3):
                leg.direction_mode(timer)
    timer.collect()
    for leg in legs:
        if leg.name.startswith("moe"):
            leg.time_graph()

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
        "config": {"workload": f"quantizer sweep: bf16 activation {q.M}x{q.K}, Student-t nu=4, "
                               f"{round(0.005 * q.K)} outlier channels x50; codes+scales+tensor "
                               "scale+residual sums, then top-64 channels"},
        "legs": {"quant": {"quantize_ms": round(q_ms, 5), "topk_ms": round(timer.avg_ms("topk"), 5),
                           "algorithmic_bytes": q.bytes}},
        "roofline": {"kernel": "nvfp4_quantize (amax + quantize + score-reduce kernels)",
                     "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic() if (q.M, q.K) == (8192, 7168) else None},
    }
    for leg in legs:
        if leg.name.startswith("moe") or leg.name in ("qat", "kv"):
            result["legs"][leg.name] = leg.report(timer)
    moe_main = [l for l in legs if l.name == "moe_prefill"] or [l for l in legs if l.name == "moe_decode"]
    if moe_main:
        r = result["legs"][moe_main[0].name]
        result["roofline_gemm"] = {"kernel": "k_moe_gemm_deq16 (%s gate/up + down)" % moe_main[0].name,
                                   "bound": "mfma", "achieved": r["gemm_tflops"],
                                   "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": r["gemm_frac_fp16_mfma_peak"],
                                   "traffic": profiled_traffic(
                                       "moe_grouped_gemm_decode_prefill.txt",
                                       ("gemm_w4a4.hip", "nvq_device.h", "nvq_internal.h",
                                        "nvq_scan.h")) if moe_main[0].name == "moe_prefill" else None,
                                   "frac_of_fp4_peak": r["gemm_frac_fp4_peak"]}
    if any(l.name == "copy" for l in legs):
        c = next(l for l in legs if l.name == "copy")
        result["legs"]["copy"] = {"ms": round(timer.avg_ms("copy"), 5), "bytes": c.bytes,
                                  "GBps": round(c.bytes / timer.avg_ms("copy") / 1e6, 1)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = q.cpu_baseline()
        for leg in legs:
            if leg.name.startswith("moe") or leg.name == "qat":
                log(f"[bench] cpu baseline: {leg.name}")
                result["legs"][leg.name]["cpu_baseline"] = leg.cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

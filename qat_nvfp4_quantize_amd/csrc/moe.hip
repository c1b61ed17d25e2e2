// MoE routing glue for the grouped GEMMs: top-k expert choice with softmax
// weights, the stable token-to-expert permutation (histogram, exclusive scan,
// stable scatter) and the weighted combine back to tokens.
//
// Method context: the TRACE post ("Fonctionnement, côté ingénierie") notes
// that the router's discrete expert choice amplifies rounding differences;
// QUADS explainer §4 runs an MoE.  The permutation is fully deterministic: no
// order-dependent atomics decide any position.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "nvq.h"
#include "nvq_device.h"
#include "nvq_internal.h"
#include "nvq_scan.h"

namespace nvq {
namespace {

constexpr int kPermChunk = 1024;  // pairs per histogram/scatter chunk
constexpr int64_t kPermOwnBaseChunks = 64;  // at most this many chunks: no scan kernel

// Order-preserving key of an fp32 logit (non-NaN), -0 folded onto +0.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Wave maximum of a 64-bit key, returned to every lane: DPP steps within
// each row of 16 lanes (quad swaps, half-row and row mirrors, as in
// wave_max_u32), then the four row maxima by readlane.  Every lane must be
// active.
__device__ __forceinline__ void max_step_u64(uint32_t& hi, uint32_t& lo, uint32_t h2, uint32_t l2) {
  const bool gt = h2 > hi || (h2 == hi && l2 > lo);
  hi = gt ? h2 : hi;
  lo = gt ? l2 : lo;
}
#define NVQ_DPP_MAX_U64(ctrl)                                                                   \
  max_step_u64(hi, lo, (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, ctrl, 0xF, 0xF, false), \
               (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, ctrl, 0xF, 0xF, false))
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  NVQ_DPP_MAX_U64(0xB1);   // quad_perm [1,0,3,2]
  NVQ_DPP_MAX_U64(0x4E);   // quad_perm [2,3,0,1]
  NVQ_DPP_MAX_U64(0x141);  // row_half_mirror
  NVQ_DPP_MAX_U64(0x140);  // row_mirror
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t x = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
    best = x > best ? x : best;
  }
  return best;
}
#undef NVQ_DPP_MAX_U64

// One wave per token: topk rounds of a 64-bit (key, ~id) wave max.  Each
// lane holds kPer = ceil(E / 64) keys (E <= 64 * kPer).
template <int kPer>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int64_t T, int E,
                                              int topk, int32_t* __restrict__ ids,
                                              float* __restrict__ weights) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* l = logits + t * E;
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((uint64_t)ordered_key(l[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e))
                     : 0ull;
  }
  // Selection: lane j keeps the j-th chosen logit (topk <= 64), taken back
  // from its key (no dependent reload; -0 comes back as +0, same exp).
  double lmax = 0.0;
  float my_lv = 0.0f;
  for (int j = 0; j < topk; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const uint32_t e = 0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (key[i] == best) key[i] = 0ull;
    const uint32_t kb = (uint32_t)(best >> 32);
    const float lv = __uint_as_float((kb & 0x80000000u) ? (kb & 0x7FFFFFFFu) : ~kb);
    if (j == 0) lmax = (double)lv;
    if (lane == (j & 63)) my_lv = lv;
    if (lane == 0) ids[t * topk + j] = (int32_t)e;
  }
  // Weights: softmax over the chosen logits in fp64, the exps one per lane,
  // their sum in selection order (the same order on every lane).
  if (topk <= 64) {
    const double x = lane < topk ? exp((double)my_lv - lmax) : 0.0;
    const uint64_t xb = __double_as_longlong(x);
    double den = 0.0;
    for (int j = 0; j < topk; ++j)  // lane j's exp, broadcast through scalar registers
      den += __longlong_as_double(
          (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(xb >> 32), j) << 32) |
                    (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)xb, j)));
    if (lane < topk) weights[t * topk + lane] = (float)(x / den);
  } else if (lane == 0) {
    double den = 0.0;
    for (int j = 0; j < topk; ++j) den += exp((double)l[ids[t * topk + j]] - lmax);
    for (int j = 0; j < topk; ++j)
      weights[t * topk + j] = (float)(exp((double)l[ids[t * topk + j]] - lmax) / den);
  }
}

// Per-chunk expert histogram (ids outside [0, E) are not counted; the
// scatter reports them).  Also clears the status word, ahead of the scatter.
__global__ __launch_bounds__(256) void k_perm_hist(const int32_t* __restrict__ ids, int64_t P, int E,
                                                  int32_t* __restrict__ counts,
                                                  uint32_t* __restrict__ status) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0u;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    const int64_t p = p0 + i;
    if (p < P) {
      const int32_t e = ids[p];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[(int64_t)blockIdx.x * E + e] = h[e];
}

// One workgroup: base[c][e] = offset of expert e + pairs of e in chunks < c.
// Each expert's chunk column is split over 1024 / E threads (8 for E = 128),
// thread t taking expert t % E, so the lanes of a wave read and write
// consecutive experts of one chunk (whole lines; with the parts of one expert
// in adjacent lanes every store touched eight lines).  A thread sums its
// contiguous range of chunks, the partial sums give each range's start, a
// workgroup scan over the expert totals gives the expert offsets, and each
// thread then rewrites its range.  Both passes over the range go in batches
// of 16 (the loads first, so they overlap).
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ counts, int64_t nchunks,
                                                   int E, int32_t* __restrict__ offsets) {
  __shared__ int32_t part_sum[1024];
  __shared__ int32_t s_off[1025];
  __shared__ int32_t s_wave[16];
  const int t = threadIdx.x;
  const int tpe = max(1, 1024 / E);
  const int part = t / E, e = t - part * E;
  const bool live = part < tpe;
  const int64_t len = (nchunks + tpe - 1) / tpe;
  const int64_t cb = min<int64_t>(part * len, nchunks), ce = min<int64_t>(cb + len, nchunks);
  int32_t sum = 0;
  if (live)
    for (int64_t c = cb; c < ce; c += 16) {  // 16 loads in flight, then the adds
      int32_t n[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) n[u] = counts[min<int64_t>(c + u, ce - 1) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) sum += c + u < ce ? n[u] : 0;
    }
  part_sum[t] = sum;
  __syncthreads();
  int32_t tot = 0;
  if (t < E)
    for (int k = 0; k < tpe; ++k) tot += part_sum[k * E + t];
  const int32_t incl = block_inclusive_scan(tot, s_wave);
  if (t < E) s_off[t] = incl - tot;
  if (t == E - 1) s_off[E] = incl;
  __syncthreads();
  if (live) {
    const int32_t off_e = s_off[e];
    int32_t run = off_e;
    for (int k = 0; k < part; ++k) run += part_sum[k * E + e];
    for (int64_t c = cb; c < ce; c += 16) {
      int32_t n[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) n[u] = counts[min<int64_t>(c + u, ce - 1) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c + u < ce) {
          counts[(c + u) * E + e] = run;
          run += n[u];
        }
    }
    if (part == 0) offsets[e] = off_e;
  }
  if (t == 0) offsets[E] = s_off[E];
}

// Stable scatter: one workgroup of kScatWaves waves per chunk, wave w taking
// the w-th quarter of the chunk's pairs, 64 at a time (its ids loaded into
// registers first, so no step waits on memory).  The rank of a pair among
// equal experts in a step is the popcount of the lower lanes whose expert
// matches (found with log2(E) ballots); each wave first ranks its pairs
// against its own earlier steps (a per-wave count per expert in LDS), then,
// after one barrier, adds the counts of the earlier waves of the chunk and
// the chunk's base.  Four waves shorten the serial chain of steps fourfold.
// kOwnBase: counts holds the chunk histograms (not yet scanned), and the
// workgroup derives its chunk's bases itself: expert e's offset (the in-order
// sum of the totals of experts < e) plus e's pairs in earlier chunks; chunk 0
// writes the expert offsets.  For few chunks this replaces k_perm_scan.
// Reports ids outside [0, E) in the status word.  LDS: 5 E ints (dynamic).
constexpr int kScatWaves = 4;
constexpr int kScatSteps = kPermChunk / (64 * kScatWaves);  // steps per wave

// Orders one wave's LDS accesses across its lanes (no instruction: a wave's
// LDS operations complete in program order; this keeps the compiler from
// moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <bool kOwnBase>
__global__ __launch_bounds__(64 * kScatWaves) void k_perm_scatter(
    const int32_t* __restrict__ ids, int64_t P, int E, int64_t nchunks, const int32_t* __restrict__ base,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pos,
    uint32_t* __restrict__ status) {
  extern __shared__ int32_t cnt[];  // [E] chunk bases, then [kScatWaves][E] per-wave counts
  __shared__ int32_t s_wave[16];
  int32_t* wcnt = cnt + E;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t p0 = (int64_t)blockIdx.x * kPermChunk + (int64_t)w * (64 * kScatSteps);
  int32_t eid[kScatSteps];
#pragma unroll
  for (int step = 0; step < kScatSteps; ++step) {
    const int64_t p = p0 + step * 64 + lane;
    eid[step] = p < P ? ids[p] : -1;
  }
  if (kOwnBase) {
    // thread t owns experts [t * per, (t + 1) * per); before: e's pairs in
    // chunks < this one, tot: in all chunks
    const int per = (E + 64 * kScatWaves - 1) / (64 * kScatWaves);
    const int c = (int)blockIdx.x;
    int32_t run = 0;  // this thread's experts' totals, in expert order
    for (int q = 0; q < per; ++q) {
      const int e = tid * per + q;
      int32_t before = 0, tot = 0;
      if (e < E) {
        for (int64_t c0 = 0; c0 < nchunks; c0 += 16) {  // 16 loads in flight, then the adds
          int32_t v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) v[u] = base[min<int64_t>(c0 + u, nchunks - 1) * E + e];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int64_t cc = c0 + u;
            tot += cc < nchunks ? v[u] : 0;
            before += cc < c ? v[u] : 0;
          }
        }
        cnt[e] = run + before;  // offset within this thread's range, fixed below
      }
      run += tot;
    }
    const int32_t incl = block_inclusive_scan(run, s_wave);  // over the thread totals
    const int32_t t_off = incl - run;
    for (int q = 0; q < per; ++q) {
      const int e = tid * per + q;
      if (e < E) {
        cnt[e] += t_off;
        if (c == 0) offsets[e] = cnt[e];  // chunk 0: no earlier chunks
      }
    }
    if (c == 0 && tid == 64 * kScatWaves - 1) offsets[E] = incl;  // all pairs
  } else {
    for (int e = tid; e < E; e += 64 * kScatWaves) cnt[e] = base[(int64_t)blockIdx.x * E + e];
  }
  int32_t* my = wcnt + w * E;
  for (int e = lane; e < E; e += 64) my[e] = 0;
  wave_lds_sync();
  uint32_t bad = 0;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t rank[kScatSteps];
#pragma unroll
  for (int step = 0; step < kScatSteps; ++step) {  // ranks within this wave's pairs
    const int64_t p = p0 + step * 64 + lane;
    const bool in = p < P;
    int32_t e = eid[step];
    const bool ok = in && e >= 0 && e < E;
    bad |= (in && !ok) ? 1u : 0u;
    if (!ok) e = -1;
    eid[step] = e;
    uint64_t match = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot(ok && ((e >> b) & 1));
      match &= (ok && ((e >> b) & 1)) ? m : ~m;
    }
    rank[step] = 0;
    if (ok) rank[step] = my[e] + __popcll(match & lt);
    wave_lds_sync();
    if (ok && (match >> lane) == 1ull) my[e] += __popcll(match);  // highest lane of its group
    wave_lds_sync();
  }
  __syncthreads();  // every wave's counts and the chunk bases are in LDS
#pragma unroll
  for (int step = 0; step < kScatSteps; ++step) {
    const int64_t p = p0 + step * 64 + lane;
    const int32_t e = eid[step];
    int32_t dst = -1;
    if (e >= 0) {
      dst = cnt[e] + rank[step];
      for (int v = 0; v < w; ++v) dst += wcnt[v * E + e];  // pairs of e in the chunk's earlier waves
      sorted_pair[dst] = (int32_t)p;
    }
    if (p < P) pos[p] = dst;
  }
  if (__any(bad) && lane == 0) atomicOr(status, (uint32_t)NVQ_STATUS_BAD_EXPERT);
}

// max |value| of the 8 bf16 of a packed uint4, as 16-bit magnitude bits
__device__ __forceinline__ uint32_t absmax8_bf16(uint4 o) {
  const uint32_t a = max(o.x & 0x7FFFu, (o.x >> 16) & 0x7FFFu), b = max(o.y & 0x7FFFu, (o.y >> 16) & 0x7FFFu);
  const uint32_t c = max(o.z & 0x7FFFu, (o.z >> 16) & 0x7FFFu), d = max(o.w & 0x7FFFu, (o.w >> 16) & 0x7FFFu);
  return max(max(a, b), max(c, d));
}

// The largest stored |out| of a 256-thread workgroup into *amax (fp32 bits
// of a non-negative value order as the values).  DPP wave maxima, the four
// of them combined by thread 0, which issues the atomic only when its value
// exceeds the word's current one: the combine launches one workgroup per
// token (and per 256 vectors), and one atomic each on a single word would
// serialize.  Every thread takes part (threads with nothing stored pass 0).
__device__ __forceinline__ void block_amax_out(uint32_t m16, uint32_t* amax) {
  __shared__ uint32_t s_wmax[4];
  const uint32_t m = wave_max_u32(m16);
  if ((threadIdx.x & 63) == 0) s_wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(s_wmax[0], s_wmax[1]), max(s_wmax[2], s_wmax[3])) << 16;
    if (b != 0u && b > __hip_atomic_load(amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(amax, b);
  }
}

// out[t, n..n+8) = bf16(sum_j w[t,j] * y[pos[t,j], n..n+8)), fp32, j ascending,
// for topk <= kMaxK: every pair's row segment is loaded before the first add,
// so all topk loads are in flight together (a dropped pair, pos < 0, reads
// the token's own output row instead, always valid memory, and is skipped in
// the sum).  The token comes from the grid's y index.  amax (nullable):
// receives max |out| over the stored bf16 values.
template <int kMaxK>
__global__ __launch_bounds__(256) void k_combine_n(const uint16_t* __restrict__ y,
                                                  const int32_t* __restrict__ pos,
                                                  const float* __restrict__ w, int topk,
                                                  int64_t N, uint16_t* __restrict__ out,
                                                  uint32_t* __restrict__ amax) {
  const int64_t nvec = N / 8;
  const int64_t v0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = v0 < nvec;
  if (!live && !amax) return;
  const int64_t v = live ? v0 : nvec - 1;  // idle lanes read a valid vector, store nothing
  const int64_t t = blockIdx.y;
  int32_t pj[kMaxK];
  uint4 q[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    pj[j] = j < topk ? pos[t * topk + j] : -1;
    const uint16_t* src = pj[j] >= 0 ? y + (int64_t)pj[j] * N : out + t * N;
    if (j < topk) q[j] = reinterpret_cast<const uint4*>(src)[v];
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= topk || pj[j] < 0) continue;
    const float wj = w[t * topk + j];
    const uint32_t q4[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc[2 * h] += wj * bf16_lo(q4[h]);
      acc[2 * h + 1] += wj * bf16_hi(q4[h]);
    }
  }
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  if (live) reinterpret_cast<uint4*>(out + t * N)[v] = o;
  if (amax) block_amax_out(live ? absmax8_bf16(o) : 0u, amax);
}

// General topk: one pair at a time.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y,
                                                const int32_t* __restrict__ pos,
                                                const float* __restrict__ w, int64_t T, int topk,
                                                int64_t N, uint16_t* __restrict__ out,
                                                uint32_t* __restrict__ amax) {
  const int64_t nvec = N / 8;
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = i0 < T * nvec;
  if (!live && !amax) return;
  const int64_t i = live ? i0 : T * nvec - 1;
  const int64_t t = i / nvec, v = i - t * nvec;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < topk; ++j) {
    const int32_t p = pos[t * topk + j];
    if (p < 0) continue;
    const float wj = w[t * topk + j];
    const uint4 q = reinterpret_cast<const uint4*>(y + (int64_t)p * N)[v];
    const uint32_t q4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc[2 * h] += wj * bf16_lo(q4[h]);
      acc[2 * h + 1] += wj * bf16_hi(q4[h]);
    }
  }
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  if (live) reinterpret_cast<uint4*>(out + t * N)[v] = o;
  if (amax) block_amax_out(live ? absmax8_bf16(o) : 0u, amax);
}

// ------------------------------------------------ chained backward glue --
// Eight consecutive columns of a [rows, ld] tensor of bf16 or fp32 as fp32.
template <bool kF32>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&v)[8]) {
  if (kF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[2 * h] = bf16_lo(w[h]);
      v[2 * h + 1] = bf16_hi(w[h]);
    }
  }
}

__device__ __forceinline__ uint4 pack8_bf16(const float (&v)[8]) {
  return make_uint4(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                    f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16),
                    f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16),
                    f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16));
}

// h = bf16(silu(g) u), gate in columns [0, I) and up in [I, 2I) of y1.  The
// result is rounded to bf16, so the hardware exp and reciprocal suffice.
template <bool kF32>
__global__ __launch_bounds__(256) void k_swiglu_fwd(const void* __restrict__ y1, int64_t rows,
                                                   int64_t I, uint16_t* __restrict__ h) {
  const int64_t nvec = I / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nvec) return;
  const int64_t r = i / nvec, c = (i - r * nvec) * 8;
  float g[8], u[8], o[8];
  load8<kF32>(y1, r * 2 * I + c, g);
  load8<kF32>(y1, r * 2 * I + I + c, u);
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = g[k] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[k])) * u[k];
  *reinterpret_cast<uint4*>(h + r * I + c) = pack8_bf16(o);
}

// (dg, du) = dh (u s (1 + g (1 - s)), g s) with s = 1 / (1 + exp(-g)),
// written as bf16 [rows, 2I] in the layout of y1.  Very negative g gives
// exp(-g) = inf and s = 0: both gradients 0.
template <bool kF32>
__global__ __launch_bounds__(256) void k_swiglu_bwd(const void* __restrict__ y1,
                                                   const uint16_t* __restrict__ dh, int64_t rows,
                                                   int64_t I, uint16_t* __restrict__ dy1) {
  const int64_t nvec = I / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nvec) return;
  const int64_t r = i / nvec, c = (i - r * nvec) * 8;
  float g[8], u[8], d[8], dg[8], du[8];
  load8<kF32>(y1, r * 2 * I + c, g);
  load8<kF32>(y1, r * 2 * I + I + c, u);
  load8<false>(dh, r * I + c, d);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[k]));
    const float ds = d[k] * sg;
    dg[k] = ds * u[k] * (1.0f + g[k] * (1.0f - sg));
    du[k] = ds * g[k];
  }
  *reinterpret_cast<uint4*>(dy1 + r * 2 * I + c) = pack8_bf16(dg);
  *reinterpret_cast<uint4*>(dy1 + r * 2 * I + I + c) = pack8_bf16(du);
}

// One workgroup per token t: for each of its pairs j (p = pos[t, j] >= 0)
//   dy[p, :] = bf16(fl32(w[t, j] dout[t, :]))
//   dw[t, j] = sum_n dout[t, n] y[p, n]   (fp32; lanes stride the columns,
//              then a wave tree and the four wave sums in order)
constexpr int kCbThreads = 256;
__global__ __launch_bounds__(kCbThreads) void k_combine_bwd(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y,
    const int32_t* __restrict__ pos, const float* __restrict__ w, int topk, int64_t N,
    uint16_t* __restrict__ dy, float* __restrict__ dw) {
  __shared__ float s_part[kCbThreads / kWave];
  const int64_t t = blockIdx.x;
  const int64_t nvec = N / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int j = 0; j < topk; ++j) {
    const int32_t p = pos[t * topk + j];  // uniform over the workgroup
    if (p < 0) {
      if (dw && threadIdx.x == 0) dw[t * topk + j] = 0.0f;
      continue;
    }
    const float wj = w[t * topk + j];
    float acc = 0.0f;
    for (int64_t v = threadIdx.x; v < nvec; v += kCbThreads) {
      float d[8], o[8];
      load8<false>(dout, t * N + 8 * v, d);
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = wj * d[k];
      *reinterpret_cast<uint4*>(dy + (int64_t)p * N + 8 * v) = pack8_bf16(o);
      if (dw) {
        float yv[8];
        load8<false>(y, (int64_t)p * N + 8 * v, yv);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += d[k] * yv[k];
      }
    }
    if (dw) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
      if (lane == 0) s_part[wave] = acc;
      __syncthreads();
      if (threadIdx.x == 0) {
        float sum = s_part[0];
#pragma unroll
        for (int q = 1; q < kCbThreads / kWave; ++q) sum += s_part[q];
        dw[t * topk + j] = sum;
      }
      __syncthreads();
    }
  }
}

}  // namespace
}  // namespace nvq

using namespace nvq;

extern "C" int nvq_moe_route(const float* logits, int64_t T, int64_t E, int64_t topk, int32_t* ids,
                             float* weights, void* stream) {
  if (T != 0 && (!logits || !ids || !weights)) return NVQ_EINVAL;
  if (T < 0 || E < 1 || E > 1024 || topk < 1 || topk > E) return NVQ_ESHAPE;
  if (T == 0) return NVQ_OK;
  const dim3 grid((unsigned)((T + 3) / 4));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (E <= 64)
    hipLaunchKernelGGL(k_route<1>, grid, dim3(256), 0, s, logits, T, (int)E, (int)topk, ids, weights);
  else if (E <= 128)
    hipLaunchKernelGGL(k_route<2>, grid, dim3(256), 0, s, logits, T, (int)E, (int)topk, ids, weights);
  else if (E <= 256)
    hipLaunchKernelGGL(k_route<4>, grid, dim3(256), 0, s, logits, T, (int)E, (int)topk, ids, weights);
  else
    hipLaunchKernelGGL(k_route<16>, grid, dim3(256), 0, s, logits, T, (int)E, (int)topk, ids, weights);
  return last_launch();
}

extern "C" size_t nvq_moe_permute_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  if (T < 0 || topk < 1 || E < 1) return kAlign;
  const int64_t nchunks = std::max<int64_t>(1, (T * topk + kPermChunk - 1) / kPermChunk);
  WsCarve c(nullptr);
  c.take<int32_t>((size_t)(nchunks * E));
  return c.off;
}

extern "C" int nvq_moe_permute(const int32_t* ids, int64_t T, int64_t topk, int64_t E,
                               int32_t* sorted_pair, int32_t* expert_offsets, int32_t* pos,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!expert_offsets || !ws || (T != 0 && (!ids || !sorted_pair || !pos))) return NVQ_EINVAL;
  if (T < 0 || topk < 1 || E < 1 || E > 1024) return NVQ_ESHAPE;
  if (!aligned256(ws)) return NVQ_EALIGN;
  const int64_t P = T * topk;
  const int64_t nchunks = std::max<int64_t>(1, (P + kPermChunk - 1) / kPermChunk);
  WsCarve c(ws);
  int32_t* counts = c.take<int32_t>((size_t)(nchunks * E));
  if (ws_bytes < c.off) return NVQ_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_perm_hist, dim3((unsigned)nchunks), dim3(256), E * sizeof(int32_t), s, ids, P,
                     (int)E, counts, c.status());
  if (int rc = last_launch()) return rc;
  // Few chunks: each scatter workgroup sums the histograms itself (reading them
  // all costs less than a separate scan launch); many: one scan workgroup.
  const bool own_base = nchunks <= kPermOwnBaseChunks && P > 0;
  if (!own_base) {
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, counts, nchunks, (int)E,
                       expert_offsets);
    if (int rc = last_launch()) return rc;
  }
  if (P == 0) return NVQ_OK;
  if (own_base)
    hipLaunchKernelGGL(k_perm_scatter<true>, dim3((unsigned)nchunks), dim3(64 * kScatWaves),
                       (1 + kScatWaves) * E * sizeof(int32_t), s, ids,
                       P, (int)E, nchunks, counts, expert_offsets, sorted_pair, pos, c.status());
  else
    hipLaunchKernelGGL(k_perm_scatter<false>, dim3((unsigned)nchunks), dim3(64 * kScatWaves),
                       (1 + kScatWaves) * E * sizeof(int32_t), s, ids,
                       P, (int)E, nchunks, counts, expert_offsets, sorted_pair, pos, c.status());
  return last_launch();
}

extern "C" int nvq_moe_combine(const uint16_t* y, const int32_t* pos, const float* weights,
                               int64_t T, int64_t topk, int64_t N, uint16_t* out, float* out_amax,
                               void* stream) {
  if (T != 0 && (!y || !pos || !weights || !out)) return NVQ_EINVAL;
  if (T < 0 || topk < 1 || N <= 0 || (N & 7)) return NVQ_ESHAPE;
  if (!aligned16(y) || !aligned16(out) || ((uintptr_t)out_amax & 3u)) return NVQ_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* amax = reinterpret_cast<uint32_t*>(out_amax);
  if (amax) {  // the maximum of no values is 0
    if (int rc = clear_status(amax, s)) return rc;
  }
  const int64_t n = T * (N / 8);
  if (n == 0) return NVQ_OK;
  if (topk <= 8 && T <= 65535 && (N / 8 + 255) / 256 <= 0x7FFFFFFF) {
    const dim3 grid((unsigned)((N / 8 + 255) / 256), (unsigned)T);
    hipLaunchKernelGGL(k_combine_n<8>, grid, dim3(256), 0, s, y, pos, weights, (int)topk, N, out,
                       amax);
  } else {
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, pos,
                       weights, T, (int)topk, N, out, amax);
  }
  return last_launch();
}

extern "C" int nvq_swiglu_forward(const void* y1, int y1_dtype, int64_t rows, int64_t I,
                                  uint16_t* h, void* stream) {
  if (y1_dtype != NVQ_F32 && y1_dtype != NVQ_BF16) return NVQ_EINVAL;
  if (rows < 0 || I <= 0 || (I & 7)) return NVQ_ESHAPE;
  const int64_t n = rows * (I / 8);
  if (n == 0) return NVQ_OK;
  if (!y1 || !h) return NVQ_EINVAL;
  if (!aligned16(y1) || !aligned16(h)) return NVQ_EALIGN;
  if ((n + 255) / 256 > 0x7FFFFFFF) return NVQ_ESHAPE;
  const dim3 grid((unsigned)((n + 255) / 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (y1_dtype == NVQ_F32)
    hipLaunchKernelGGL(k_swiglu_fwd<true>, grid, dim3(256), 0, s, y1, rows, I, h);
  else
    hipLaunchKernelGGL(k_swiglu_fwd<false>, grid, dim3(256), 0, s, y1, rows, I, h);
  return last_launch();
}

extern "C" int nvq_swiglu_backward(const void* y1, int y1_dtype, const uint16_t* dh, int64_t rows,
                                   int64_t I, uint16_t* dy1, void* stream) {
  if (y1_dtype != NVQ_F32 && y1_dtype != NVQ_BF16) return NVQ_EINVAL;
  if (rows < 0 || I <= 0 || (I & 7)) return NVQ_ESHAPE;
  const int64_t n = rows * (I / 8);
  if (n == 0) return NVQ_OK;
  if (!y1 || !dh || !dy1) return NVQ_EINVAL;
  if (!aligned16(y1) || !aligned16(dh) || !aligned16(dy1)) return NVQ_EALIGN;
  if ((n + 255) / 256 > 0x7FFFFFFF) return NVQ_ESHAPE;
  const dim3 grid((unsigned)((n + 255) / 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (y1_dtype == NVQ_F32)
    hipLaunchKernelGGL(k_swiglu_bwd<true>, grid, dim3(256), 0, s, y1, dh, rows, I, dy1);
  else
    hipLaunchKernelGGL(k_swiglu_bwd<false>, grid, dim3(256), 0, s, y1, dh, rows, I, dy1);
  return last_launch();
}

extern "C" int nvq_moe_combine_backward(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                                        const float* weights, int64_t T, int64_t topk, int64_t N,
                                        uint16_t* dy, float* dw, void* stream) {
  if (T < 0 || topk < 1 || N <= 0 || (N & 7)) return NVQ_ESHAPE;
  if (T == 0) return NVQ_OK;
  if (!dout || !pos || !weights || !dy || (dw && !y)) return NVQ_EINVAL;
  if (!aligned16(dout) || !aligned16(dy) || (dw && !aligned16(y))) return NVQ_EALIGN;
  if (T > 0x7FFFFFFF) return NVQ_ESHAPE;
  hipLaunchKernelGGL(k_combine_bwd, dim3((unsigned)T), dim3(kCbThreads), 0,
                     static_cast<hipStream_t>(stream), dout, y, pos, weights, (int)topk, N, dy, dw);
  return last_launch();
}

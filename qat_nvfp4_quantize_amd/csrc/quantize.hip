// NVFP4 quantization, residual channel scores, top-k channel selection,
// residual gather and dequantization for gfx950.
//
// Method: QUADS explainer §1 (E2M1 grid), §2.1 (online activation
// quantization, shared weight quantize-dequantize path), §2.2-B (residual
// channel selection); TRACE post "Fonctionnement, côté ingénierie" (block
// scaling, per-element up/down rounding).  NVFP4 layout: 16-element blocks
// along K, E4M3 block scales, fp32 tensor scale s_t = amax / (6 * 448),
// nearest rounding with ties to even, two codes per byte (even element low).
//
// Every decision is exact.  The per-element fast path multiplies by an fp32
// reciprocal scale and lets the hardware FP4 conversion round; it is taken
// only when the approximate quotient is provably away from every E2M1
// decision midpoint (all of which have 21 trailing zero mantissa bits).  Any
// element near a midpoint (and any block with an extreme tensor scale) is
// decided in fp64, where the midpoint products are exact.  The E4M3 block
// scale uses the same scheme with its own midpoints.
//
// This translation unit is compiled with -ffp-contract=off: the dequantized
// value fl32(fl32(G s_b) s_t) and the residual fl32(x - v) are two separate
// roundings by definition.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "nvq.h"
#include "nvq_device.h"
#include "nvq_internal.h"

namespace nvq {
namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxWgMax = 1024;     // workgroups per call, split over batch items
constexpr int kQRows = 128;          // rows per quantize workgroup (one score chunk)
constexpr int kQSub = 16;            // rows per wave (one score sub-chunk)
constexpr int kQBlocksPerWave = 64;  // 16-element blocks per wave row (one per lane)
constexpr int kQCols = kQBlocksPerWave * 16;

// Pass 1 workgroups per batch item; a pure function of the shape so the
// workspace query and the launch agree.
int amax_wg_per_item(int64_t batch, int64_t n_vec_per_item) {
  int64_t per_item = std::max<int64_t>(1, kAmaxWgMax / std::max<int64_t>(batch, 1));
  int64_t need = (n_vec_per_item + kAmaxThreads * 4 - 1) / (kAmaxThreads * 4);
  return (int)std::max<int64_t>(1, std::min(per_item, need));
}

// ---------------------------------------------------------------- pass 1 --
// Partial max of |x| (as fp32 bits) over a strided slice of one batch item:
// each wave reduces with DPP and its lane 0 writes the wave's partial straight
// to the workspace (kAmaxThreads / 64 partials per workgroup, no LDS).
// Non-finite values compare above all finite ones and are reported by pass 2.
// Also clears the status word.
constexpr int kAmaxWaves = kAmaxThreads / 64;

// |x| bits of the 8 bf16 or 4 fp32 values of a 16-byte vector, folded into m
// (bf16 magnitudes as 16-bit patterns, shifted to fp32 position at the end).
template <bool kBF16>
__device__ __forceinline__ void amax_fold(uint32_t& m, uint4 q) {
  if (kBF16) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  } else {
    m = max(m, max(max(q.x & 0x7FFFFFFFu, q.y & 0x7FFFFFFFu), max(q.z & 0x7FFFFFFFu, q.w & 0x7FFFFFFFu)));
  }
}

template <bool kBF16>
__device__ __forceinline__ void amax_store_wave(uint32_t m, uint32_t* __restrict__ partial, int nwg,
                                                uint32_t* __restrict__ status) {
  if (kBF16) m <<= 16;
  m = wave_max_u32(m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
    partial[((int64_t)blockIdx.y * nwg + blockIdx.x) * kAmaxWaves + wave] = m;
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = 0;
}

// Dense tensor: the item is one flat run of vec_per_item 16-byte vectors.
template <bool kBF16>
__global__ __launch_bounds__(kAmaxThreads) void k_amax(const uint4* __restrict__ x,
                                                      int64_t vec_per_item, int nwg,
                                                      uint32_t* __restrict__ partial,
                                                      uint32_t* __restrict__ status) {
  const int item = blockIdx.y;
  const uint4* xi = x + (int64_t)item * vec_per_item;
  const int64_t stride = (int64_t)nwg * kAmaxThreads;
  int64_t v = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  uint32_t m = 0;
  for (; v + 3 * stride < vec_per_item; v += 4 * stride) {
    const uint4 a = xi[v], b = xi[v + stride], c = xi[v + 2 * stride], d = xi[v + 3 * stride];
    amax_fold<kBF16>(m, a);
    amax_fold<kBF16>(m, b);
    amax_fold<kBF16>(m, c);
    amax_fold<kBF16>(m, d);
  }
  for (; v < vec_per_item; v += stride) amax_fold<kBF16>(m, xi[v]);
  amax_store_wave<kBF16>(m, partial, nwg, status);
}

// Amax pass laid out like the quantize pass that follows it (one item, the
// scored row tile): workgroup (bx, by) reads exactly the rows and block
// columns that quantize workgroup (bx, by) will read, wave w its 16-row
// sub-chunk, lane l its block column, but each wave walks its rows last to
// first.  Workgroups go to the XCDs in the same round-robin order in both
// launches, so the rows a quantize wave starts with are the ones its amax
// wave read last and may still be in that XCD's L2.  Four rows in flight per
// lane; one partial per wave.
template <bool kBF16>
__global__ __launch_bounds__(512) void k_amax_tiles(const void* __restrict__ xv, int64_t rows,
                                                   int64_t K, int64_t ldx,
                                                   uint32_t* __restrict__ partial,
                                                   uint32_t* __restrict__ status) {
  constexpr int kVec = kBF16 ? 2 : 4;  // 16-byte vectors per block
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nblk = K >> 4;
  const int64_t blk = (int64_t)blockIdx.x * kQBlocksPerWave + lane;
  const int64_t r0 = (int64_t)blockIdx.y * kQRows + wave * kQSub;
  const int nrows = (int)max<int64_t>(0, min<int64_t>(kQSub, rows - r0));
  uint32_t m = 0;
  if (blk < nblk && nrows > 0) {
    const int64_t xrow = ldx * (kBF16 ? 2 : 4);
    const char* base = static_cast<const char*>(xv) + (r0 * ldx + blk * 16) * (kBF16 ? 2 : 4);
    // rows nrows-1 .. 0 in groups of four; a group's rows past the sub-chunk
    // are clamped to its row 0 (read, folded again, harmless for a max)
#pragma unroll 1
    for (int top = nrows - 1; top >= 0; top -= 4) {
      uint4 v[4][kVec];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = max(top - u, 0);
        const uint4* p = reinterpret_cast<const uint4*>(base + rr * xrow);
#pragma unroll
        for (int q = 0; q < kVec; ++q) v[u][q] = p[q];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < kVec; ++q) amax_fold<kBF16>(m, v[u][q]);
    }
  }
  if (kBF16) m <<= 16;
  m = wave_max_u32(m);
  if (lane == 0) partial[((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 8 + wave] = m;
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = 0;
}

// Row-strided tensor: rows of vpr vectors, ldv vectors apart (item b starts
// at row b * rows).  Wave w of workgroup g takes rows 4 g + w, 4 g + w +
// 4 nwg, ...; its lanes stride along the row.
template <bool kBF16>
__global__ __launch_bounds__(kAmaxThreads) void k_amax_rows(const uint4* __restrict__ x, int64_t rows,
                                                           int64_t vpr, int64_t ldv, int nwg,
                                                           uint32_t* __restrict__ partial,
                                                           uint32_t* __restrict__ status) {
  const uint4* xi = x + (int64_t)blockIdx.y * rows * ldv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t m = 0;
  for (int64_t r = (int64_t)blockIdx.x * kAmaxWaves + wave; r < rows; r += (int64_t)nwg * kAmaxWaves) {
    const uint4* row = xi + r * ldv;
    for (int64_t c = lane; c < vpr; c += 64) amax_fold<kBF16>(m, row[c]);
  }
  amax_store_wave<kBF16>(m, partial, nwg, status);
}

__global__ void k_clear_status(uint32_t* status) { *status = 0; }

// No rows: the amax over nothing is 0 (or amax_in), so s_t = fl32(amax / 2688)
// as in pass 2, and every channel's residual sum is the empty sum 0.
__global__ void k_quant_empty(const float* __restrict__ amax_in, int64_t batch, float* __restrict__ tensor_scale,
                              float* __restrict__ chan_score, int64_t K, uint32_t* __restrict__ status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *status = 0;
  if (i < batch) tensor_scale[i] = amax_in ? (float)((double)amax_in[i] / 2688.0) : 0.0f;
  if (chan_score && i < K) chan_score[i] = 0.0f;
}

// ---------------------------------------------------------------- pass 2 --
// E4M3 code (0..0x7E) -> fp32.
__device__ __forceinline__ float e4m3_value_f32(uint32_t sc) {
  return (sc >= 8u) ? __uint_as_float((sc + 960u) << 20) : (float)sc * 0x1p-9f;
}

template <int kSel>
__device__ __forceinline__ uint32_t cvt_fp4_pair(uint32_t w, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, kSel);
}

template <int kSel>
__device__ __forceinline__ float2 fp4_pair_to_f32(uint32_t w) {
  auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, kSel);
  return make_float2(t[0], t[1]);
}

// Block scale for a tensor scale in the fast range: the E4M3 value nearest the
// real quotient am / (6 s_t), ties to even, saturating at 0x7E (448).
// q = fl(am * g), g = fl(1 / (6 s_t)), is within about 1 ulp of the quotient,
// so it decides alone unless it lies within 8 ulp of an E4M3 midpoint (a
// value with one more significant bit than the grid).  There, the sign of
// am - 6 mid s_t decides: 6 mid has at most 7 significant bits, so
// fma(-(6 mid), s_t, am) rounds the exact difference once and keeps its sign,
// and it is zero exactly on a tie, which goes to the even code.
__device__ __forceinline__ uint32_t e4m3_code_fast(float am, float g, float s_t) {
  const float q = am * g;
  if (!(q < 448.0f)) return 0x7E;
  const uint32_t qb = __float_as_uint(q);
  uint32_t c_lo;
  float mid;
  if (q >= 0.015625f) {
    // normal E4M3: grid = 3 mantissa bits; midpoints have bit 19 set and the
    // low 19 bits clear
    if ((qb & 0xFFFFFu) - 0x80000u + 8u >= 16u)
      return (qb - (120u << 23) + 0x7FFFFu + ((qb >> 20) & 1u)) >> 20;
    mid = __uint_as_float((qb & 0xFFF00000u) | 0x80000u);
    c_lo = ((qb & 0xFFF00000u) - (120u << 23)) >> 20;
  } else {
    // subnormal E4M3: grid 2^-9, midpoints at odd multiples of 2^-10
    const float t = q * 512.0f;
    const float fl = __builtin_floorf(t);
    if (!(fabsf((t - fl) - 0.5f) < 0x1p-16f)) return (uint32_t)__builtin_rintf(t);
    mid = (fl + 0.5f) * 0x1p-9f;
    c_lo = (uint32_t)fl;
  }
  const float d = __builtin_fmaf(-(6.0f * mid), s_t, am);
  return c_lo + ((d > 0.0f || (d == 0.0f && (c_lo & 1u))) ? 1u : 0u);
}

template <bool kBF16>
struct RowBlock {
  uint4 q[kBF16 ? 2 : 4];
  // block blk of row `row` of a tensor whose rows are ld elements apart
  __device__ __forceinline__ void load(const void* xv, int64_t row, int64_t ld, int64_t blk) {
    load_at(static_cast<const char*>(xv) + (row * ld + blk * 16) * (kBF16 ? 2 : 4));
  }
  __device__ __forceinline__ void load_at(const char* at) {
    const uint4* p = reinterpret_cast<const uint4*>(at);
#pragma unroll
    for (int i = 0; i < (kBF16 ? 2 : 4); ++i) q[i] = p[i];
  }
  __device__ __forceinline__ uint32_t word(int i) const {
    const uint4& v = q[i >> 2];
    return (i & 3) == 0 ? v.x : (i & 3) == 1 ? v.y : (i & 3) == 2 ? v.z : v.w;
  }
  __device__ __forceinline__ void unpack(float (&xf)[16]) const {
    if (kBF16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xf[2 * j] = bf16_lo(word(j));
        xf[2 * j + 1] = bf16_hi(word(j));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) xf[j] = __uint_as_float(word(j));
    }
  }
  // Stores the raw words into this lane's LDS slot (element j readable by slot_elem).
  __device__ __forceinline__ void to_slot(uint32_t* slot) const {
    uint4* s4 = reinterpret_cast<uint4*>(slot);
#pragma unroll
    for (int i = 0; i < (kBF16 ? 2 : 4); ++i) s4[i] = q[i];
  }
  __device__ static __forceinline__ float slot_elem(const uint32_t* slot, int j) {
    if (kBF16) {
      const uint32_t w = slot[j >> 1];
      return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    return __uint_as_float(slot[j]);
  }
};

// v = fl32(fl32(|G| s_b) s_t) for the 16 codes of a block; acc[j] += |r_j| with
// r_j = fl32(x_j - v_j) (|r| = | |x| - v | since v carries the sign of x).
__device__ __forceinline__ void add_residual(const float (&xf)[16], uint2 cw, float s_b, float s_t,
                                             float (&acc)[16]) {
  float2 g2[8];
  g2[0] = fp4_pair_to_f32<0>(cw.x);
  g2[1] = fp4_pair_to_f32<1>(cw.x);
  g2[2] = fp4_pair_to_f32<2>(cw.x);
  g2[3] = fp4_pair_to_f32<3>(cw.x);
  g2[4] = fp4_pair_to_f32<0>(cw.y);
  g2[5] = fp4_pair_to_f32<1>(cw.y);
  g2[6] = fp4_pair_to_f32<2>(cw.y);
  g2[7] = fp4_pair_to_f32<3>(cw.y);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v0 = (fabsf(g2[j].x) * s_b) * s_t;
    const float v1 = (fabsf(g2[j].y) * s_b) * s_t;
    acc[2 * j] += fabsf(fabsf(xf[2 * j]) - v0);
    acc[2 * j + 1] += fabsf(fabsf(xf[2 * j + 1]) - v1);
  }
}

// One block, tensor scale in the fast range.  Element codes: the hardware FP4
// conversion rounds y = x h with h bracketed at (1 -+ 2^-20) / (s_b s_t); y is
// within 2^-21.5 of the real quotient, so both brackets agree unless the
// quotient is within 2^-19 of an E2M1 midpoint.  Where they disagree the
// upper index is the lower plus one and the sign of |x| - m s_b s_t (m the
// midpoint between them; m s_b has at most 7 significant bits, so one fma
// rounds the exact difference once) decides; zero is a tie, which goes to the
// even index.  slot: this lane's LDS words for the rare fix-up.
template <bool kBF16, bool kScore>
__device__ __forceinline__ void encode_block_fast(const RowBlock<kBF16>& rb, float s_t, float g,
                                                  float inv_st, uint32_t& sc_out, uint2& cw_out,
                                                  float (&acc)[16], uint32_t& bad, uint32_t* slot) {
  float xf[16];
  rb.unpack(xf);
  float am = __builtin_fmaxf(__builtin_fmaxf(fabsf(xf[0]), fabsf(xf[1])), fabsf(xf[2]));
#pragma unroll
  for (int j = 3; j < 15; j += 2) am = __builtin_fmaxf(__builtin_fmaxf(am, fabsf(xf[j])), fabsf(xf[j + 1]));
  am = __builtin_fmaxf(am, fabsf(xf[15]));
  if (!(am <= 3.40282347e38f)) bad = 1;
  const uint32_t sc = e4m3_code_fast(am, g, s_t);
  sc_out = sc;
  const float s_b = e4m3_value_f32(sc);
  const float h = sc == 0 ? 0.0f : __builtin_amdgcn_rcpf(s_b) * inv_st;
  const float h_lo = h * 0.99999904632568359375f;  // 1 - 2^-20
  const float h_hi = h * 1.00000095367431640625f;  // 1 + 2^-20
  uint32_t lo0 = 0, lo1 = 0, hi0 = 0, hi1 = 0;
  lo0 = cvt_fp4_pair<0>(lo0, xf[0] * h_lo, xf[1] * h_lo);
  lo0 = cvt_fp4_pair<1>(lo0, xf[2] * h_lo, xf[3] * h_lo);
  lo0 = cvt_fp4_pair<2>(lo0, xf[4] * h_lo, xf[5] * h_lo);
  lo0 = cvt_fp4_pair<3>(lo0, xf[6] * h_lo, xf[7] * h_lo);
  lo1 = cvt_fp4_pair<0>(lo1, xf[8] * h_lo, xf[9] * h_lo);
  lo1 = cvt_fp4_pair<1>(lo1, xf[10] * h_lo, xf[11] * h_lo);
  lo1 = cvt_fp4_pair<2>(lo1, xf[12] * h_lo, xf[13] * h_lo);
  lo1 = cvt_fp4_pair<3>(lo1, xf[14] * h_lo, xf[15] * h_lo);
  hi0 = cvt_fp4_pair<0>(hi0, xf[0] * h_hi, xf[1] * h_hi);
  hi0 = cvt_fp4_pair<1>(hi0, xf[2] * h_hi, xf[3] * h_hi);
  hi0 = cvt_fp4_pair<2>(hi0, xf[4] * h_hi, xf[5] * h_hi);
  hi0 = cvt_fp4_pair<3>(hi0, xf[6] * h_hi, xf[7] * h_hi);
  hi1 = cvt_fp4_pair<0>(hi1, xf[8] * h_hi, xf[9] * h_hi);
  hi1 = cvt_fp4_pair<1>(hi1, xf[10] * h_hi, xf[11] * h_hi);
  hi1 = cvt_fp4_pair<2>(hi1, xf[12] * h_hi, xf[13] * h_hi);
  hi1 = cvt_fp4_pair<3>(hi1, xf[14] * h_hi, xf[15] * h_hi);
  uint32_t d0 = lo0 ^ hi0, d1 = lo1 ^ hi1;
  if (d0 | d1) {
    rb.to_slot(slot);
    const float half_sb = 0.5f * s_b;
#pragma unroll 1
    while (d0 | d1) {
      const bool first = d0 != 0;
      const uint32_t sh = __builtin_ctz(first ? d0 : d1) & ~3u;
      const int j = (first ? 0 : 8) + (int)(sh >> 2);
      const uint32_t wl = first ? lo0 : lo1;
      const uint32_t il = (wl >> sh) & 7u, ih = ((first ? hi0 : hi1) >> sh) & 7u;
      // |G_lo| and |G_hi| from one conversion of the byte (il, ih)
      const float2 gg = fp4_pair_to_f32<0>(il | (ih << 4));
      const float d = __builtin_fmaf(-((gg.x + gg.y) * half_sb), s_t,
                                     fabsf(RowBlock<kBF16>::slot_elem(slot, j)));
      const uint32_t pick = (d > 0.0f || (d == 0.0f && !(ih & 1u))) ? ih : il;
      const uint32_t nw = (wl & ~(7u << sh)) | (pick << sh);
      if (first) {
        lo0 = nw;
        d0 &= ~(15u << sh);
      } else {
        lo1 = nw;
        d1 &= ~(15u << sh);
      }
    }
  }
  cw_out = make_uint2(lo0, lo1);
  if (kScore) add_residual(xf, cw_out, s_b, s_t, acc);
}

// One block decided entirely in fp64 (tensor scale outside [2^-100, 2^100],
// where the fp32 reciprocals would overflow).  Off the hot path.
template <bool kBF16, bool kScore>
__device__ __forceinline__ void encode_block_exact(const RowBlock<kBF16>& rb, float s_t,
                                                   double six_st, uint32_t& sc_out,
                                                   uint2& cw_out, float (&acc)[16],
                                                   uint32_t& bad, uint32_t* slot) {
  float xf[16];
  rb.unpack(xf);
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) am = __builtin_fmaxf(am, fabsf(xf[j]));
  if (!(am <= 3.40282347e38f)) bad = 1;
  const uint32_t sc = s_t > 0.0f ? e4m3_code_exact(am, six_st) : 0u;
  sc_out = sc;
  const float s_b = e4m3_value_f32(sc);
  rb.to_slot(slot);
  const double S = (double)s_b * (double)s_t;
  uint32_t c0 = 0u, c1 = 0u;
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const float v = RowBlock<kBF16>::slot_elem(slot, j);
    const uint32_t idx = (sc == 0) ? 0u : e2m1_index_exact(fabsf(v), S);
    const uint32_t nib = (idx | ((__float_as_uint(v) >> 28) & 8u)) << (4 * (j & 7));
    c0 |= (j < 8) ? nib : 0u;
    c1 |= (j < 8) ? 0u : nib;
  }
  cw_out = make_uint2(c0, c1);
  if (kScore) add_residual(xf, cw_out, s_b, s_t, acc);
}

struct RowsResult {
  float acc[16];
  uint32_t bad;
};

template <bool kBF16, bool kScore>
__device__ __attribute__((noinline)) RowsResult quantize_rows_exact(
    const void* xv, int64_t row0, int nrows, int64_t K, int64_t ldx, int64_t blk, float s_t,
    double six_st, uint8_t* codes, uint8_t* scales, uint32_t* slot) {
  RowsResult res;
#pragma unroll
  for (int j = 0; j < 16; ++j) res.acc[j] = 0.0f;
  res.bad = 0;
  const int64_t nblk = K >> 4;
  for (int rr = 0; rr < nrows; ++rr) {
    RowBlock<kBF16> rb;
    rb.load(xv, row0 + rr, ldx, blk);
    uint32_t sc;
    uint2 cw;
    encode_block_exact<kBF16, kScore>(rb, s_t, six_st, sc, cw, res.acc, res.bad, slot);
    *reinterpret_cast<uint2*>(codes + (row0 + rr) * (K >> 1) + blk * 8) = cw;
    scales[(row0 + rr) * nblk + blk] = (uint8_t)sc;
  }
  return res;
}

// Workgroup = 8 waves = one 128-row chunk x 1024 columns; wave w = the 16-row
// sub-chunk w; lane l = one 16-element block column.  Each lane quantizes its
// block in each of its rows (three rows in flight) and keeps 16 per-column
// residual sums, sequential in row order.  The chunk partial is the in-order
// sum of the 8 wave sums, via LDS.
template <bool kBF16, bool kScore>
__global__ __launch_bounds__(512, 2) void k_quantize(
    const void* __restrict__ xv, int64_t rows, int64_t K, int64_t ldx,
    const uint32_t* __restrict__ amax_partial, int n_partial, const float* __restrict__ amax_in,
    uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale,
    float* __restrict__ chunk_partial, uint32_t* __restrict__ status) {
  __shared__ float s_part[kScore ? 8 * kQCols : 1];
  __shared__ uint32_t s_slot[512 * (kBF16 ? 8 : 16)];
  __shared__ float s_amax;
  const int item = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* slot = s_slot + threadIdx.x * (kBF16 ? 8 : 16);

  const int64_t nblk = K >> 4;
  const int64_t blk = (int64_t)blockIdx.x * kQBlocksPerWave + lane;
  const int64_t r0 = (int64_t)blockIdx.y * kQRows + wave * kQSub;
  const bool active = blk < nblk;
  const int nrows = (int)max<int64_t>(0, min<int64_t>(kQSub, rows - r0));
  const int64_t row0 = (int64_t)item * rows + r0;
  const int64_t last = row0 + max(nrows, 1) - 1;
  // first rows in flight before the tensor amax is known
  RowBlock<kBF16> b0, b1, b2;
  if (active && nrows > 0) {
    b0.load(xv, row0, ldx, blk);
    b1.load(xv, min(row0 + 1, last), ldx, blk);
    b2.load(xv, min(row0 + 2, last), ldx, blk);
  }

  {
    // Tensor amax: every thread loads its share of the pass-1 partials at once.
    __shared__ uint32_t s_wmax[8];
    uint32_t m = 0;
    if (amax_in) {
      m = __float_as_uint(amax_in[item]);
    } else {
      const uint32_t* p = amax_partial + (int64_t)item * n_partial;
      for (int i = threadIdx.x; i < n_partial; i += 512) m = max(m, p[i]);
      m = wave_max_u32(m);
    }
    if (lane == 0) s_wmax[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t r = s_wmax[0];
#pragma unroll
      for (int w = 1; w < 8; ++w) r = max(r, s_wmax[w]);
      s_amax = __uint_as_float(r);
    }
  }
  __syncthreads();
  const float amax = s_amax;
  // s_t = fl32(amax / 2688): the fp64 quotient rounded to fp32 equals the
  // correctly rounded fp32 quotient (53 >= 2*24 + 2).
  const float s_t = (float)((double)amax / 2688.0);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) tensor_scale[item] = s_t;
  const double six_st = 6.0 * (double)s_t;  // exact
  // Extreme tensor scales would overflow the fp32 reciprocals: decide all in fp64.
  const bool fast = (s_t >= 0x1p-100f) && (s_t <= 0x1p100f);
  const float g = fast ? (float)(1.0 / six_st) : 0.0f;
  const float inv_st = fast ? (float)(1.0 / (double)s_t) : 0.0f;

  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
  uint32_t bad = 0;

  if (active && !fast) {
    const RowsResult res = quantize_rows_exact<kBF16, kScore>(xv, row0, nrows, K, ldx, blk, s_t,
                                                              six_st, codes, scales, slot);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = res.acc[j];
    bad = res.bad;
  } else if (active && nrows > 0) {
    // Row addresses advance by adds (no 64-bit multiply per row); refills
    // past the sub-chunk's last row are clamped to it.
    const int64_t xrow = ldx * (kBF16 ? 2 : 4), crow = K >> 1;
    const char* xp = static_cast<const char*>(xv) + (row0 * ldx + blk * 16) * (kBF16 ? 2 : 4);
    const char* const xlast = xp + (last - row0) * xrow;
    uint8_t* cp = codes + row0 * crow + blk * 8;
    uint8_t* sp = scales + row0 * nblk + blk;
    auto process = [&](const RowBlock<kBF16>& rb, uint8_t* c_at, uint8_t* s_at) {
      uint32_t sc;
      uint2 cw;
      encode_block_fast<kBF16, kScore>(rb, s_t, g, inv_st, sc, cw, acc, bad, slot);
      *reinterpret_cast<uint2*>(c_at) = cw;
      *s_at = (uint8_t)sc;
    };
    auto clamp = [&](const char* a) { return a < xlast ? a : xlast; };
    // Three rotating row buffers: row rr + 3 is loaded into a buffer right
    // after that buffer's row is processed.  Refill addresses are clamped to
    // the last row instead of branching, so no load sits under a branch and
    // the waits the compiler places stay exact.  Rows past nrows are loaded
    // (clamped) but never processed.
#pragma unroll 1
    for (int rr = 0; rr < nrows; rr += 3) {
      process(b0, cp, sp);
      b0.load_at(clamp(xp + 3 * xrow));
      __builtin_amdgcn_sched_barrier(0);
      if (rr + 1 < nrows) process(b1, cp + crow, sp + nblk);
      b1.load_at(clamp(xp + 4 * xrow));
      __builtin_amdgcn_sched_barrier(0);
      if (rr + 2 < nrows) process(b2, cp + 2 * crow, sp + 2 * nblk);
      b2.load_at(clamp(xp + 5 * xrow));
      __builtin_amdgcn_sched_barrier(0);
      xp += 3 * xrow;
      cp += 3 * crow;
      sp += 3 * nblk;
    }
  }

  if (kScore) {
#pragma unroll
    for (int j = 0; j < 16; ++j) s_part[wave * kQCols + lane * 16 + j] = acc[j];
    __syncthreads();
    for (int cc = threadIdx.x; cc < kQCols; cc += 512) {
      const int64_t col = (int64_t)blockIdx.x * kQCols + cc;
      if (col < K) {
        float P = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) P += s_part[w * kQCols + cc];
        chunk_partial[(int64_t)blockIdx.y * K + col] = P;
      }
    }
  }
  if (wave_or_u32(bad) && lane == 0) atomicOr(status, (uint32_t)NVQ_STATUS_NONFINITE);
}

// Scored quantization with one 16-element block per thread, for tensors
// whose row tile would leave CUs idle (few rows): workgroup = one 128-row
// score chunk x 64 columns, thread t = row t / 4, block column t % 4.  Each
// thread writes its block's 16 residual magnitudes to LDS; lane c of wave w
// then adds column c over rows 16 w .. 16 w + 15 in order (a sub-chunk sum),
// and thread c < 64 adds the 8 sub-chunk sums in order: the row tile's order,
// so the chunk partials, and the scores after k_score_reduce, are
// bit-identical to the row tile's.  Sixteen times the threads of the row
// tile for the same bytes.
constexpr int kTbCols = 64;
// k_quantize_tb runs when the row tile would have fewer workgroups than a
// third of the CUs (measured: at 64 row-tile workgroups on 256 CUs the
// thread-per-block tile wins, 28 against 31 us; at 112 and above the row tile)
constexpr int kTbCuDiv = 3;
template <bool kBF16>
__global__ __launch_bounds__(512) void k_quantize_tb(
    const void* __restrict__ xv, int64_t rows, int64_t K, int64_t ldx,
    const uint32_t* __restrict__ amax_partial, int n_partial, const float* __restrict__ amax_in,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ tensor_scale,
    float* __restrict__ chunk_partial, uint32_t* __restrict__ status) {
  __shared__ float s_r[kQRows][kTbCols + 1];  // +1: a write instruction's rows hit distinct banks
  __shared__ float s_sub[kQRows / kQSub][kTbCols];
  __shared__ uint32_t s_slot[512 * (kBF16 ? 8 : 16)];
  __shared__ uint32_t s_wmax[8];
  __shared__ float s_amax;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int rr = t >> 2, b = t & 3;
  uint32_t* slot = s_slot + t * (kBF16 ? 8 : 16);
  const int64_t nblk = K >> 4;
  const int64_t blk = (int64_t)blockIdx.x * (kTbCols / 16) + b;
  const int64_t row = (int64_t)blockIdx.y * kQRows + rr;
  const bool active = blk < nblk && row < rows;
  RowBlock<kBF16> rb;
  if (active) rb.load(xv, row, ldx, blk);  // in flight before the tensor amax is known

  {
    uint32_t m = 0;
    if (amax_in) {
      m = __float_as_uint(amax_in[0]);
    } else {
      for (int i = t; i < n_partial; i += 512) m = max(m, amax_partial[i]);
      m = wave_max_u32(m);
    }
    if (lane == 0) s_wmax[wave] = m;
    __syncthreads();
    if (t == 0) {
      uint32_t r = s_wmax[0];
#pragma unroll
      for (int w = 1; w < 8; ++w) r = max(r, s_wmax[w]);
      s_amax = __uint_as_float(r);
    }
  }
  __syncthreads();
  const float amax = s_amax;
  const float s_t = (float)((double)amax / 2688.0);  // fl32(amax / 2688), as in k_quantize
  if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0) tensor_scale[0] = s_t;
  const double six_st = 6.0 * (double)s_t;
  const bool fast = (s_t >= 0x1p-100f) && (s_t <= 0x1p100f);
  const float g = fast ? (float)(1.0 / six_st) : 0.0f;
  const float inv_st = fast ? (float)(1.0 / (double)s_t) : 0.0f;

  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
  uint32_t bad = 0;
  if (active) {
    uint32_t sc;
    uint2 cw;
    if (fast)
      encode_block_fast<kBF16, true>(rb, s_t, g, inv_st, sc, cw, acc, bad, slot);
    else
      encode_block_exact<kBF16, true>(rb, s_t, six_st, sc, cw, acc, bad, slot);
    *reinterpret_cast<uint2*>(codes + row * (K >> 1) + blk * 8) = cw;
    scales[row * nblk + blk] = (uint8_t)sc;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) s_r[rr][16 * b + j] = acc[j];
  __syncthreads();
  {
    // wave w: the sub-chunk sums of rows 16 w .. 16 w + 15, lane = column
    const int nr = (int)max<int64_t>(0, min<int64_t>(kQRows, rows - (int64_t)blockIdx.y * kQRows));
    float v[kQSub];
#pragma unroll
    for (int q = 0; q < kQSub; ++q) v[q] = s_r[kQSub * wave + q][lane];
    float sub = 0.0f;
#pragma unroll
    for (int q = 0; q < kQSub; ++q)
      if (kQSub * wave + q < nr) sub += v[q];
    s_sub[wave][lane] = sub;
  }
  __syncthreads();
  if (t < kTbCols) {
    const int64_t col = (int64_t)blockIdx.x * kTbCols + t;
    float P = 0.0f;
#pragma unroll
    for (int w = 0; w < kQRows / kQSub; ++w) P += s_sub[w][t];
    if (col < K) chunk_partial[(int64_t)blockIdx.y * K + col] = P;
  }
  if (wave_or_u32(bad) && lane == 0) atomicOr(status, (uint32_t)NVQ_STATUS_NONFINITE);
}

// Score-free quantization: without residual sums there is no row order to
// keep, so thread t of item z takes blocks t, t + T, t + 2T, ... of the item's
// flat block list (block f = elements 16f..16f+15 of the row-major tensor,
// codes at byte 8f, scale at byte f).  Consecutive lanes read consecutive
// blocks whatever K is; with the row-major tile of k_quantize a K of 128
// would leave 56 of 64 lanes idle.  One block in flight ahead, clamped to
// the item's last block.
constexpr int kFlatThreads = 256;
constexpr int kFlatBlocksPerThread = 4;

template <bool kBF16>
__global__ __launch_bounds__(kFlatThreads) void k_quantize_flat(
    const void* __restrict__ xv, int64_t nb_item, const uint32_t* __restrict__ amax_partial,
    int n_partial, const float* __restrict__ amax_in, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale,
    uint32_t* __restrict__ status) {
  constexpr int64_t kBlockBytes = 16 * (kBF16 ? 2 : 4);
  __shared__ uint32_t s_slot[kFlatThreads * (kBF16 ? 8 : 16)];
  __shared__ uint32_t s_wmax[kFlatThreads / kWave];
  __shared__ float s_amax;
  const int item = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* slot = s_slot + threadIdx.x * (kBF16 ? 8 : 16);
  const int64_t base = (int64_t)item * nb_item;
  const char* xb = static_cast<const char*>(xv) + base * kBlockBytes;
  const int64_t stride = (int64_t)gridDim.x * kFlatThreads;
  const int64_t last = nb_item - 1;
  int64_t f = (int64_t)blockIdx.x * kFlatThreads + threadIdx.x;
  RowBlock<kBF16> cur;
  cur.load_at(xb + min(f, last) * kBlockBytes);

  uint32_t m = 0;
  if (amax_in) {
    m = __float_as_uint(amax_in[item]);
  } else {
    const uint32_t* p = amax_partial + (int64_t)item * n_partial;
    for (int i = threadIdx.x; i < n_partial; i += kFlatThreads) m = max(m, p[i]);
    m = wave_max_u32(m);
  }
  if (lane == 0) s_wmax[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = s_wmax[0];
#pragma unroll
    for (int w = 1; w < kFlatThreads / kWave; ++w) r = max(r, s_wmax[w]);
    s_amax = __uint_as_float(r);
  }
  __syncthreads();
  // s_t exactly as in k_quantize
  const float s_t = (float)((double)s_amax / 2688.0);
  if (blockIdx.x == 0 && threadIdx.x == 0) tensor_scale[item] = s_t;
  const double six_st = 6.0 * (double)s_t;
  const bool fast = (s_t >= 0x1p-100f) && (s_t <= 0x1p100f);
  const float g = fast ? (float)(1.0 / six_st) : 0.0f;
  const float inv_st = fast ? (float)(1.0 / (double)s_t) : 0.0f;

  float acc[16];  // no residual sums on this path
  uint32_t bad = 0;
  uint2* cw_out = reinterpret_cast<uint2*>(codes) + base;
  uint8_t* sc_out = scales + base;
#pragma unroll 1
  while (f < nb_item) {
    const int64_t fn = f + stride;
    RowBlock<kBF16> nxt;
    nxt.load_at(xb + min(fn, last) * kBlockBytes);
    uint32_t sc;
    uint2 cw;
    if (fast)
      encode_block_fast<kBF16, false>(cur, s_t, g, inv_st, sc, cw, acc, bad, slot);
    else
      encode_block_exact<kBF16, false>(cur, s_t, six_st, sc, cw, acc, bad, slot);
    cw_out[f] = cw;
    sc_out[f] = (uint8_t)sc;
    cur = nxt;
    f = fn;
  }
  if (wave_or_u32(bad) && lane == 0) atomicOr(status, (uint32_t)NVQ_STATUS_NONFINITE);
}

// score[c] = sum over chunks j ascending of P[j][c] (fp32, sequential).  One
// column per thread, 64-thread workgroups so the columns spread over many CUs;
// the partials of a group of 64 chunks are all loaded before the in-order sum.
// score[c] = sum over chunks j = 0, 1, ... of partial[j][c], strictly in
// chunk order (one fp32 add per chunk).  The add chain is inherently serial,
// so the loads are spread over a whole workgroup: a workgroup owns 32
// columns; all four waves stream blocks of 256 chunks into a transposed,
// double-buffered LDS tile (32 loads in flight per thread), while lanes
// 0..31 of wave 0 add the previous block in order, four chunks per LDS read.
constexpr int kScoreCols = 32, kScoreBlock = 256, kScorePitch = kScoreBlock + 4;
__global__ __launch_bounds__(256) void k_score_reduce(const float* __restrict__ partial,
                                                     int64_t nchunks, int64_t K,
                                                     float* __restrict__ score) {
  __shared__ __attribute__((aligned(16))) float tile[2][kScoreCols * kScorePitch];
  const int t = threadIdx.x, col = t & 31, r0 = t >> 5;  // chunk rows r0 + 8 i
  const int64_t c = (int64_t)blockIdx.x * kScoreCols + col;
  const int64_t cl = min<int64_t>(c, K - 1);  // columns past K load a valid one, never stored
  if (nchunks <= 0) {  // no rows: every sum is empty
    if (t < 32 && c < K) score[c] = 0.0f;
    return;
  }
  const int nb = (int)((nchunks + kScoreBlock - 1) / kScoreBlock);
  float v[kScoreBlock / 8];
  auto load = [&](int b) {
    const int64_t j0 = (int64_t)b * kScoreBlock;
#pragma unroll
    for (int i = 0; i < kScoreBlock / 8; ++i) {
      const int64_t j = min<int64_t>(j0 + r0 + 8 * i, nchunks - 1);
      v[i] = partial[j * K + cl];
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kScoreBlock / 8; ++i) tile[buf][col * kScorePitch + r0 + 8 * i] = v[i];
  };
  float acc = 0.0f;
  load(0);
  put(0);
  __syncthreads();
  for (int b = 0; b < nb; ++b) {
    if (b + 1 < nb) load(b + 1);
    if (t < 32) {
      const int n = (int)min<int64_t>(kScoreBlock, nchunks - (int64_t)b * kScoreBlock);
      const float* src = &tile[b & 1][col * kScorePitch];
      int j = 0;
      for (; j + 4 <= n; j += 4) {
        const float4 q = *reinterpret_cast<const float4*>(src + j);
        acc += q.x;
        acc += q.y;
        acc += q.z;
        acc += q.w;
      }
      for (; j < n; ++j) acc += src[j];
    }
    if (b + 1 < nb) put((b + 1) & 1);
    __syncthreads();
  }
  if (t < 32 && c < K) score[c] = acc;
}

// Recomputes the residual sub-chunk/chunk partials from an existing NVFP4
// record (no requantization): same order as k_quantize.
template <bool kBF16>
__global__ __launch_bounds__(512) void k_resid_partials(const void* __restrict__ xv, int64_t rows,
                                                       int64_t K, int64_t ldx,
                                                       const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ tensor_scale,
                                                       float* __restrict__ chunk_partial) {
  __shared__ float s_part[8 * kQCols];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float s_t = tensor_scale[0];
  const int64_t nblk = K >> 4;
  const int64_t blk = (int64_t)blockIdx.x * kQBlocksPerWave + lane;
  const int64_t r0 = (int64_t)blockIdx.y * kQRows + wave * kQSub;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
  if (blk < nblk) {
    for (int rr = 0; rr < kQSub; ++rr) {
      const int64_t r = r0 + rr;
      if (r >= rows) break;
      const uint2 cwv = *reinterpret_cast<const uint2*>(codes + r * (K >> 1) + blk * 8);
      const uint32_t cw[2] = {cwv.x, cwv.y};
      const float s_b = e4m3_to_f32(scales[r * nblk + blk]);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t c = blk * 16 + j;
        const float xj = kBF16 ? bf16_to_f32(static_cast<const uint16_t*>(xv)[r * ldx + c])
                               : static_cast<const float*>(xv)[r * ldx + c];
        const uint32_t nib = (cw[j >> 3] >> (4 * (j & 7))) & 7u;
        const float v = (e2m1_mag(nib) * s_b) * s_t;
        acc[j] += fabsf(fabsf(xj) - v);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) s_part[wave * kQCols + lane * 16 + j] = acc[j];
  __syncthreads();
  for (int cc = threadIdx.x; cc < kQCols; cc += 512) {
    const int64_t col = (int64_t)blockIdx.x * kQCols + cc;
    if (col < K) {
      float P = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) P += s_part[w * kQCols + cc];
      chunk_partial[(int64_t)blockIdx.y * K + col] = P;
    }
  }
}

// Order-preserving map of fp32 bits to uint32 (larger float -> larger key;
// -0 and +0 map to the same key, so they tie like equal values).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  const uint32_t u = __float_as_uint(f) == 0x80000000u ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of K scores by (score desc, index asc) with a bitonic sort of 64-bit
// keys in LDS; one workgroup.  Kp = padded power of two.  Used for k > 1024.
__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ score, int K, int Kp,
                                              int k, int32_t* __restrict__ idx_out) {
  extern __shared__ uint64_t keys[];
  for (int i = threadIdx.x; i < Kp; i += 1024)
    keys[i] = (i < K) ? (((uint64_t)f32_order_key(score[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i))
                      : 0ull;
  __syncthreads();
  for (int size = 2; size <= Kp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (Kp >> 1); i += 1024) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a < b) == up) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = threadIdx.x; j < k; j += 1024)
    idx_out[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[j] & 0xFFFFFFFFull));
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkMaxK = 1024;
constexpr int kTopkRegs = 8;  // keys per thread held in registers when K <= 8192

// Top-k (k <= 1024) of K scores by (score desc, index asc); one workgroup.
// Radix select on the order keys, 8 bits per pass from the top: each pass
// histograms the digit of the keys that match the prefix found so far and
// picks the digit holding the k-th largest key.  The threshold key T ends up
// exact; every key above T is taken, and of the keys equal to T the needed
// number with the lowest indices (an index-ordered scan).  The k winners are
// then put in rank order by counting, for each, the winners with a larger
// (key, -index).  Thread t owns the contiguous index range [t C, t C + C);
// with kRegs its keys stay in registers (C <= 8), else every pass re-reads
// the scores.  All loops are bounded by K and k.
template <bool kRegs>
__global__ __launch_bounds__(kTopkThreads) void k_topk_radix(const float* __restrict__ score, int K,
                                                            int k, int32_t* __restrict__ idx_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_bin;     // chosen digit
  __shared__ uint32_t s_above;   // keys above the chosen digit (within the prefix)
  __shared__ uint32_t s_cnt;     // winners placed so far
  __shared__ uint32_t s_wave[kTopkThreads / 64];
  __shared__ uint64_t sel[kTopkMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = (K + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(K, tid * C), i1 = min(K, i0 + C);
  uint32_t kr[kRegs ? kTopkRegs : 1];
  if (kRegs) {
#pragma unroll
    for (int j = 0; j < kTopkRegs; ++j) kr[j] = (i0 + j < i1) ? f32_order_key(score[i0 + j]) : 0u;
  }
  auto key_at = [&](int j) -> uint32_t {  // j-th key of this thread's range
    if (kRegs) {
      uint32_t v = kr[0];
#pragma unroll
      for (int t = 1; t < kTopkRegs; ++t) v = (j == t) ? kr[t] : v;
      return v;
    }
    return f32_order_key(score[i0 + j]);
  };

  uint32_t prefix = 0, mask = 0, need = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    if (kRegs) {
#pragma unroll
      for (int j = 0; j < kTopkRegs; ++j)
        if (i0 + j < i1 && (kr[j] & mask) == prefix) atomicAdd(&hist[(kr[j] >> shift) & 255u], 1u);
    } else {
      for (int j = 0; j < i1 - i0; ++j) {
        const uint32_t key = key_at(j);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 4l..4l+3; suffix sums over lanes from the top
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                     h3 = hist[4 * lane + 3];
      const uint32_t own = h0 + h1 + h2 + h3;
      uint32_t suf = own;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_down((int)suf, d, 64);
        if (lane + d < 64) suf += o;
      }
      const uint32_t above = suf - own;  // keys in digits of higher lanes
      // the k-th largest lies in this lane's digits iff above < need <= suf
      if (above < need && need <= suf) {
        uint32_t a = above, dsel = 4 * lane + 3;
        if (a + h3 < need) {
          a += h3;
          dsel = 4 * lane + 2;
          if (a + h2 < need) {
            a += h2;
            dsel = 4 * lane + 1;
            if (a + h1 < need) {
              a += h1;
              dsel = 4 * lane;
            }
          }
        }
        s_bin = dsel;
        s_above = a;
      }
    }
    __syncthreads();
    prefix |= s_bin << shift;
    mask |= 255u << shift;
    need -= s_above;
    __syncthreads();
  }
  // prefix = T, the k-th largest key; take all keys > T and the `need`
  // lowest-index keys == T, by an exclusive scan of the equal counts in
  // index order.
  uint32_t eq = 0;
  if (kRegs) {
#pragma unroll
    for (int j = 0; j < kTopkRegs; ++j) eq += (i0 + j < i1 && kr[j] == prefix) ? 1u : 0u;
  } else {
    for (int j = 0; j < i1 - i0; ++j) eq += key_at(j) == prefix;
  }
  uint32_t inc = eq;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (tid == 0) s_cnt = 0;
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  uint32_t base = inc - eq;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  auto place = [&](uint32_t key, int i) {
    bool take = key > prefix;
    if (key == prefix) take = (base++ < need);
    if (take) {
      const uint32_t slot = atomicAdd(&s_cnt, 1u);
      if (slot < (uint32_t)kTopkMaxK)
        sel[slot] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
    }
  };
  if (kRegs) {
#pragma unroll
    for (int j = 0; j < kTopkRegs; ++j)
      if (i0 + j < i1) place(kr[j], i0 + j);
  } else {
    for (int j = 0; j < i1 - i0; ++j) place(key_at(j), i0 + j);
  }
  __syncthreads();
  if (tid < k) {
    const uint64_t mine = sel[tid];
    int rank = 0;
    for (int j = 0; j < k; ++j) rank += sel[j] > mine;
    idx_out[rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)(mine & 0xFFFFFFFFull));
  }
}

// resid[m, j] = bf16(fl32(x[m, idx[j]] - v[m, idx[j]])).
template <bool kBF16>
__global__ __launch_bounds__(256) void k_resid_gather(const void* __restrict__ xv, int64_t rows,
                                                     int64_t K, int64_t ldx,
                                                     const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     const float* __restrict__ tensor_scale,
                                                     const int32_t* __restrict__ idx, int k,
                                                     uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * k) return;
  const int64_t m = i / k;
  const int64_t c = idx[i - m * k];
  const float xj = kBF16 ? bf16_to_f32(static_cast<const uint16_t*>(xv)[m * ldx + c])
                         : static_cast<const float*>(xv)[m * ldx + c];
  const uint32_t byte = codes[m * (K >> 1) + (c >> 1)];
  const uint32_t nib = (c & 1) ? (byte >> 4) : (byte & 15u);
  const uint32_t mi = nib & 7u;
  const float mag = (e2m1_mag(mi) * e4m3_to_f32(scales[m * (K >> 4) + (c >> 4)])) * tensor_scale[0];
  const float v = (nib & 8u) ? -mag : mag;
  const float r = xj - v;
  out[i] = (uint16_t)f32_to_bf16_rne(r);
}

// Dequantize 8 elements (one code word) per thread.
// y = sign * fl32(fl32(G s_b) s_t) for one 16-element block per thread: 8
// bytes of codes and one scale in, 32 (bf16) or 64 (fp32) bytes out; the
// item (tensor scale) comes from the grid, not a division.
template <bool kOutBF16>
__global__ __launch_bounds__(256) void k_dequant(const uint2* __restrict__ codes,
                                                const uint8_t* __restrict__ scales,
                                                const float* __restrict__ tensor_scale,
                                                int64_t blocks_per_item, void* __restrict__ y) {
  const int64_t in_item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (in_item >= blocks_per_item) return;
  const int64_t blk = (int64_t)blockIdx.y * blocks_per_item + in_item;
  const float s_t = tensor_scale[blockIdx.y];
  const float s_b = e4m3_to_f32(scales[blk]);
  const uint2 cw = codes[blk];
  float v[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w = h ? cw.y : cw.x;
    float2 g[4];
    g[0] = fp4_pair_to_f32<0>(w);
    g[1] = fp4_pair_to_f32<1>(w);
    g[2] = fp4_pair_to_f32<2>(w);
    g[3] = fp4_pair_to_f32<3>(w);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * h + 2 * j] = (g[j].x * s_b) * s_t;
      v[8 * h + 2 * j + 1] = (g[j].y * s_b) * s_t;
    }
  }
  if (kOutBF16) {
    uint4* o = static_cast<uint4*>(y) + 2 * blk;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float* u = v + 8 * q;
      o[q] = make_uint4(f32_to_bf16_rne(u[0]) | (f32_to_bf16_rne(u[1]) << 16),
                        f32_to_bf16_rne(u[2]) | (f32_to_bf16_rne(u[3]) << 16),
                        f32_to_bf16_rne(u[4]) | (f32_to_bf16_rne(u[5]) << 16),
                        f32_to_bf16_rne(u[6]) | (f32_to_bf16_rne(u[7]) << 16));
    }
  } else {
    float4* o = static_cast<float4*>(y) + 4 * blk;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
}

struct QuantLayout {
  int nwg;        // pass-1 workgroups per item
  int n_partial;  // pass-1 wave partials per item
  int64_t n_partial_tiles;  // partials of the tiled pass 1 (one item, scored)
  int64_t nchunks;
  size_t bytes;
  uint32_t* status;
  uint32_t* amax_partial;
  float* chunk_partial;
};

QuantLayout quant_layout(void* ws, int64_t batch, int64_t rows, int64_t K, int x_dtype) {
  QuantLayout L;
  const int64_t elem_bytes = (x_dtype == NVQ_BF16) ? 2 : 4;
  const int64_t vec_per_item = rows * K * elem_bytes / 16;
  L.nwg = amax_wg_per_item(batch, vec_per_item);
  L.n_partial = L.nwg * kAmaxWaves;
  L.nchunks = (rows + kQRows - 1) / kQRows;
  // the tiled amax pass (one item with a score, at most 1024 quantize
  // workgroups) writes one partial per wave of the quantize grid
  L.n_partial_tiles = (int64_t)((K / 16 + kQBlocksPerWave - 1) / kQBlocksPerWave) * L.nchunks * 8;
  WsCarve c(ws);
  L.amax_partial = c.take<uint32_t>((size_t)std::max<int64_t>(
      (int64_t)batch * L.n_partial, std::min<int64_t>(L.n_partial_tiles, 1024 * 8)));
  L.chunk_partial = c.take<float>((size_t)L.nchunks * K);
  L.bytes = c.off;
  L.status = c.status();
  return L;
}

}  // namespace

int topk_launch(const float* score, int64_t K, int32_t k, int32_t* idx, hipStream_t s) {
  if (k == 0) return NVQ_OK;
  if (K > INT32_MAX) return NVQ_EUNSUPPORTED;
  if (k <= kTopkMaxK) {
    if (K <= (int64_t)kTopkThreads * kTopkRegs)
      hipLaunchKernelGGL(k_topk_radix<true>, dim3(1), dim3(kTopkThreads), 0, s, score, (int)K, (int)k,
                         idx);
    else
      hipLaunchKernelGGL(k_topk_radix<false>, dim3(1), dim3(kTopkThreads), 0, s, score, (int)K, (int)k,
                         idx);
    return last_launch();
  }
  int Kp = 1;
  while (Kp < K) Kp <<= 1;
  if (Kp > 8192) return NVQ_EUNSUPPORTED;  // 64 KB of LDS keys
  hipLaunchKernelGGL(k_topk, dim3(1), dim3(1024), Kp * sizeof(uint64_t), s, score, (int)K, Kp, (int)k,
                     idx);
  return last_launch();
}

}  // namespace nvq

using namespace nvq;

extern "C" size_t nvfp4_quantize_workspace_bytes(int64_t batch, int64_t rows, int64_t K) {
  if (batch <= 0 || rows < 0 || K <= 0) return kAlign;
  // sized for the larger (fp32) element type so one query serves both dtypes
  return std::max(quant_layout(nullptr, batch, rows, K, NVQ_F32).bytes,
                  quant_layout(nullptr, batch, rows, K, NVQ_BF16).bytes);
}

namespace nvq {
namespace {
// Host-side argument checks of nvfp4_quantize apart from the workspace (no
// HIP call).  ldx == 0 becomes K.
int quantize_check_args(const void* x, int x_dtype, int64_t batch, int64_t rows, int64_t K,
                        int64_t& ldx, const uint8_t* codes, const uint8_t* scales,
                        const float* tensor_scale, const float* chan_score) {
  if (!tensor_scale || (rows != 0 && (!x || !codes || !scales))) return NVQ_EINVAL;
  if (x_dtype != NVQ_F32 && x_dtype != NVQ_BF16) return NVQ_EINVAL;
  if (batch <= 0 || batch > 65535 || rows < 0 || K <= 0 || (K & 15)) return NVQ_ESHAPE;
  if (ldx == 0) ldx = K;
  if (ldx < K) return NVQ_ESHAPE;
  if (chan_score && batch != 1) return NVQ_ESHAPE;
  const int64_t eb = (x_dtype == NVQ_BF16) ? 2 : 4;
  if (!aligned16(x) || ((uintptr_t)codes & 7u) || (ldx * eb) % 16) return NVQ_EALIGN;
  return NVQ_OK;
}
}  // namespace
}  // namespace nvq

extern "C" int nvfp4_quantize(const void* x, int x_dtype, int64_t batch, int64_t rows, int64_t K,
                              int64_t ldx, const float* amax_in, uint8_t* codes, uint8_t* scales,
                              float* tensor_scale, float* chan_score, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!ws) return NVQ_EINVAL;
  if (int rc = quantize_check_args(x, x_dtype, batch, rows, K, ldx, codes, scales, tensor_scale,
                                   chan_score))
    return rc;
  const int64_t eb = (x_dtype == NVQ_BF16) ? 2 : 4;
  if (!aligned256(ws)) return NVQ_EALIGN;
  QuantLayout L = quant_layout(ws, batch, rows, K, x_dtype);
  if (ws_bytes < L.bytes) return NVQ_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = x_dtype == NVQ_BF16;
  if (rows == 0) {
    const int64_t n = std::max<int64_t>(batch, chan_score ? K : 0);
    hipLaunchKernelGGL(k_quant_empty, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, amax_in, batch,
                       tensor_scale, chan_score, K, L.status);
    return last_launch();
  }
  const bool score = chan_score != nullptr;
  const dim3 qgrid((unsigned)((K / 16 + kQBlocksPerWave - 1) / kQBlocksPerWave), (unsigned)L.nchunks,
                   (unsigned)batch);
  int n_partial = L.n_partial;
  // The tiled amax pass pays off when the whole quantize grid is resident at
  // once (two 512-thread workgroups per CU), so both launches place workgroup
  // i on the same XCD at about the same time; larger grids take the flat pass.
  const int64_t qwgs = (int64_t)qgrid.x * qgrid.y;
  // A scored row tile with few workgroups leaves the chip mostly idle (each
  // wave walks 16 rows); the thread-per-block tile computes the same chunk
  // partials with sixteen times the threads, after the flat amax.
  const bool tb = score && qwgs * kTbCuDiv < (int64_t)device_cu_count();
  if (!amax_in && score && !tb && qwgs <= 1024 && qwgs <= 2 * device_cu_count()) {
    n_partial = (int)L.n_partial_tiles;
    if (bf16)
      hipLaunchKernelGGL(k_amax_tiles<true>, dim3(qgrid.x, qgrid.y), dim3(512), 0, s, x, rows, K, ldx,
                         L.amax_partial, L.status);
    else
      hipLaunchKernelGGL(k_amax_tiles<false>, dim3(qgrid.x, qgrid.y), dim3(512), 0, s, x, rows, K, ldx,
                         L.amax_partial, L.status);
  } else if (!amax_in) {
    dim3 grid(L.nwg, (unsigned)batch);
    const uint4* xv = static_cast<const uint4*>(x);
    if (ldx == K) {
      const int64_t vec_per_item = rows * K * eb / 16;
      if (bf16)
        hipLaunchKernelGGL(k_amax<true>, grid, dim3(kAmaxThreads), 0, s, xv, vec_per_item, L.nwg,
                           L.amax_partial, L.status);
      else
        hipLaunchKernelGGL(k_amax<false>, grid, dim3(kAmaxThreads), 0, s, xv, vec_per_item, L.nwg,
                           L.amax_partial, L.status);
    } else {
      const int64_t vpr = K * eb / 16, ldv = ldx * eb / 16;
      if (bf16)
        hipLaunchKernelGGL(k_amax_rows<true>, grid, dim3(kAmaxThreads), 0, s, xv, rows, vpr, ldv,
                           L.nwg, L.amax_partial, L.status);
      else
        hipLaunchKernelGGL(k_amax_rows<false>, grid, dim3(kAmaxThreads), 0, s, xv, rows, vpr, ldv,
                           L.nwg, L.amax_partial, L.status);
    }
  } else {
    hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(1), 0, s, L.status);
  }
  if (int rc = last_launch()) return rc;
  // The flat score-free kernel walks the item as one run of blocks, so it
  // takes dense tensors only; row-strided ones go through the row tile.
  if (!score && ldx == K) {
    const int64_t nb_item = rows * (K / 16);
    const int64_t per_wg = (int64_t)kFlatThreads * kFlatBlocksPerThread;
    const int64_t nwg = std::min<int64_t>(std::max<int64_t>(1, (nb_item + per_wg - 1) / per_wg), 65535);
    dim3 fgrid((unsigned)nwg, (unsigned)batch);
    if (bf16)
      hipLaunchKernelGGL(k_quantize_flat<true>, fgrid, dim3(kFlatThreads), 0, s, x, nb_item,
                         L.amax_partial, L.n_partial, amax_in, codes, scales, tensor_scale, L.status);
    else
      hipLaunchKernelGGL(k_quantize_flat<false>, fgrid, dim3(kFlatThreads), 0, s, x, nb_item,
                         L.amax_partial, L.n_partial, amax_in, codes, scales, tensor_scale, L.status);
    return last_launch();
  }
  if (tb) {
    const dim3 tgrid((unsigned)((K + kTbCols - 1) / kTbCols), (unsigned)L.nchunks);
    if (bf16)
      hipLaunchKernelGGL(k_quantize_tb<true>, tgrid, dim3(512), 0, s, x, rows, K, ldx, L.amax_partial,
                         n_partial, amax_in, codes, scales, tensor_scale, L.chunk_partial, L.status);
    else
      hipLaunchKernelGGL(k_quantize_tb<false>, tgrid, dim3(512), 0, s, x, rows, K, ldx, L.amax_partial,
                         n_partial, amax_in, codes, scales, tensor_scale, L.chunk_partial, L.status);
    if (int rc = last_launch()) return rc;
    hipLaunchKernelGGL(k_score_reduce, dim3((unsigned)((K + kScoreCols - 1) / kScoreCols)), dim3(256), 0, s,
                       L.chunk_partial, L.nchunks, K, chan_score);
    return last_launch();
  }
#define NVQ_LAUNCH_Q(B, S)                                                                    \
  hipLaunchKernelGGL((k_quantize<B, S>), qgrid, dim3(512), 0, s, x, rows, K, ldx, L.amax_partial, \
                     n_partial, amax_in, codes, scales, tensor_scale, L.chunk_partial, L.status)
  if (bf16) {
    if (score) NVQ_LAUNCH_Q(true, true); else NVQ_LAUNCH_Q(true, false);
  } else {
    if (score) NVQ_LAUNCH_Q(false, true); else NVQ_LAUNCH_Q(false, false);
  }
#undef NVQ_LAUNCH_Q
  if (int rc = last_launch()) return rc;
  if (score) {
    hipLaunchKernelGGL(k_score_reduce, dim3((unsigned)((K + kScoreCols - 1) / kScoreCols)), dim3(256), 0, s,
                       L.chunk_partial, L.nchunks, K, chan_score);
    return last_launch();
  }
  return NVQ_OK;
}

// ------------------------------------------------------------------------
// Allocation-free variant of nvfp4_quantize.  Its scratch (status word, amax
// partials, residual chunk partials) is a file-scope device array: every GPU
// the library runs on holds one copy of kQuantScratchBytes until the process
// ends, and every call on that GPU shares it.  In host code `nvq_quant_scratch`
// names a host-side stand-in, so its device address is taken once per device
// with hipGetSymbolAddress and only that address reaches the kernels.
constexpr size_t kQuantScratchBytes = NVQ_QUANTIZE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char nvq_quant_scratch[kQuantScratchBytes];

namespace nvq {
namespace {
constexpr int kScratchMaxDevices = 64;
std::atomic<void*> g_quant_scratch[kScratchMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on each device; a racing second lookup stores the same value).
int quant_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVQ_EHIP;
  if (dev < 0 || dev >= kScratchMaxDevices) return NVQ_EUNSUPPORTED;
  void* p = g_quant_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(nvq_quant_scratch)) != hipSuccess || !p) return NVQ_EHIP;
    g_quant_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return NVQ_OK;
}
}  // namespace
}  // namespace nvq

extern "C" int nvfp4_quantize_noalloc(const void* x, int x_dtype, int64_t batch, int64_t rows,
                                      int64_t K, int64_t ldx, const float* amax_in, uint8_t* codes,
                                      uint8_t* scales, float* tensor_scale, float* chan_score,
                                      void* stream) {
  if (int rc = quantize_check_args(x, x_dtype, batch, rows, K, ldx, codes, scales, tensor_scale,
                                   chan_score))
    return rc;
  if (nvfp4_quantize_workspace_bytes(batch, rows, K) > kQuantScratchBytes) return NVQ_EWORKSPACE;
  void* ws = nullptr;
  if (int rc = quant_scratch(&ws)) return rc;
  return nvfp4_quantize(x, x_dtype, batch, rows, K, ldx, amax_in, codes, scales, tensor_scale,
                        chan_score, ws, kQuantScratchBytes, stream);
}

extern "C" int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                                const float* tensor_scale, int64_t batch, int64_t rows, int64_t K,
                                void* y, int y_dtype, void* stream) {
  if (y_dtype != NVQ_F32 && y_dtype != NVQ_BF16) return NVQ_EINVAL;
  if (batch <= 0 || batch > 65535 || rows < 0 || K <= 0 || (K & 15)) return NVQ_ESHAPE;
  const int64_t per_item = rows * (K / 16);
  if (per_item == 0) return NVQ_OK;
  if (!codes || !scales || !tensor_scale || !y) return NVQ_EINVAL;
  if (((uintptr_t)codes & 7u) || !aligned16(y)) return NVQ_EALIGN;
  if ((per_item + 255) / 256 > 0x7FFFFFFF) return NVQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((per_item + 255) / 256), (unsigned)batch);
  const uint2* cw = reinterpret_cast<const uint2*>(codes);
  if (y_dtype == NVQ_BF16)
    hipLaunchKernelGGL(k_dequant<true>, grid, dim3(256), 0, s, cw, scales, tensor_scale, per_item, y);
  else
    hipLaunchKernelGGL(k_dequant<false>, grid, dim3(256), 0, s, cw, scales, tensor_scale, per_item, y);
  return last_launch();
}

extern "C" size_t residual_topk_workspace_bytes(int64_t rows, int64_t K, int32_t k) {
  (void)k;
  if (rows < 0 || K <= 0) return kAlign;
  WsCarve c(nullptr);
  c.take<float>((size_t)((rows + kQRows - 1) / kQRows) * K);
  c.take<float>((size_t)K);
  return c.off;
}

extern "C" int residual_topk_channels(const void* x, int x_dtype, int64_t rows, int64_t K,
                                      int64_t ldx, const uint8_t* codes, const uint8_t* scales,
                                      const float* tensor_scale, const float* scores_in,
                                      float* scores_out, int32_t k, int32_t* idx_out,
                                      uint16_t* resid_out, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (x_dtype != NVQ_F32 && x_dtype != NVQ_BF16) return NVQ_EINVAL;
  if (rows < 0 || K <= 0 || (K & 15) || k < 0 || k > K) return NVQ_ESHAPE;
  if (ldx == 0) ldx = K;
  if (ldx < K) return NVQ_ESHAPE;
  if (k > 0 && !idx_out) return NVQ_EINVAL;
  if (!ws || !aligned256(ws)) return ws ? NVQ_EALIGN : NVQ_EINVAL;
  const bool need_record = !scores_in || resid_out;
  if (need_record && (!x || !codes || !scales || !tensor_scale)) return NVQ_EINVAL;
  WsCarve c(ws);
  const int64_t nchunks = (rows + kQRows - 1) / kQRows;
  float* chunk_partial = c.take<float>((size_t)nchunks * K);
  float* score_tmp = c.take<float>((size_t)K);
  if (ws_bytes < c.off) return NVQ_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = x_dtype == NVQ_BF16;
  const float* score = scores_in;
  if (!score) {
    float* dst = scores_out ? scores_out : score_tmp;
    if (rows > 0) {
      dim3 grid((unsigned)((K / 16 + kQBlocksPerWave - 1) / kQBlocksPerWave), (unsigned)nchunks);
      if (bf16)
        hipLaunchKernelGGL(k_resid_partials<true>, grid, dim3(512), 0, s, x, rows, K, ldx, codes,
                           scales, tensor_scale, chunk_partial);
      else
        hipLaunchKernelGGL(k_resid_partials<false>, grid, dim3(512), 0, s, x, rows, K, ldx, codes,
                           scales, tensor_scale, chunk_partial);
      if (int rc = last_launch()) return rc;
    }
    hipLaunchKernelGGL(k_score_reduce, dim3((unsigned)((K + kScoreCols - 1) / kScoreCols)), dim3(256), 0, s,
                       chunk_partial, nchunks, K, dst);
    if (int rc = last_launch()) return rc;
    score = dst;
  } else if (scores_out && scores_out != scores_in) {
    if (int rc = hip_status(hipMemcpyAsync(scores_out, scores_in, K * sizeof(float),
                                           hipMemcpyDeviceToDevice, s)))
      return rc;
  }
  if (int rc = topk_launch(score, K, k, idx_out, s)) return rc;
  if (resid_out && k > 0 && rows > 0) {
    const int64_t n = rows * k;
    dim3 grid((unsigned)((n + 255) / 256));
    if (bf16)
      hipLaunchKernelGGL(k_resid_gather<true>, grid, dim3(256), 0, s, x, rows, K, ldx, codes,
                         scales, tensor_scale, idx_out, (int)k, resid_out);
    else
      hipLaunchKernelGGL(k_resid_gather<false>, grid, dim3(256), 0, s, x, rows, K, ldx, codes,
                         scales, tensor_scale, idx_out, (int)k, resid_out);
    return last_launch();
  }
  return NVQ_OK;
}

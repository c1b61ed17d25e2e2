// Rollout-guided rounding for gfx950: the compact guidance record and the
// trainer-side requantization of drifted master weights from it.
//
// Method: TRACE post ("TRACE : un entraînement conscient de la quantification
// guidé par le rollout ..."), "L'idée centrale de TRACE" -- the rollout's
// quantization result guides the trainer's rounding, and the cache keeps only
// the mantissa and the scale factors -- and "Fonctionnement, côté ingénierie"
// -- each value rounds to the grid point above or below, the one discrete
// choice the two sides must share.
//
// Record (one bit per element, element c in bit c % 8 of byte c / 8 of its
// row), next to the rollout's block scales and tensor scale:
//   NVQ_GUIDE_MANTISSA  the mantissa bit of the rollout's E2M1 code;
//   NVQ_GUIDE_DIRECTION 1 when the rollout's magnitude G s_b s_t lies strictly
//                       above |x| (the value was rounded up).
// Requantization of a master value w under the cached scales: with lo the
// largest index whose scaled grid point G[lo] s_b s_t is <= |w| and hi the
// smallest whose point is >= |w| (7 when |w| lies beyond the grid),
//   mantissa:  of a = min(lo, 6) and a + 1 (adjacent points, whose mantissa
//              bits differ), the one carrying the cached bit;
//   direction: bit 1 -> hi, bit 0 -> lo.
// Sign from signbit(w); a zero scale product gives magnitude 0.  Both modes
// have a fast path on fp32 bit patterns for tensor scales in [2^-100, 2^100]
// and a general seven-threshold path for the rest.
//
// Exactness: G s_b is exact in fp32 (<= 6 significant bits), and its product
// with s_t (<= 30 bits) is exact in fp64.  Each block turns its seven grid
// products into fp32 thresholds rounded up (RU) and down (RD); for an fp32
// |w|,  p <= |w|  <=>  RU(p) <= |w|  and  p < |w|  <=>  RD(p) < |w|,
// so every decision is a plain fp32 compare.  A thread handles one
// 16-element block: its loads and stores are contiguous across the wave.

#include <hip/hip_runtime.h>

#include "nvq.h"
#include "nvq_device.h"
#include "nvq_internal.h"

namespace nvq {
namespace {

constexpr int kGuideThreads = 256;

// fp32 value of a positive fp64 number rounded up / down (exact inputs only
// matter here: p is an exact product).  Overflow goes to +inf (up) or FLT_MAX
// (down); values below the smallest subnormal go to 2^-149 (up) or 0 (down).
__device__ __forceinline__ float f32_round_up(double p) {
  float f = (float)p;
  if ((double)f < p) f = __uint_as_float(__float_as_uint(f) + 1u);
  return f;
}
__device__ __forceinline__ float f32_round_down(double p) {
  float f = (float)p;
  if ((double)f > p) f = __uint_as_float(__float_as_uint(f) - 1u);
  return f;
}

// The 16 values of block `blk` as fp32 (bf16 widening is exact).
template <bool kBF16>
__device__ __forceinline__ void load_block(const void* __restrict__ x, int64_t blk, float v[16]) {
  if (kBF16) {
    const uint4* p = static_cast<const uint4*>(x) + 2 * blk;
    const uint4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = bf16_lo(w[j]);
      v[2 * j + 1] = bf16_hi(w[j]);
    }
  } else {
    const float4* p = static_cast<const float4*>(x) + 4 * blk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 q = p[j];
      v[4 * j] = q.x;
      v[4 * j + 1] = q.y;
      v[4 * j + 2] = q.z;
      v[4 * j + 3] = q.w;
    }
  }
}

// -------------------------------------------------------------- record ----
// bits of block blk (16 elements -> one uint16).  Mantissa mode reads only
// the codes; direction mode also reads x and the block's scale.
template <int kMode, bool kBF16>
__global__ __launch_bounds__(kGuideThreads) void k_guidance_record(
    const void* __restrict__ x, const uint2* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tensor_scale, int64_t blocks_per_item,
    uint16_t* __restrict__ bits) {
  const int64_t in_item = (int64_t)blockIdx.x * kGuideThreads + threadIdx.x;
  if (in_item >= blocks_per_item) return;
  const int64_t blk = (int64_t)blockIdx.y * blocks_per_item + in_item;
  const uint2 cw = codes[blk];
  uint32_t out = 0;
  if (kMode == NVQ_GUIDE_MANTISSA) {
    // mantissa bit of nibble j sits at bit 4j of the 64-bit code word
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      out |= ((cw.x >> (4 * j)) & 1u) << j;
      out |= ((cw.y >> (4 * j)) & 1u) << (8 + j);
    }
  } else {
    float v[16];
    load_block<kBF16>(x, blk, v);
    const float s_b = e4m3_to_f32(scales[blk]);
    const double s_t = (double)tensor_scale[blockIdx.y];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t nib = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 7u;
      // G s_b exact in fp32; times s_t exact in fp64; |x| exact in fp64
      const double p = (double)(e2m1_mag(nib) * s_b) * s_t;
      out |= (uint32_t)(p > (double)fabsf(v[j])) << j;
    }
  }
  bits[blk] = (uint16_t)out;
}

// Mantissa bits of one 32-bit word of codes (8 nibbles) -> 8 bits.
__device__ __forceinline__ uint32_t mantissa8(uint32_t w) {
  uint32_t x = w & 0x11111111u;          // bit 0 of every nibble
  x = (x | (x >> 3)) & 0x03030303u;      // two per byte, at bits 0-1
  x = (x | (x >> 6)) & 0x000F000Fu;      // four per half word, at bits 0-3
  return (x | (x >> 12)) & 0xFFu;
}

// Mantissa record, four blocks per thread (32 bytes of codes -> 8 bytes of
// bits); needs only the codes, so items do not matter.  The last thread
// takes the 1-3 blocks past the last full group.
__global__ __launch_bounds__(kGuideThreads) void k_mantissa_record4(
    const uint4* __restrict__ codes, int64_t n_blocks, uint2* __restrict__ bits4,
    uint16_t* __restrict__ bits) {
  const int64_t t = (int64_t)blockIdx.x * kGuideThreads + threadIdx.x;
  const int64_t b0 = 4 * t;
  if (b0 >= n_blocks) return;
  if (b0 + 4 <= n_blocks) {
    const uint4 a = codes[2 * t], b = codes[2 * t + 1];
    uint2 o;
    o.x = mantissa8(a.x) | (mantissa8(a.y) << 8) | (mantissa8(a.z) << 16) | (mantissa8(a.w) << 24);
    o.y = mantissa8(b.x) | (mantissa8(b.y) << 8) | (mantissa8(b.z) << 16) | (mantissa8(b.w) << 24);
    bits4[t] = o;
  } else {
    const uint2* c2 = reinterpret_cast<const uint2*>(codes);
    for (int64_t blk = b0; blk < n_blocks; ++blk) {
      const uint2 cw = c2[blk];
      bits[blk] = (uint16_t)(mantissa8(cw.x) | (mantissa8(cw.y) << 8));
    }
  }
}

// ------------------------------------------------------- requantization ----
template <int kMode, bool kBF16>
__global__ __launch_bounds__(kGuideThreads) void k_guided_quantize(
    const void* __restrict__ w, const uint16_t* __restrict__ bits,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale,
    int64_t blocks_per_item, uint2* __restrict__ codes, uint32_t* __restrict__ status) {
  const int64_t in_item = (int64_t)blockIdx.x * kGuideThreads + threadIdx.x;
  if (in_item >= blocks_per_item) return;
  const int64_t blk = (int64_t)blockIdx.y * blocks_per_item + in_item;
  float v[16];
  load_block<kBF16>(w, blk, v);
  const uint32_t rec = bits[blk];
  const float s_b = e4m3_to_f32(scales[blk]);
  const double s_t = (double)tensor_scale[blockIdx.y];
  const bool zero_scale = (double)s_b * s_t == 0.0;

  // one non-finite test per block: the largest |w| bit pattern
  uint32_t amax_bits = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) amax_bits = max(amax_bits, __float_as_uint(v[j]) & 0x7FFFFFFFu);
  const bool nonfinite = amax_bits >= 0x7F800000u;
  uint32_t out[2] = {0u, 0u};
  if (kMode == NVQ_GUIDE_MANTISSA && s_t >= 0x1p-100 && s_t <= 0x1p100 && !zero_scale) {
    // Fast path.  Here every threshold is a normal fp32 number, RU(2^k p) =
    // 2^k RU(p), and bits(2^k T) = bits(T) + k 2^23; the bit patterns of
    // non-negative floats order as the values.  With R1 = RU(s_b s_t) and
    // R15 = RU(1.5 s_b s_t) the grid thresholds are
    //   points 1, 3, 5 (even result, bit 0): R1 / 2, R15, 2 R15
    //   points 2, 4, 6 (odd result, bit 1):  R1, 2 R1, 4 R1
    // and the chosen index is 2 * (number of those thresholds <= |w|) + bit:
    // of the two neighbours of |w|, the one with the recorded mantissa bit.
    // The last two thresholds of each set are one binade apart, so their
    // count is clamp((bits(|w|) - bits(first) + 2^23) >> 23, 0, 2).
    const int32_t r1 = (int32_t)__float_as_uint(f32_round_up((double)s_b * s_t));
    const int32_t r15 = (int32_t)__float_as_uint(f32_round_up((double)(1.5f * s_b) * s_t));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = __float_as_uint(v[j]);
      const int32_t a = (int32_t)(u & 0x7FFFFFFFu);
      const uint32_t b = (rec >> j) & 1u;
      const int32_t t0 = b ? r1 : r1 - (1 << 23);
      const int32_t base = b ? r1 : r15 - (1 << 23);
      const int32_t pair = min(max((a - base) >> 23, 0), 2);
      const uint32_t idx = 2u * (uint32_t)(pair + (a >= t0)) + b;
      out[j >> 3] |= (idx | ((u >> 28) & 8u)) << (4 * (j & 7));
    }
  } else if (kMode == NVQ_GUIDE_DIRECTION && s_t >= 0x1p-100 && s_t <= 0x1p100 && !zero_scale) {
    // Fast path, direction mode.  The grid products p_i (i = 1..7) are
    // {1/2, 1, 2, 4} P and {1, 2, 4} 1.5 P with P = s_b s_t: two chains of
    // binade steps plus the first point.  lo counts p_i <= |w| against the
    // round-up thresholds (R1 = RU(P), R15 = RU(1.5 P)); hi counts p_i < |w|
    // (point 0 included) against the smallest floats above the round-down
    // values (N1 = next(RD(P)), N15 = next(RD(1.5 P))), capped at 7.  In
    // normal range both kinds of threshold scale exactly by 2 down a chain.
    const double P = (double)s_b * s_t, P15 = (double)(1.5f * s_b) * s_t;
    const int32_t r1 = (int32_t)__float_as_uint(f32_round_up(P));
    const int32_t r15 = (int32_t)__float_as_uint(f32_round_up(P15));
    const int32_t n1 = (int32_t)__float_as_uint(f32_round_down(P)) + 1;
    const int32_t n15 = (int32_t)__float_as_uint(f32_round_down(P15)) + 1;
    auto chain3 = [](int32_t a, int32_t base) {  // thresholds base, 2 base, 4 base
      return min(max((a - base + (1 << 23)) >> 23, 0), 3);
    };
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = __float_as_uint(v[j]);
      const int32_t a = (int32_t)(u & 0x7FFFFFFFu);
      const uint32_t b = (rec >> j) & 1u;
      // one count with the thresholds of the recorded side (no divergence)
      const int32_t base1 = b ? n1 : r1, base15 = b ? n15 : r15;
      const int32_t cnt = (int32_t)(b & (uint32_t)(a > 0)) + (a >= base1 - (1 << 23)) +
                          chain3(a, base1) + chain3(a, base15);
      const uint32_t idx = (uint32_t)min(cnt, 7);
      out[j >> 3] |= (idx | ((u >> 28) & 8u)) << (4 * (j & 7));
    }
  } else {
  // thresholds of grid points 1..7: RU for "point <= |w|", RD for "point < |w|"
  float up[7], dn[7];
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const double p = (double)(e2m1_mag((uint32_t)i + 1u) * s_b) * s_t;
    up[i] = f32_round_up(p);
    if (kMode == NVQ_GUIDE_DIRECTION) dn[i] = f32_round_down(p);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t u = __float_as_uint(v[j]);
    const float aw = fabsf(v[j]);
    uint32_t lo = 0;
#pragma unroll
    for (int i = 0; i < 7; ++i) lo += aw >= up[i];
    const uint32_t b = (rec >> j) & 1u;
    uint32_t idx;
    if (kMode == NVQ_GUIDE_MANTISSA) {
      const uint32_t a = lo < 6u ? lo : 6u;
      idx = a + ((a ^ b) & 1u);
    } else {
      uint32_t below = aw > 0.0f;  // grid point 0 lies strictly below |w|
#pragma unroll
      for (int i = 0; i < 7; ++i) below += aw > dn[i];
      const uint32_t hi = below < 7u ? below : 7u;
      idx = b ? hi : lo;
    }
    if (zero_scale) idx = 0;
    const uint32_t nib = idx | ((u >> 28) & 8u);
    out[j >> 3] |= nib << (4 * (j & 7));
  }
  }
  codes[blk] = make_uint2(out[0], out[1]);
  if (status) {
    const uint64_t any = __ballot(nonfinite);
    if (any != 0ull && (threadIdx.x & (kWave - 1)) == (unsigned)__builtin_ctzll(any))
      atomicOr(status, NVQ_STATUS_NONFINITE);
  }
}

}  // namespace
}  // namespace nvq

using namespace nvq;

extern "C" int nvfp4_guidance_record(const void* x, int x_dtype, const uint8_t* codes,
                                     const uint8_t* scales, const float* tensor_scale,
                                     int64_t batch, int64_t rows, int64_t K, int mode,
                                     uint8_t* bits, void* stream) {
  if (mode != NVQ_GUIDE_MANTISSA && mode != NVQ_GUIDE_DIRECTION) return NVQ_EINVAL;
  if (mode == NVQ_GUIDE_DIRECTION && x_dtype != NVQ_F32 && x_dtype != NVQ_BF16) return NVQ_EINVAL;
  if (batch <= 0 || rows < 0 || K <= 0 || (K & 15)) return NVQ_ESHAPE;
  const int64_t per_item = rows * (K / 16);
  const int64_t n_blocks = batch * per_item;
  if (n_blocks == 0) return NVQ_OK;
  if (!codes || !bits) return NVQ_EINVAL;
  if (mode == NVQ_GUIDE_DIRECTION && (!x || !scales || !tensor_scale)) return NVQ_EINVAL;
  if (((uintptr_t)codes & 7u) || ((uintptr_t)bits & 1u)) return NVQ_EALIGN;
  if (mode == NVQ_GUIDE_DIRECTION && !aligned16(x)) return NVQ_EALIGN;
  if ((per_item + kGuideThreads - 1) / kGuideThreads > 0x7FFFFFFF || batch > 65535)
    return NVQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((per_item + kGuideThreads - 1) / kGuideThreads), (unsigned)batch);
  const uint2* cw = reinterpret_cast<const uint2*>(codes);
  uint16_t* b16 = reinterpret_cast<uint16_t*>(bits);
  if (mode == NVQ_GUIDE_MANTISSA && ((uintptr_t)codes & 15u) == 0 && ((uintptr_t)bits & 7u) == 0) {
    const int64_t nthr = (n_blocks + 3) / 4;
    if ((nthr + kGuideThreads - 1) / kGuideThreads > 0x7FFFFFFF) return NVQ_ESHAPE;
    hipLaunchKernelGGL(k_mantissa_record4,
                       dim3((unsigned)((nthr + kGuideThreads - 1) / kGuideThreads)),
                       dim3(kGuideThreads), 0, s, reinterpret_cast<const uint4*>(codes), n_blocks,
                       reinterpret_cast<uint2*>(bits), b16);
  } else if (mode == NVQ_GUIDE_MANTISSA)
    hipLaunchKernelGGL((k_guidance_record<NVQ_GUIDE_MANTISSA, true>), grid, dim3(kGuideThreads),
                       0, s, x, cw, scales, tensor_scale, per_item, b16);
  else if (x_dtype == NVQ_BF16)
    hipLaunchKernelGGL((k_guidance_record<NVQ_GUIDE_DIRECTION, true>), grid,
                       dim3(kGuideThreads), 0, s, x, cw, scales, tensor_scale, per_item, b16);
  else
    hipLaunchKernelGGL((k_guidance_record<NVQ_GUIDE_DIRECTION, false>), grid,
                       dim3(kGuideThreads), 0, s, x, cw, scales, tensor_scale, per_item, b16);
  return last_launch();
}

extern "C" int nvfp4_guided_quantize(const void* w, int w_dtype, int64_t batch, int64_t rows,
                                     int64_t K, const uint8_t* bits, const uint8_t* scales,
                                     const float* tensor_scale, int mode, uint8_t* codes,
                                     void* ws, size_t ws_bytes, void* stream) {
  if (mode != NVQ_GUIDE_MANTISSA && mode != NVQ_GUIDE_DIRECTION) return NVQ_EINVAL;
  if (w_dtype != NVQ_F32 && w_dtype != NVQ_BF16) return NVQ_EINVAL;
  if (batch <= 0 || rows < 0 || K <= 0 || (K & 15)) return NVQ_ESHAPE;
  const int64_t per_item = rows * (K / 16);
  const int64_t n_blocks = batch * per_item;
  if (n_blocks > 0 && (!w || !bits || !scales || !codes)) return NVQ_EINVAL;
  if ((per_item + kGuideThreads - 1) / kGuideThreads > 0x7FFFFFFF || batch > 65535)
    return NVQ_ESHAPE;
  if (!tensor_scale) return NVQ_EINVAL;
  if (ws && !aligned256(ws)) return NVQ_EALIGN;
  if (ws && ws_bytes < kAlign) return NVQ_EWORKSPACE;
  if (n_blocks > 0 && (!aligned16(w) || ((uintptr_t)codes & 7u) || ((uintptr_t)bits & 1u)))
    return NVQ_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* status = ws ? WsCarve(ws).status() : nullptr;
  if (status) {
    const int rc = clear_status(status, s);
    if (rc != NVQ_OK) return rc;
  }
  if (n_blocks == 0) return NVQ_OK;
  const dim3 grid((unsigned)((per_item + kGuideThreads - 1) / kGuideThreads), (unsigned)batch);
  const uint16_t* b16 = reinterpret_cast<const uint16_t*>(bits);
  uint2* cw = reinterpret_cast<uint2*>(codes);
  const bool bf16 = w_dtype == NVQ_BF16;
  if (mode == NVQ_GUIDE_MANTISSA) {
    if (bf16)
      hipLaunchKernelGGL((k_guided_quantize<NVQ_GUIDE_MANTISSA, true>), grid,
                         dim3(kGuideThreads), 0, s, w, b16, scales, tensor_scale, per_item,
                         cw, status);
    else
      hipLaunchKernelGGL((k_guided_quantize<NVQ_GUIDE_MANTISSA, false>), grid,
                         dim3(kGuideThreads), 0, s, w, b16, scales, tensor_scale, per_item,
                         cw, status);
  } else {
    if (bf16)
      hipLaunchKernelGGL((k_guided_quantize<NVQ_GUIDE_DIRECTION, true>), grid,
                         dim3(kGuideThreads), 0, s, w, b16, scales, tensor_scale, per_item,
                         cw, status);
    else
      hipLaunchKernelGGL((k_guided_quantize<NVQ_GUIDE_DIRECTION, false>), grid,
                         dim3(kGuideThreads), 0, s, w, b16, scales, tensor_scale, per_item,
                         cw, status);
  }
  return last_launch();
}

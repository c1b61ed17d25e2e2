// Device-side helpers shared by the HIP kernels of libnvq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvq {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16 --
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------- wave reductions --
// Max over the 64 lanes of a wave with DPP row operations and four
// readlanes; every lane receives the result.  No LDS traffic.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) | (uint32_t)__builtin_amdgcn_readlane((int)v, 16) |
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) | (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// ------------------------------------------------------------ E4M3 / E2M1 --
// E4M3 ("FN") code -> fp32 value; code in 0..0x7E.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xF, m = code & 7;
  if (e == 0) return (float)m * 0.001953125f;  // m/8 * 2^-6
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude of index 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_mag(uint32_t mi) {
  return mi < 2 ? 0.5f * (float)mi : (float)(1u << ((mi >> 1) - 1)) * ((mi & 1) ? 1.5f : 1.0f);
}

// Nearest E4M3 code to q >= 0, ties to even, saturating at 0x7E (448).  Exact
// for any fp32 q; callers pass an approximation of the real quotient only when
// it is provably not near an E4M3 decision midpoint.
__device__ __forceinline__ uint32_t e4m3_rne_f32(float q) {
  if (!(q < 448.0f)) return 0x7E;
  if (q < 0.015625f) return (uint32_t)__builtin_rintf(q * 512.0f);  // subnormal grid 2^-9
  const uint32_t b = __float_as_uint(q);
  return (b - (120u << 23) + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
}

// Nearest E4M3 code to the real quotient amax_b / six_st, exact: the fp64
// quotient is correctly rounded, and an E4M3 midpoint (5 significant bits)
// differs from a quotient of a 24-bit by a 26-bit number by more than 2^-31
// relative unless equal, so rounding the fp64 quotient decides as the real one.
__device__ __forceinline__ uint32_t e4m3_code_exact(float amax_b, double six_st) {
  const double q = (double)amax_b / six_st;
  if (!(q < 448.0)) return 0x7E;
  if (q < 0.015625) return (uint32_t)__builtin_rint(q * 512.0);
  const uint64_t b = (uint64_t)__double_as_longlong(q);
  return (uint32_t)((b - (1016ull << 52) + ((1ull << 48) - 1ull) + ((b >> 49) & 1ull)) >> 49);
}

// Exact E2M1 magnitude index of |x| against the scale S = s_b * s_t (exact in
// fp64): count the decision midpoints below |x|; a value exactly on a
// midpoint goes to the even index.
__device__ __forceinline__ uint32_t e2m1_index_exact(float ax, double S) {
  const double a = (double)ax;
  uint32_t i = 0;
  i += a > 0.25 * S;
  i += a >= 0.75 * S;
  i += a > 1.25 * S;
  i += a >= 1.75 * S;
  i += a > 2.5 * S;
  i += a >= 3.5 * S;
  i += a > 5.0 * S;
  return i;
}

}  // namespace nvq

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

// ------------------------------------------------------- tile stores --
// Stores a wave's 128 x 64 outputs bf16(acc * scale) as 16-byte row pieces
// through LDS.  acc[i][j][v] is row 32 i + 8 (v / 4) + 4 h + v % 4, column
// 32 j + l32 of the wave tile, so a store straight from the accumulators
// writes 2 bytes per lane (128 store instructions).  Here adjacent lanes
// first trade one value (a DPP swap), so each lane holds a bf16 pair of one
// row and writes it to the wave's LDS region (128 rows x 128 bytes, 16-byte
// chunk q of row r at slot q ^ 4 (r & 1), which keeps the two rows of a write
// instruction in different banks); then each lane reads 16-byte row pieces
// and stores them (16 store instructions).  Rows at or past nrows are not
// stored.  region: this wave's 16 KB of LDS, free of other use.
template <class Acc>
__device__ __forceinline__ void store_tile_bf16_lds(const Acc (&acc)[4][2], float scale,
                                                    uint8_t* region, uint16_t* out, int64_t ld,
                                                    int nrows) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const bool odd = (l32 & 1) != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        // rows r, r + 1 of column c: the even lane keeps row r and sends row
        // r + 1 to its odd neighbour, which keeps row r + 1
        const float a = acc[i][j][v] * scale, b = acc[i][j][v + 1] * scale;
        const float send = odd ? a : b;
        const float recv = __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(send), 0xB1, 0xF, 0xF, false));
        const float lo = odd ? recv : a, hi = odd ? b : recv;
        const int row = 32 * i + 8 * (v >> 2) + 4 * h + (v & 3) + (odd ? 1 : 0);
        const int col = 32 * j + l32 - (odd ? 1 : 0);  // even column of the pair
        const int slot = (col >> 3) ^ ((row & 1) << 2);
        *reinterpret_cast<uint32_t*>(region + row * 128 + slot * 16 + (col & 7) * 2) =
            f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
      }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int row = (lane >> 3) + 8 * m, q = lane & 7;
    if (row >= nrows) continue;
    const uint4 v4 = *reinterpret_cast<const uint4*>(region + row * 128 + ((q ^ ((row & 1) << 2)) << 4));
    *reinterpret_cast<uint4*>(out + (int64_t)row * ld + 8 * q) = v4;
  }
}

}  // namespace nvq

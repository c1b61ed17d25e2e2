// Asymmetric W4A16 QAT grouped GEMMs (gfx950): forward, input gradient and
// weight gradient of a fake-quantized MoE projection.
//
// Method: QUADS explainer §2.2-A -- the trainer forward sees the NVFP4
// weights the rollout uses (fake quantization of W only) while activations
// stay BF16; TRACE post, "L'idée centrale de TRACE" -- the trainer takes its
// rounding from the rollout's recorded quantization, so the weight operand
// here is the cached NVFP4 record (codes, E4M3 scales, tensor scale) itself,
// dequantized exactly inside the kernel.  The straight-through gradient is
// the identity (a reading: the pages name no clipping):
//   FWD    y[p, n]  = sum_c x[a_row(p), c] W^_e[n, c]
//   DGRAD  dx[p, c] = sum_n dy[p, n] W^_e[n, c]
//   WGRAD  dW_e[n, c] (+)= sum_{p in e} dy[p, n] x[a_row(p), c]
// with W^ = G * s_b * s_t.  bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32
// accumulation; s_t is applied to the fp32 accumulators.
//
// Both operands are staged as bf16 tiles in LDS in a fragment-ready layout
// [k/8][row][8 values], so every mode shares one MFMA loop.  Four loaders fill
// the tiles: bf16 rows with the contraction index contiguous (x, dy), bf16
// sources whose contraction index is the row (dy and x in WGRAD: transposed
// through register byte permutes), FP4 weight rows (FWD: each element
// dequantized once per workgroup, G * s_b exact in bf16), and FP4 weight
// rows transposed (DGRAD: the contraction runs over the weight's rows).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "nvq.h"
#include "nvq_device.h"
#include "nvq_internal.h"
#include "nvq_scan.h"

namespace nvq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int QBM = 128;   // output rows per workgroup
constexpr int QBN = 256;   // output columns per workgroup (2 waves x 128)
constexpr int QBK = 32;    // contraction per LDS stage (48 KB of LDS: two workgroups per CU)
constexpr int QT = 128;    // threads
constexpr int QQ = QBK / 8;

enum { LD_ROWS = 0, LD_ROWS_T = 1, LD_FP4 = 2, LD_FP4_T = 3 };

struct QatParams {
  int mode;
  int accumulate;
  int64_t rows, K, N, E;
  const int32_t* a_row;
  const int32_t* off;
  const uint16_t* x;
  const uint16_t* dy;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_st;
  uint16_t* out_bf16;
  float* out_f32;
  float* dw;
  const int32_t* tiles;
  const int32_t* ntiles;
  int max_tiles;
  int n_tiles_n;
  int n_tiles_m;  // WGRAD: row tiles over N
};

__global__ __launch_bounds__(1024) void k_qat_tile_table(const int32_t* __restrict__ off, int E,
                                                        int32_t* __restrict__ tiles,
                                                        int32_t* __restrict__ ntiles, int max_tiles,
                                                        int bm) {
  __shared__ int32_t s_wave[16];
  __shared__ int32_t s_incl[1024];
  build_tile_table(off, E, bm, tiles, ntiles, max_tiles, s_wave, s_incl);
}

// Two FP4 codes (a byte) times the block scale -> packed bf16 pair, exact
// (G * s_b has <= 6 significant bits).
template <int kSel>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float s_b) {
  auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, kSel);
  const uint32_t lo = __float_as_uint(g[0] * s_b), hi = __float_as_uint(g[1] * s_b);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // [hi.bf16 : lo.bf16]
}

// 8 codes (one dword) -> 4 packed bf16 pairs.
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t w, float s_b) {
  return make_uint4(fp4x2_to_bf16x2<0>(w, s_b), fp4x2_to_bf16x2<1>(w, s_b),
                    fp4x2_to_bf16x2<2>(w, s_b), fp4x2_to_bf16x2<3>(w, s_b));
}

// Low/high 16-bit halves of two dwords packed together.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // [b.lo : a.lo]
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // [b.hi : a.hi]
}

// One operand tile: kRows tile rows x QBK contraction values, staged as
// [QQ][kRows][8] bf16 in LDS.  Each loader splits into load() (global ->
// registers, issued before the MFMA work of the current stage) and store()
// (registers -> LDS, with any dequantization or transposition).
struct TileSrc {
  const uint16_t* bf;      // bf16 source
  int64_t ld;              // its row stride (elements)
  const int32_t* row_map;  // source row of a logical row (nullptr: identity)
  int64_t row_base;        // first logical row (LD_ROWS) / first contraction row (LD_ROWS_T)
  int64_t row_end;         // end of valid logical rows / contraction rows
  int64_t col_base;        // first source column of the tile (LD_ROWS_T, LD_FP4*)
  int64_t col_end;
  const uint8_t* codes;    // FP4 weight of the expert [wN, wK/2]
  const uint8_t* scales;   // [wN, wK/16]
  int64_t wK, wN;
};

__device__ __forceinline__ int64_t src_row(const TileSrc& s, int64_t i) {
  return s.row_map ? (int64_t)s.row_map[i] : i;
}

template <int kKind, int kRows>
struct Loader;

// bf16 rows, contraction contiguous: 8 threads per row, 16 B each.
template <int kRows>
struct Loader<LD_ROWS, kRows> {
  static constexpr int kN = kRows * QQ / QT;
  uint4 v[kN];
  __device__ __forceinline__ void load(const TileSrc& s, int ks, int t) {
    const int64_t k0 = (int64_t)ks * QBK;
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int c = t + QT * u, r = c / QQ, q = c % QQ;
      const int64_t gr = s.row_base + r;
      v[u] = make_uint4(0, 0, 0, 0);
      if (gr < s.row_end) v[u] = *reinterpret_cast<const uint4*>(s.bf + src_row(s, gr) * s.ld + k0 + q * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int t) const {
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int c = t + QT * u, r = c / QQ, q = c % QQ;
      *reinterpret_cast<uint4*>(dst + ((size_t)q * kRows + r) * 8) = v[u];
    }
  }
};

// bf16 source whose rows are the contraction: task = 4 source rows x 8
// columns, transposed with byte permutes into 4-value runs.
template <int kRows>
struct Loader<LD_ROWS_T, kRows> {
  static constexpr int kN = (QBK / 4) * (kRows / 8) / QT;
  uint4 v[kN][4];
  __device__ __forceinline__ void load(const TileSrc& s, int ks, int t) {
    const int64_t k0 = (int64_t)ks * QBK;
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int task = t + QT * u, cg = task % (kRows / 8), pg = task / (kRows / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t pr = s.row_base + k0 + 4 * pg + i;
        v[u][i] = make_uint4(0, 0, 0, 0);
        if (pr < s.row_end && s.col_base + 8 * cg < s.col_end)
          v[u][i] = *reinterpret_cast<const uint4*>(s.bf + src_row(s, pr) * s.ld + s.col_base + 8 * cg);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int t) const {
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int task = t + QT * u, cg = task % (kRows / 8), pg = task / (kRows / 8);
      const int q = (4 * pg) / 8, off4 = (4 * pg) % 8;
      const uint32_t w0[4] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w};
      const uint32_t w1[4] = {v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
      const uint32_t w2[4] = {v[u][2].x, v[u][2].y, v[u][2].z, v[u][2].w};
      const uint32_t w3[4] = {v[u][3].x, v[u][3].y, v[u][3].z, v[u][3].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 lo = make_uint2(pack_lo(w0[j], w1[j]), pack_lo(w2[j], w3[j]));
        const uint2 hi = make_uint2(pack_hi(w0[j], w1[j]), pack_hi(w2[j], w3[j]));
        *reinterpret_cast<uint2*>(dst + ((size_t)q * kRows + 8 * cg + 2 * j) * 8 + off4) = lo;
        *reinterpret_cast<uint2*>(dst + ((size_t)q * kRows + 8 * cg + 2 * j + 1) * 8 + off4) = hi;
      }
    }
  }
};

// FP4 weight rows (tile row = weight row), contraction along the weight's K:
// task = one row x 32 values (16 B codes, 2 block scales); dequantized once.
template <int kRows>
struct Loader<LD_FP4, kRows> {
  static constexpr int kN = kRows * (QBK / 32) / QT;
  uint4 cw[kN];
  uint32_t sc[kN];
  __device__ __forceinline__ void load(const TileSrc& s, int ks, int t) {
    const int64_t k0 = (int64_t)ks * QBK;
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int task = t + QT * u, r = task / (QBK / 32), hq = task % (QBK / 32);
      const int64_t n = s.col_base + r;
      const int64_t kk = k0 + 32 * hq;
      cw[u] = make_uint4(0, 0, 0, 0);
      sc[u] = 0;
      if (n < s.wN) {
        cw[u] = *reinterpret_cast<const uint4*>(s.codes + n * (s.wK >> 1) + (kk >> 1));
        sc[u] = *reinterpret_cast<const uint16_t*>(s.scales + n * (s.wK >> 4) + (kk >> 4));
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int t) const {
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int task = t + QT * u, r = task / (QBK / 32), hq = task % (QBK / 32);
      const float sb0 = e4m3_to_f32(sc[u] & 0xFFu), sb1 = e4m3_to_f32(sc[u] >> 8);
      const int q0 = 4 * hq;
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 0) * kRows + r) * 8) = fp4x8_to_bf16(cw[u].x, sb0);
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 1) * kRows + r) * 8) = fp4x8_to_bf16(cw[u].y, sb0);
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 2) * kRows + r) * 8) = fp4x8_to_bf16(cw[u].z, sb1);
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 3) * kRows + r) * 8) = fp4x8_to_bf16(cw[u].w, sb1);
    }
  }
};

// FP4 weight with the contraction over the weight's rows (tile row = weight
// column): task = 4 weight rows x 16 columns (one block per row), dequantized
// and transposed.
template <int kRows>
struct Loader<LD_FP4_T, kRows> {
  static constexpr int kN = (QBK / 4) * (kRows / 16) / QT;
  uint2 cw[kN][4];
  uint32_t sc[kN][4];
  __device__ __forceinline__ void load(const TileSrc& s, int ks, int t) {
    const int64_t k0 = (int64_t)ks * QBK;
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int task = t + QT * u, cb = task % (kRows / 16), ng = task / (kRows / 16);
      const int64_t c0 = s.col_base + 16 * cb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = k0 + 4 * ng + i;
        cw[u][i] = make_uint2(0, 0);
        sc[u][i] = 0;
        if (n < s.wN && c0 < s.col_end) {
          cw[u][i] = *reinterpret_cast<const uint2*>(s.codes + n * (s.wK >> 1) + (c0 >> 1));
          sc[u][i] = s.scales[n * (s.wK >> 4) + (c0 >> 4)];
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int t) const {
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int task = t + QT * u, cb = task % (kRows / 16), ng = task / (kRows / 16);
      uint32_t rowv[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sb = e4m3_to_f32(sc[u][i]);
        const uint4 a = fp4x8_to_bf16(cw[u][i].x, sb), b = fp4x8_to_bf16(cw[u][i].y, sb);
        rowv[i][0] = a.x; rowv[i][1] = a.y; rowv[i][2] = a.z; rowv[i][3] = a.w;
        rowv[i][4] = b.x; rowv[i][5] = b.y; rowv[i][6] = b.z; rowv[i][7] = b.w;
      }
      const int q = (4 * ng) / 8, off4 = (4 * ng) % 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint2 lo = make_uint2(pack_lo(rowv[0][j], rowv[1][j]), pack_lo(rowv[2][j], rowv[3][j]));
        const uint2 hi = make_uint2(pack_hi(rowv[0][j], rowv[1][j]), pack_hi(rowv[2][j], rowv[3][j]));
        *reinterpret_cast<uint2*>(dst + ((size_t)q * kRows + 16 * cb + 2 * j) * 8 + off4) = lo;
        *reinterpret_cast<uint2*>(dst + ((size_t)q * kRows + 16 * cb + 2 * j + 1) * 8 + off4) = hi;
      }
    }
  }
};

// acc += A[QBM x QBK] * B[QBK x (this wave's 128 columns)] from one LDS stage.
__device__ __forceinline__ void mfma_stage(const uint16_t* sa, const uint16_t* sb, int wave, int l32,
                                           int h, floatx16_t (&acc)[4][4]) {
#pragma unroll
  for (int s = 0; s < QBK / 16; ++s) {
    const int q = 2 * s + h;
    bf16x8_t af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(&sa[((size_t)q * QBM + 32 * i + l32) * 8]);
      __builtin_memcpy(&af[i], &v, 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(&sb[((size_t)q * QBN + 128 * wave + 32 * j + l32) * 8]);
      __builtin_memcpy(&bf[j], &v, 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
}

// Output tile QBM x QBN = (rows of A) x (rows of B); contraction nk stages,
// software-pipelined: stage ks + 1 is read from global memory before the
// MFMA work of stage ks and written to the other LDS buffer after it (the
// last stage re-reads itself into the idle buffer, which nobody reads).
template <int kMode, int kKA, int kKB>
__global__ __launch_bounds__(QT) void k_qat_gemm(QatParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA0[QQ * QBM * 8];
  __shared__ __attribute__((aligned(16))) uint16_t sA1[QQ * QBM * 8];
  __shared__ __attribute__((aligned(16))) uint16_t sB0[QQ * QBN * 8];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[QQ * QBN * 8];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, l32 = lane & 31, h = lane >> 5;

  TileSrc A, B;
  A.row_map = nullptr;
  B.row_map = nullptr;
  int e;
  int64_t out_r0, out_r_end, out_c0, out_c_end, nk;
  const int G = gridDim.x, per = G >> 3;
  const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);

  if (kMode == NVQ_QAT_WGRAD) {
    const int per_e = p.n_tiles_m * p.n_tiles_n;
    e = logical / per_e;
    if (e >= p.E) return;
    const int rem = logical % per_e;
    const int mt = rem % p.n_tiles_m, nt = rem / p.n_tiles_m;
    const int64_t pe0 = p.off[e], pe1 = p.off[e + 1];
    out_r0 = (int64_t)mt * QBM; out_r_end = p.N;
    out_c0 = (int64_t)nt * QBN; out_c_end = p.K;
    nk = (pe1 - pe0 + QBK - 1) / QBK;
    A.bf = p.dy; A.ld = p.N; A.row_base = pe0; A.row_end = pe1; A.col_base = out_r0; A.col_end = p.N;
    B.bf = p.x; B.ld = p.K; B.row_base = pe0; B.row_end = pe1; B.col_base = out_c0; B.col_end = p.K;
    B.row_map = p.a_row;
  } else {
    const int mt = logical % p.max_tiles, nt = logical / p.max_tiles;
    if (nt >= p.n_tiles_n || mt >= *p.ntiles) return;
    e = p.tiles[2 * mt];
    out_r0 = p.tiles[2 * mt + 1];
    out_r_end = p.off[e + 1];
    out_c0 = (int64_t)nt * QBN;
    B.codes = p.w_codes + (int64_t)e * p.N * (p.K >> 1);
    B.scales = p.w_scales + (int64_t)e * p.N * (p.K >> 4);
    B.wK = p.K; B.wN = p.N; B.col_base = out_c0;
    A.row_base = out_r0; A.row_end = out_r_end;
    if (kMode == NVQ_QAT_FWD) {
      out_c_end = p.N;
      nk = p.K / QBK;
      A.bf = p.x; A.ld = p.K; A.row_map = p.a_row;
      B.col_end = p.N;
    } else {
      out_c_end = p.K;
      nk = p.N / QBK;
      A.bf = p.dy; A.ld = p.N;
      B.col_end = p.K;
    }
  }

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  Loader<kKA, QBM> la;
  Loader<kKB, QBN> lb;
  if (nk > 0) {
    la.load(A, 0, t);
    lb.load(B, 0, t);
    la.store(sA0, t);
    lb.store(sB0, t);
  }
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const bool odd = ks & 1;
    // Next stage (clamped to the last one, so no load sits under a branch).
    const int nx = ks + 1 < nk ? ks + 1 : ks;
    la.load(A, nx, t);
    lb.load(B, nx, t);
    mfma_stage(odd ? sA1 : sA0, odd ? sB1 : sB0, wave, l32, h, acc);
    la.store(odd ? sA0 : sA1, t);
    lb.store(odd ? sB0 : sB1, t);
    __syncthreads();
  }

  const float scale = (kMode == NVQ_QAT_WGRAD) ? 1.0f : p.w_st[e];
  // acc[i][j][v]: row 32i + 8(v/4) + 4h + v%4, column 32j + l32 of the wave tile.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t r = out_r0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      if (r >= out_r_end) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = out_c0 + 128 * wave + 32 * j + l32;
        if (c >= out_c_end) continue;
        const float y = acc[i][j][v] * scale;
        if (kMode == NVQ_QAT_WGRAD) {
          float* d = p.dw + ((int64_t)e * p.N + r) * p.K + c;
          *d = p.accumulate ? *d + y : y;
        } else {
          const int64_t ld = out_c_end;
          if (p.out_f32) p.out_f32[r * ld + c] = y;
          if (p.out_bf16) p.out_bf16[r * ld + c] = (uint16_t)f32_to_bf16_rne(y);
        }
      }
    }
}

// ------------------------------------------------------ forward, 2 WG/CU --
// The forward in the grouped-GEMM layout: workgroup = 4 waves = 128 sorted
// rows x 256 output columns; wave = 128 x 64 with accumulators in VGPRs (two
// workgroups share a CU).  K advances 128 elements per step.
//  * A (x rows gathered through a_row, bf16, shared by the four waves) goes
//    straight from global memory into a double-buffered LDS tile with
//    global_load_lds_dwordx4 (no registers): LDS slot = base + 16 lane, so
//    lane l of load instruction I carries row 4 I + l / 16, slot l % 16.  The
//    slot of 16-byte chunk c of row r is c ^ (r & 15) (256-byte rows, XOR
//    swizzle: the fragment reads of 16 consecutive rows hit distinct banks).
//  * B (this wave's 64 weight rows, FP4) is loaded in fragment order two steps
//    ahead and dequantized exactly to bf16 in registers: G * s_b has <= 6
//    significant bits.
// Within a step lane half h owns elements [64h, 64h + 64); sub-step d takes
// 64h + 8d .. +8 for A and B alike.
constexpr int FBM = 128, FBN = 256, FWN = 64, FSE = 128;

struct QStage {
  uint4 b[2][2];
  uint32_t bs[2];
};

__device__ __forceinline__ bf16x8_t fp4x8_bf16(uint32_t w, float s_b) {
  const uint4 v = fp4x8_to_bf16(w, s_b);
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// E4M3 code (0..0x7E) -> fp32 without branches: (8 [e > 0] + m) 2^(max(e, 1) - 10),
// always a normal fp32 (smallest nonzero 2^-9).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
  const uint32_t mant = m | (e != 0u ? 8u : 0u);
  return __builtin_amdgcn_ldexpf((float)mant, (int)(e != 0u ? e : 1u) - 10);
}

// XCD-aware order over the real tiles: groups of kGm row tiles x all column
// tiles (the row tiles of a group read the same weight tile at about the same
// time), each of the 8 XCDs (blockIdx.x % 8) takes a contiguous range of the
// order.  False for surplus workgroups.  Measured: 8 for the forward's
// 128-row tiles; 1 for the input gradient, whose 1.5 MB dy row block (read by
// every column tile) is eight times its weight slice, so consecutive
// workgroups should share the rows, not the weight.
constexpr int kFwdGroupM = 8, kDgradGroupM = 1;
template <int kGm>
__device__ __forceinline__ bool pick_tile(const QatParams& p, int& mt, int& nt) {
  const int n_mt = min(*p.ntiles, p.max_tiles);
  const int n_groups = (n_mt + kGm - 1) / kGm;
  const int total = n_groups * kGm * p.n_tiles_n;
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  if (slot >= per) return false;
  const int logical = (blockIdx.x & 7) * per + slot;
  if (logical >= total) return false;
  const int group_span = kGm * p.n_tiles_n;
  const int grp = logical / group_span, rem = logical - grp * group_span;
  mt = kGm * grp + (rem % kGm);
  nt = rem / kGm;
  return mt < n_mt;
}
// Grid of the order above: every group slot, rounded up to the 8 XCDs.
inline int64_t pick_grid(int64_t max_tiles, int gm, int n_tiles_n) {
  return ((max_tiles + gm - 1) / gm * gm * n_tiles_n + 7) / 8 * 8;
}

__global__ __launch_bounds__(256, 2) void k_qat_fwd2(QatParams p) {
  __shared__ __attribute__((aligned(16))) uint4 lds[2][FBM * 16];
  int mt, nt;
  if (!pick_tile<kFwdGroupM>(p, mt, nt)) return;
  const int e = p.tiles[2 * mt];
  const int64_t row0 = p.tiles[2 * mt + 1];
  const int64_t row_end = p.off[e + 1];
  const int64_t K = p.K, N = p.N;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, l32 = lane & 31, h = lane >> 5;

  // A: this lane's 8 load instructions (I = 4 q + wave) per step; rows past
  // the expert's end read a clamped valid row (never stored).
  const uint16_t* a_src[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int I = 4 * q + wave;
    const int r = 4 * I + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const int64_t pr = min<int64_t>(row0 + r, row_end - 1);
    const int64_t tok = p.a_row ? (int64_t)p.a_row[pr] : pr;
    a_src[q] = p.x + tok * K + 8 * c;
  }
  auto a_load = [&](int buf, int step) {
    const int64_t k0 = (int64_t)min(step, (int)(K / FSE) - 1) * FSE;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int I = 4 * q + wave;
      __builtin_amdgcn_global_load_lds((const void*)(a_src[q] + k0),
                                       (__attribute__((address_space(3))) void*)&lds[buf][64 * I], 16, 0, 0);
    }
  };
  // B: fragment j = weight row 64 wave + 32 j + l32 of this column tile
  const uint8_t* b_src[2];
  const uint8_t* b_ssrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = min<int64_t>((int64_t)nt * FBN + FWN * wave + 32 * j + l32, N - 1);
    b_src[j] = p.w_codes + ((int64_t)e * N + n) * (K >> 1) + 32 * h;
    b_ssrc[j] = p.w_scales + ((int64_t)e * N + n) * (K >> 4) + 4 * h;
  }
  const int nst = (int)(K / FSE);
  auto b_load = [&](QStage& S, int step) {
    const int64_t sc = min(step, nst - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S.b[j][0] = *reinterpret_cast<const uint4*>(b_src[j] + sc * 64);
      S.b[j][1] = *reinterpret_cast<const uint4*>(b_src[j] + sc * 64 + 16);
      S.bs[j] = *reinterpret_cast<const uint32_t*>(b_ssrc[j] + sc * 8);
    }
  };

  floatx16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto mfma_step = [&](const QStage& S, int buf) {
    float sb[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) sb[j][b] = e4m3_value((S.bs[j] >> (8 * b)) & 0xFFu);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      bf16x8_t af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + l32;
        const int c = 8 * h + d;
        af[i] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][16 * r + (c ^ (r & 15))]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4& v = S.b[j][d >> 2];
        const uint32_t w = (d & 3) == 0 ? v.x : (d & 3) == 1 ? v.y : (d & 3) == 2 ? v.z : v.w;
        bf[j] = fp4x8_bf16(w, sb[j][d >> 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Pipeline over step pairs: each step first issues the A tile (into the
  // other LDS buffer) and the B stage of the next step, runs its MFMAs, then
  // waits for every load of this thread and meets the other waves at a
  // barrier, so a load has one step of MFMA work to land.  The scheduling
  // barriers keep the loads ahead of the MFMAs (the compiler otherwise sinks
  // them to the wait).  A load past the last step re-reads the last one
  // into the idle buffer; it has landed by the loop's final wait.  An odd
  // step count ends with one more step outside the loop.
  QStage X0, X1;
  a_load(0, 0);
  b_load(X0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  const int npair = nst >> 1;
  for (int it = 0; it < npair; ++it) {
    const int st = 2 * it;
    a_load(1, st + 1);
    b_load(X1, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(X0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    a_load(0, st + 2);
    b_load(X0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(X1, 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if (nst & 1) mfma_step(X0, 0);

  const float stw = p.w_st[e];
  // A wave whose rows and columns are all inside the output stores without
  // per-element checks (wave-uniform branches on which outputs are wanted).
  auto emit = [&](auto&& store, bool check) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t pr = row0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (check && pr >= row_end) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t n = (int64_t)nt * FBN + FWN * wave + 32 * j + l32;
          if (check && n >= N) continue;
          store(pr * N + n, acc[i][j][v] * stw);
        }
      }
  };
  auto st_f32 = [&](int64_t o, float y) { p.out_f32[o] = y; };
  auto st_bf16 = [&](int64_t o, float y) { p.out_bf16[o] = (uint16_t)f32_to_bf16_rne(y); };
  auto st_both = [&](int64_t o, float y) { st_f32(o, y); st_bf16(o, y); };
  const bool cols_full = (int64_t)nt * FBN + FWN * (wave + 1) <= N;
  const bool full = row0 + FBM <= row_end && cols_full;
  // bf16 rows as 16-byte pieces through LDS when the wave's 64 columns are
  // inside the output (the LDS tiles are free after the barrier)
  const bool bf16_lds = p.out_bf16 && (N % 8 == 0) && ((uintptr_t)p.out_bf16 % 16 == 0) && cols_full;
  if (p.out_f32 && p.out_bf16 && !bf16_lds)
    full ? emit(st_both, false) : emit(st_both, true);
  else if (p.out_f32)
    full ? emit(st_f32, false) : emit(st_f32, true);
  else if (!bf16_lds)
    full ? emit(st_bf16, false) : emit(st_bf16, true);
  if (p.out_bf16) {
    __syncthreads();  // every wave is past its last LDS read
    if (bf16_lds)
      store_tile_bf16_lds(acc, stw, reinterpret_cast<uint8_t*>(&lds[0][0]) + 16384 * wave,
                          p.out_bf16 + row0 * N + (int64_t)nt * FBN + FWN * wave, N,
                          (int)min<int64_t>(FBM, row_end - row0));
  }
}

// ------------------------------------------------ input gradient, 2 WG/CU --
// dx[p, c] = sum_n dy[p, n] W^_e[n, c]: the contraction runs over the
// weight's rows, so an MFMA lane (8 consecutive contraction values of one
// column) needs a column strip of W.  Workgroup = 4 waves = 256 sorted rows x
// 128 output columns; wave = 64 rows x 128 columns as 4 x 8 tiles of the
// 16x16x32 bf16 MFMA (accumulators in VGPRs).
//  * The weight tile of a step (128 rows n x 128 columns c, FP4) is
//    dequantized once per workgroup, exactly, and written transposed as bf16
//    into a double-buffered LDS tile [c][n] (256-byte rows, 16-byte chunk n/8
//    stored at slot (n/8) ^ (c & 15)).  Thread t takes rows 4 (t & 31) .. +3
//    and columns 16 (t >> 5) .. +15: one block scale per row.
//  * dy rows are private to a wave, so lanes keep their fragments in
//    registers.  In the 16x16x32 layout lane (l16, g) holds row l16 and
//    contraction values 32 d + 8 g .. +8 of sub-step d, so the four lanes of a
//    row read 64 contiguous bytes (one load instruction touches 16 rows, not
//    32 rows x 2 as the 32x32 layout would).  Fragments roll two sub-steps
//    ahead.
#define NVQ_LDS __attribute__((address_space(3)))
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Two LDS transpose reads (ds_read_b64_tr_b16) -> one 8-element bf16 MFMA
// operand: in each group of 16 lanes, lane i receives element i % 4 of the
// 8-byte reads of lanes i / 4 + 4 m, m = 0..3 (measured), so a source lane
// that points at 4 consecutive columns of contraction row k0 + s / 4 hands
// lane i the values of column 4 (s % 4) + i % 4 at rows k0 .. k0 + 3.
__device__ __forceinline__ bf16x8_t tr_pair(const NVQ_LDS char* base, uint32_t off0, uint32_t off1) {
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((NVQ_LDS v4i16_t*)(base + off0));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((NVQ_LDS v4i16_t*)(base + off1));
  typedef short v8i16_t __attribute__((ext_vector_type(8)));
  const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

constexpr int DBM = 256, DBN = 128, DSE = 128;
// Output widths that are multiples of DBN take the wide weight path: thread t
// loads contraction row t / 2 of the step, 64 columns (two 16-byte code loads
// and one scale dword, 3 load instructions against 8), and writes it
// dequantized in its natural [n][c] layout (rows of DBN bf16 at a 288-byte
// pitch, so the 4 rows x 32 bytes of one transpose read fall in distinct
// banks); the MFMA B operands come out through tr_pair.  The input gradient
// is bound by the vector memory address path, so load instructions count.
constexpr int DW_PITCH = 2 * DBN + 32, DW_BUF = DSE * DW_PITCH;

typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <bool kWide>
struct WStage {
  uint2 c[4];
  uint32_t s[4];
};
template <>
struct WStage<true> {
  uint4 c[2];
  uint32_t s;
};

template <int kSel>
__device__ __forceinline__ void fp4_pair_rows(const uint32_t (&w)[4], const float (&sb)[4],
                                              float (&f)[4][2]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[r], 1.0f, kSel);
    f[r][0] = g[0] * sb[r];
    f[r][1] = g[1] * sb[r];
  }
}

template <bool kWide>
__global__ __launch_bounds__(256, 2) void k_qat_dgrad2(QatParams p) {
  __shared__ __attribute__((aligned(16))) char wt[kWide ? 2 * DW_BUF : 2 * DBN * 256];
  int mt, nt;
  if (!pick_tile<kDgradGroupM>(p, mt, nt)) return;
  const int e = p.tiles[2 * mt];
  const int64_t row0 = p.tiles[2 * mt + 1];
  const int64_t row_end = p.off[e + 1];
  const int64_t Nc = p.N, Ko = p.K;  // contraction length, output columns
  const int64_t c0 = (int64_t)nt * DBN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, l16 = lane & 15, g = lane >> 4;
  const int nst = (int)(Nc / DSE);

  // Addresses are a uniform base plus a 32-bit per-lane byte offset (the
  // tile's 256 rows of dy; one expert's weight, < 2 GiB by the host check).
  const char* const dy_t = reinterpret_cast<const char*>(p.dy + row0 * Nc);
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t pr = min<int64_t>(row0 + 64 * wave + 16 * i + l16, row_end - 1);
    a_off[i] = (uint32_t)(((pr - row0) * Nc + 8 * g) * 2);
  }
  auto a_frag = [&](int i, int64_t u) {  // element u of the step sequence
    return *reinterpret_cast<const bf16x8_t*>(dy_t + 2 * u + a_off[i]);
  };
  // weight rows and column block of this thread (columns past K read the last
  // valid block; their outputs are never stored)
  const int q = t & 31, cb = t >> 5;
  const int64_t cw = min<int64_t>(c0 + 16 * cb, Ko - 16);
  const uint8_t* const w_e = p.w_codes + (int64_t)e * Nc * (Ko >> 1);
  const uint8_t* const s_e = p.w_scales + (int64_t)e * Nc * (Ko >> 4);
  const uint32_t w_off = (uint32_t)(4 * q * (Ko >> 1) + (cw >> 1));
  const uint32_t s_off = (uint32_t)(4 * q * (Ko >> 4) + (cw >> 4));
  // wide path: contraction row wr of the step, columns c0 + 64 wh .. +63
  const int wr = t >> 1, wh = t & 1;
  const uint32_t ww_off = (uint32_t)(wr * (Ko >> 1) + ((c0 + 64 * wh) >> 1));
  const uint32_t ws_off = (uint32_t)(wr * (Ko >> 4) + ((c0 + 64 * wh) >> 4));
  auto w_load = [&](WStage<kWide>& W, int step) {
    if constexpr (kWide) {
      const uint8_t* const cr = w_e + (int64_t)step * DSE * (Ko >> 1) + ww_off;
      W.c[0] = *reinterpret_cast<const uint4*>(cr);
      W.c[1] = *reinterpret_cast<const uint4*>(cr + 16);
      W.s = *reinterpret_cast<const uint32_t*>(s_e + (int64_t)step * DSE * (Ko >> 4) + ws_off);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = (int64_t)step * DSE + r;
        W.c[r] = *reinterpret_cast<const uint2*>(w_e + row * (Ko >> 1) + w_off);
        W.s[r] = *(s_e + row * (Ko >> 4) + s_off);
      }
    }
  };
  char* const wt_base = &wt[0];
  auto w_store = [&](const WStage<kWide>& W, int buf) {
    if constexpr (kWide) {
      char* const dst = wt_base + buf * DW_BUF + wr * DW_PITCH + 128 * wh;
      const uint32_t w[8] = {W.c[0].x, W.c[0].y, W.c[0].z, W.c[0].w, W.c[1].x, W.c[1].y, W.c[1].z, W.c[1].w};
#pragma unroll
      for (int u = 0; u < 8; ++u)
        *reinterpret_cast<uint4*>(dst + 16 * u) = fp4x8_to_bf16(w[u], e4m3_value((W.s >> (8 * (u >> 1))) & 0xFFu));
    } else {
      float sb[4];
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sb[r] = e4m3_value(W.s[r]);
        lo[r] = W.c[r].x;
        hi[r] = W.c[r].y;
      }
      char* const dst = wt_base + buf * (DBN * 256) + 8 * (q & 1);
      auto put = [&](const float (&f)[4][2], int u) {  // columns u, u + 1 of the block
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int c = 16 * cb + u + k;
          uint2 v;
          v.x = __builtin_amdgcn_perm(__float_as_uint(f[1][k]), __float_as_uint(f[0][k]), 0x07060302u);
          v.y = __builtin_amdgcn_perm(__float_as_uint(f[3][k]), __float_as_uint(f[2][k]), 0x07060302u);
          *reinterpret_cast<uint2*>(dst + c * 256 + 16 * ((q >> 1) ^ (c & 15))) = v;
        }
      };
      float f[4][2];
      fp4_pair_rows<0>(lo, sb, f); put(f, 0);
      fp4_pair_rows<1>(lo, sb, f); put(f, 2);
      fp4_pair_rows<2>(lo, sb, f); put(f, 4);
      fp4_pair_rows<3>(lo, sb, f); put(f, 6);
      fp4_pair_rows<0>(hi, sb, f); put(f, 8);
      fp4_pair_rows<1>(hi, sb, f); put(f, 10);
      fp4_pair_rows<2>(hi, sb, f); put(f, 12);
      fp4_pair_rows<3>(hi, sb, f); put(f, 14);
    }
  };

  floatx4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  // dy fragments of sub-step u = 4 st + d live in slot u % 2
  bf16x8_t a[2][4];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int i = 0; i < 4; ++i) a[s2][i] = a_frag(i, 32 * s2);

  // One step: MFMAs over LDS buffer st % 2; with next the weight tile of step
  // st + 1 is loaded first and dequantized into the other buffer after the
  // MFMAs.  Scheduling barriers between sub-steps keep every load where it is
  // issued (the scheduler otherwise sinks them next to their use).
  // wide path transpose-read offsets: source lane s = l16 points at columns
  // 4 (s & 3) .. +3 of contraction row 32 d + 8 g + 4 hf + s / 4
  const NVQ_LDS char* const wt_lds = (const NVQ_LDS char*)wt;
  uint32_t tr_off[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) tr_off[hf] = (uint32_t)((8 * g + 4 * hf + (l16 >> 2)) * DW_PITCH + 8 * (l16 & 3));
  auto step = [&](int st, WStage<kWide>& W, bool next) {
    const int buf = st & 1;
    const char* const src = wt_base + buf * (DBN * 256);
    if (next) w_load(W, st + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        bf16x8_t bfr[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if constexpr (kWide) {
            const uint32_t o = buf * DW_BUF + 32 * d * DW_PITCH + 32 * (4 * jh + jj);
            bfr[jj] = tr_pair(wt_lds, tr_off[0] + o, tr_off[1] + o);
          } else {
            const int c = 16 * (4 * jh + jj) + l16;
            bfr[jj] = *reinterpret_cast<const bf16x8_t*>(src + c * 256 + 16 * ((4 * d + g) ^ (c & 15)));
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[i][4 * jh + jj] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[d & 1][i], bfr[jj], acc[i][4 * jh + jj], 0, 0, 0);
      }
      if (d < 2 || next) {
        const int64_t u = (int64_t)st * DSE + 32 * ((d + 2) & 3) + (d < 2 ? 0 : DSE);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[d & 1][i] = a_frag(i, u);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (next) w_store(W, buf ^ 1);
  };

  WStage<kWide> W;
  w_load(W, 0);
  w_store(W, 0);
  __syncthreads();
  // A wave whose 64 rows all lie past the expert's end (in its last tile)
  // loads no dy and runs no MFMAs: it only stages its share of the weight
  // tiles, with the same barriers, and stores nothing.
  if (__builtin_amdgcn_readfirstlane(64 * wave) >= row_end - row0) {
    for (int st = 0; st + 1 < nst; ++st) {
      w_load(W, st + 1);
      w_store(W, (st & 1) ^ 1);
      __syncthreads();
    }
    return;
  }
  for (int st = 0; st + 1 < nst; ++st) {
    step(st, W, true);
    __syncthreads();
  }
  step(nst - 1, W, false);

  const float stw = p.w_st[e];
  // A wave whose rows and columns are all inside the output stores without
  // per-element checks (wave-uniform branches on which outputs are wanted).
  auto emit = [&](auto&& store, bool check) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t pr = row0 + 64 * wave + 16 * i + 4 * g + v;
        if (check && pr >= row_end) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t c = c0 + 16 * j + l16;
          if (check && c >= Ko) continue;
          store(pr * Ko + c, acc[i][j][v] * stw);
        }
      }
  };
  auto st_f32 = [&](int64_t o, float y) { p.out_f32[o] = y; };
  auto st_bf16 = [&](int64_t o, float y) { p.out_bf16[o] = (uint16_t)f32_to_bf16_rne(y); };
  auto st_both = [&](int64_t o, float y) { st_f32(o, y); st_bf16(o, y); };
  const bool full = row0 + 64 * (wave + 1) <= row_end && c0 + DBN <= Ko;
  if (p.out_f32 && p.out_bf16)
    full ? emit(st_both, false) : emit(st_both, true);
  else if (p.out_f32)
    full ? emit(st_f32, false) : emit(st_f32, true);
  else
    full ? emit(st_bf16, false) : emit(st_bf16, true);
}

// ------------------------------------------------- weight gradient, 2 WG/CU --
// dW[e, n, c] (+)= sum_{p of e} dy[p, n] x[a_row[p], c]: the contraction runs
// over the rows of both operands.  Workgroup = 8 waves = 256 n x 256 c of one
// expert (one workgroup per CU); wave (wn, wc) = 64 n x 128 c as 2 x 4 tiles
// of the 32x32x16 bf16 MFMA.  The square tile halves the re-reads of x
// against 128 x 256 (every n tile reads the whole x panel of its columns),
// and the operand re-reads are what bounds this kernel.  A step takes 48
// contraction rows: dy[48][256] and the gathered x[48][256] (24 KB each)
// stream from global memory into LDS with direct loads, in their natural row
// layout, three stages deep (145 KB of LDS; 48-row steps measured 1.5-4%
// faster than 32-row ones: fewer barriers per row and a longer lead).  The MFMA operands (8
// consecutive contraction rows of one column) come out of those row-major
// tiles through the LDS transpose read ds_read_b64_tr_b16: in each group of
// 16 lanes, lane i receives element i % 4 of the 8-byte reads of lanes
// i / 4 + 4 m, m = 0..3, so source lane s points at 4 consecutive columns of
// contraction row k0 + s / 4.  16-byte chunk c of tile row r is stored at
// slot c ^ (2 (r & 7)): the 4 rows x 32 bytes of one 16-lane read fall in
// distinct banks.  Rows past the expert's end are zeroed in LDS by the wave
// that loaded them.
// The direct loads are issued from inline assembly and ordered by explicit
// waits: a compiler-visible one makes the compiler drain every load before
// any LDS read, which would empty the pipeline.  The x row indices of a step
// (a_row) are themselves staged into LDS by a direct load one step earlier
// than the step's tiles, ahead of them in issue order, so the only vector
// memory operations in the loop are these direct loads.
constexpr int GBN = 256, GBC = 256, GPS = 48;
constexpr int G_LD = GPS / 16;  // load instructions per tile per thread (2 rows each, 8 waves)
constexpr int G_DY = GPS * GBN * 2, G_X = GPS * GBC * 2, G_TOK = 256;
constexpr int G_STAGE = G_DY + G_X + G_TOK;

// Global -> LDS direct loads; lane l lands at LDS byte lds_addr + size * l.
// lds_addr must be wave-uniform; it is read from the first lane so that it
// is in a scalar register even where the compiler cannot prove uniformity.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}

__global__ __launch_bounds__(512, 1) void k_qat_wgrad2(QatParams p) {
  __shared__ __attribute__((aligned(16))) char lds[3 * G_STAGE];
  const int n_tn = p.n_tiles_m, n_tc = p.n_tiles_n;
  const int per_e = n_tn * n_tc;
  const int total = (int)p.E * per_e;
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  if (slot >= per) return;
  const int logical = (blockIdx.x & 7) * per + slot;  // XCD blockIdx % 8 takes a contiguous range
  if (logical >= total) return;
  const int e = logical / per_e, rem = logical - e * per_e;
  // Order of an expert's tiles: the 32 workgroups an XCD runs at once should
  // touch few dy (n) and x (c) panels.  n-tile-major order covers 32 / n_tc
  // n-tiles x all c-tiles; with 8 or more c-tiles, bands of 4 n-tiles walked
  // c-tile-major cover 4 x 8 instead (12 panels rather than 18 at n_tc = 16).
  int tn, tc;
  if (n_tc >= 8) {
    constexpr int kBand = 4;
    const int band = rem / (kBand * n_tc), ib = rem - band * (kBand * n_tc);
    const int brows = min(kBand, n_tn - band * kBand);
    tc = ib / brows;
    tn = band * kBand + (ib - tc * brows);
  } else {
    tn = rem / n_tc;
    tc = rem - tn * n_tc;
  }
  const int64_t N = p.N, K = p.K, rows = p.rows;
  const int64_t n0 = (int64_t)tn * GBN, c0 = (int64_t)tc * GBC;
  const int64_t p_beg = p.off[e], p_end = p.off[e + 1];
  const int nsteps = (int)((p_end - p_beg + GPS - 1) / GPS);
  const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, h = lane >> 5, s16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave & 3, wc = wave >> 2;

  floatx16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  if (nsteps > 0) {
    NVQ_LDS char* const lb = (NVQ_LDS char*)lds;
    const uint32_t lb_addr = (uint32_t)(uintptr_t)lb;
    // loads of this lane: instructions I = G_LD wave + k of each tile (rows
    // 2 I + lane / 32, 32 slots of 16 bytes a row), so wave w loads rows
    // 2 G_LD w .. 2 G_LD w + 2 G_LD - 1 of both tiles; every row is clamped
    // into [0, rows) and every column chunk into the matrix (rows past the
    // expert's end are zeroed later, columns past N or K are never stored)
    int dy_r[G_LD], x_r[G_LD];
    int64_t dy_col[G_LD], x_col[G_LD];
#pragma unroll
    for (int k = 0; k < G_LD; ++k) {
      const int I = G_LD * wave + k, r = 2 * I + (lane >> 5);
      dy_r[k] = r;
      x_r[k] = r;
      dy_col[k] = min<int64_t>(n0 + 8 * ((lane & 31) ^ (2 * (r & 7))), N - 8);
      x_col[k] = min<int64_t>(c0 + 8 * ((lane & 31) ^ (2 * (r & 7))), K - 8);
    }
    auto prow = [&](int st, int r) { return min<int64_t>(p_beg + (int64_t)st * GPS + r, rows - 1); };
    auto stage_of = [](int st) { return st % 3; };
    // x row indices of step st -> the tok area of its stage (wave 0; lanes
    // past the step's rows repeat its last row)
    auto issue_tok = [&](int st) {
      if (wave == 0 && p.a_row)
        dma4(p.a_row + prow(st, min(lane, GPS - 1)), lb_addr + stage_of(st) * G_STAGE + G_DY + G_X);
    };
    auto issue = [&](int st) {
      const int sg = stage_of(st);
      const uint32_t base = lb_addr + sg * G_STAGE;
      const NVQ_LDS int32_t* tok_lds = (const NVQ_LDS int32_t*)(lb + sg * G_STAGE + G_DY + G_X);
      int64_t tok[G_LD];  // read before the first load is issued (the loads order all memory)
      if (p.a_row) {
#pragma unroll
        for (int k = 0; k < G_LD; ++k) tok[k] = tok_lds[x_r[k]];
      } else {
#pragma unroll
        for (int k = 0; k < G_LD; ++k) tok[k] = prow(st, x_r[k]);
      }
#pragma unroll
      for (int k = 0; k < G_LD; ++k)
        dma16(p.dy + prow(st, dy_r[k]) * N + dy_col[k], base + 1024 * (G_LD * wave + k));
#pragma unroll
      for (int k = 0; k < G_LD; ++k)
        dma16(p.x + tok[k] * K + x_col[k], base + G_DY + 1024 * (G_LD * wave + k));
    };
    // rows of step st past the expert's end -> zero (this lane's own slots)
    auto zero_tail = [&](int st) {
      const int64_t nvalid = p_end - p_beg - (int64_t)st * GPS;
      if (nvalid >= GPS) return;
      NVQ_LDS char* const base = lb + stage_of(st) * G_STAGE;
#pragma unroll
      for (int k = 0; k < G_LD; ++k)
        if (dy_r[k] >= nvalid) {
          *(NVQ_LDS u32x4_t*)(base + 1024 * (G_LD * wave + k) + 16 * lane) = u32x4_t{0, 0, 0, 0};
          *(NVQ_LDS u32x4_t*)(base + G_DY + 1024 * (G_LD * wave + k) + 16 * lane) = u32x4_t{0, 0, 0, 0};
        }
    };

    // transpose-read offsets: operand row (n or c) base of this lane's group,
    // 4 columns per source lane; contraction row k0 + s16 / 4
    uint32_t a_off[2][2], b_off[4][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 8 * h + 4 * hf + (s16 >> 2);  // contraction row within a 16-row sub-step
      const int f = 2 * (r & 7);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int col = 64 * wn + 32 * i + 16 * (l32 >> 4) + 4 * (s16 & 3);
        a_off[i][hf] = (uint32_t)(r * (GBN * 2) + 16 * ((col >> 3) ^ f) + 8 * ((col >> 2) & 1));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 128 * wc + 32 * j + 16 * (l32 >> 4) + 4 * (s16 & 3);
        b_off[j][hf] = (uint32_t)(G_DY + r * (GBC * 2) + 16 * ((col >> 3) ^ f) + 8 * ((col >> 2) & 1));
      }
    }
    auto compute = [&](int st) {
      const NVQ_LDS char* const base = lb + stage_of(st) * G_STAGE;
#pragma unroll
      for (int sub = 0; sub < GPS / 16; ++sub) {
        bf16x8_t af[2], bfr[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = tr_pair(base + sub * 16 * (GBN * 2), a_off[i][0], a_off[i][1]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = tr_pair(base + sub * 16 * (GBC * 2), b_off[j][0], b_off[j][1]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    };
    auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    // prologue: row indices of steps 0..2, then the tiles of steps 0 and 1
    issue_tok(0);
    if (nsteps > 1) issue_tok(1);
    if (nsteps > 2) issue_tok(2);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();
    issue(0);
    if (nsteps > 1) {
      issue(1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G_LD) : "memory");  // step 0 landed
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      zero_tail(0);
    }
    barrier();

    // step st: [row indices of st + 3][tiles of st + 2] are issued, step st
    // is computed, then the tiles of st + 1 (and every older load) must have
    // landed while the 2 G_LD tile loads of st + 2 may still be in flight
    for (int st = 0; st < nsteps; ++st) {
      const bool ahead = st + 2 < nsteps;
      if (ahead) {
        if (st + 3 < nsteps) issue_tok(st + 3);
        issue(st + 2);
      }
      compute(st);
      if (st + 1 < nsteps) {
        if (ahead)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G_LD) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (st + 1 == nsteps - 1) zero_tail(st + 1);
        barrier();
      }
    }
  } else if (p.accumulate) {
    return;  // no rows: dW unchanged
  }

  // Tiles wholly inside dW (every tile when N and K are multiples of 256) take
  // branch-free stores; with accumulate the 16 old values of a 32 x 32 tile
  // are loaded together, then added and stored.  Partial tiles check each
  // element.
  auto idx = [](int v) { return (int64_t)(8 * (v >> 2) + (v & 3)); };
  const bool full = n0 + GBN <= N && c0 + GBC <= K;
  if (full && !p.accumulate) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* const d = p.dw + ((int64_t)e * N + n0 + 64 * wn + 32 * i + 4 * h) * K + c0 + 128 * wc + 32 * j + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) __builtin_nontemporal_store(acc[i][j][v], &d[idx(v) * K]);
      }
  } else if (full) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* const d = p.dw + ((int64_t)e * N + n0 + 64 * wn + 32 * i + 4 * h) * K + c0 + 128 * wc + 32 * j + l32;
        float old[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) old[v] = d[idx(v) * K];
#pragma unroll
        for (int v = 0; v < 16; ++v) d[idx(v) * K] = old[v] + acc[i][j][v];
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + 128 * wc + 32 * j + l32;
        const int64_t nb = n0 + 64 * wn + 32 * i + 4 * h;
        float* const d = p.dw + ((int64_t)e * N + nb) * K + c;
        auto ok = [&](int v) { return c < K && nb + idx(v) < N; };
        float old[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) old[v] = (p.accumulate && ok(v)) ? d[idx(v) * K] : 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (ok(v)) d[idx(v) * K] = old[v] + acc[i][j][v];
      }
  }
}

struct QatLayout {
  int max_tiles;
  int32_t* tiles;
  int32_t* ntiles;
  size_t bytes;
};

QatLayout qat_layout(void* ws, int64_t rows, int64_t E) {
  QatLayout L;
  L.max_tiles = (int)((rows + QBM - 1) / QBM + E);
  WsCarve c(ws);
  L.tiles = c.take<int32_t>((size_t)L.max_tiles * 2);
  L.ntiles = c.take<int32_t>(1);
  L.bytes = c.off;
  return L;
}

}  // namespace
}  // namespace nvq

using namespace nvq;

extern "C" size_t qat_gemm_workspace_bytes(int64_t rows, int64_t E) {
  if (rows < 0 || E < 1) return kAlign;
  return qat_layout(nullptr, rows, E).bytes;
}

extern "C" int qat_fakequant_gemm_w4a16(const nvq_qat_gemm_args* a, void* stream) {
  if (!a || a->struct_size < sizeof(nvq_qat_gemm_args)) return NVQ_EINVAL;
  if (a->mode != NVQ_QAT_FWD && a->mode != NVQ_QAT_DGRAD && a->mode != NVQ_QAT_WGRAD)
    return NVQ_EINVAL;
  if (!a->expert_offsets || !a->ws) return NVQ_EINVAL;
  if (a->rows < 0 || a->E < 1 || a->E > 1024 || a->N <= 0 || a->K <= 0) return NVQ_ESHAPE;
  if (a->K % QBK != 0 || a->N % QBK != 0) return NVQ_ESHAPE;  // 32-element contraction stages
  const bool wgrad = a->mode == NVQ_QAT_WGRAD;
  // the row buffers (x, dy, outputs of FWD and DGRAD) may be NULL when there are no rows
  if (a->rows != 0 && a->mode != NVQ_QAT_DGRAD && !a->x) return NVQ_EINVAL;
  if (a->rows != 0 && a->mode != NVQ_QAT_FWD && !a->dy) return NVQ_EINVAL;
  if (!wgrad && (!a->w_codes || !a->w_scales || !a->w_tensor_scale)) return NVQ_EINVAL;
  if (!wgrad && a->rows != 0 && !a->out_bf16 && !a->out_f32) return NVQ_EINVAL;
  if (wgrad && !a->dw) return NVQ_EINVAL;
  if ((a->x && !aligned16(a->x)) || (a->dy && !aligned16(a->dy)) ||
      (a->w_codes && ((uintptr_t)a->w_codes & 15u)))
    return NVQ_EALIGN;
  if (!aligned256(a->ws)) return NVQ_EALIGN;
  QatLayout L = qat_layout(a->ws, a->rows, a->E);
  if (a->ws_bytes < L.bytes) return NVQ_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  QatParams p;
  p.mode = a->mode; p.accumulate = a->accumulate;
  p.rows = a->rows; p.K = a->K; p.N = a->N; p.E = a->E;
  p.a_row = a->a_row; p.off = a->expert_offsets;
  p.x = a->x; p.dy = a->dy;
  p.w_codes = a->w_codes; p.w_scales = a->w_scales; p.w_st = a->w_tensor_scale;
  p.out_bf16 = a->out_bf16; p.out_f32 = a->out_f32; p.dw = a->dw;
  p.tiles = L.tiles; p.ntiles = L.ntiles; p.max_tiles = L.max_tiles;
  if (wgrad) {
    // transpose-read kernel, 256 x 256 tiles (no rows: every expert has no
    // contraction steps, so it only writes zeros, or leaves dW with accumulate)
    p.n_tiles_m = (int)((a->N + GBN - 1) / GBN);
    p.n_tiles_n = (int)((a->K + GBC - 1) / GBC);
    const int64_t G2 = (a->E * p.n_tiles_m * p.n_tiles_n + 7) / 8 * 8;
    hipLaunchKernelGGL(k_qat_wgrad2, dim3((unsigned)G2), dim3(512), 0, s, p);
    return last_launch();
  }
  if (a->rows == 0) return NVQ_OK;
  // input gradient with 256-row tiles when the contraction (N) splits into
  // 128-element steps; everything else tiles rows by 128
  const bool dgrad2 = a->mode == NVQ_QAT_DGRAD && a->N % DSE == 0 && ((uintptr_t)a->w_codes & 7u) == 0 &&
                      a->N * (a->K / 2) < ((int64_t)1 << 31) && (int64_t)DBM * a->N * 2 < ((int64_t)1 << 31);
  hipLaunchKernelGGL(k_qat_tile_table, dim3(1), dim3(1024), 0, s, a->expert_offsets, (int)a->E,
                     L.tiles, L.ntiles, L.max_tiles, dgrad2 ? DBM : QBM);
  if (int rc = last_launch()) return rc;
  if (dgrad2) {
    p.n_tiles_n = (int)((a->K + DBN - 1) / DBN);
    const int64_t mt = (a->rows + DBM - 1) / DBM + a->E;
    const int64_t G2 = pick_grid(mt, kDgradGroupM, p.n_tiles_n);
    // wide weight path: whole 128-column tiles, 16-byte code and 4-byte scale loads
    if (a->K % DBN == 0 && ((uintptr_t)a->w_codes & 15u) == 0 && ((uintptr_t)a->w_scales & 3u) == 0)
      hipLaunchKernelGGL(k_qat_dgrad2<true>, dim3((unsigned)G2), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(k_qat_dgrad2<false>, dim3((unsigned)G2), dim3(256), 0, s, p);
    return last_launch();
  }
  p.n_tiles_m = 0;
  const int64_t cols = (a->mode == NVQ_QAT_FWD) ? a->N : a->K;
  p.n_tiles_n = (int)((cols + QBN - 1) / QBN);
  const int64_t G0 = (int64_t)L.max_tiles * p.n_tiles_n;
  const int64_t G = (G0 + 7) / 8 * 8;
  if (a->mode == NVQ_QAT_FWD && a->K % FSE == 0 && ((uintptr_t)a->w_scales & 3u) == 0) {
    p.n_tiles_n = (int)((a->N + FBN - 1) / FBN);
    const int64_t G2 = pick_grid(L.max_tiles, kFwdGroupM, p.n_tiles_n);
    hipLaunchKernelGGL(k_qat_fwd2, dim3((unsigned)G2), dim3(256), 0, s, p);
  } else if (a->mode == NVQ_QAT_FWD)
    hipLaunchKernelGGL((k_qat_gemm<NVQ_QAT_FWD, LD_ROWS, LD_FP4>), dim3((unsigned)G), dim3(QT), 0, s, p);
  else
    hipLaunchKernelGGL((k_qat_gemm<NVQ_QAT_DGRAD, LD_ROWS, LD_FP4_T>), dim3((unsigned)G), dim3(QT), 0, s,
                       p);
  return last_launch();
}

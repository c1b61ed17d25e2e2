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

namespace nvq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int QBM = 128;   // output rows per workgroup
constexpr int QBN = 256;   // output columns per workgroup (2 waves x 128)
constexpr int QBK = 64;    // contraction per LDS stage
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
                                                        int32_t* __restrict__ ntiles, int max_tiles) {
  __shared__ int32_t s_first[1025];
  const int e = threadIdx.x;
  int nt = 0;
  if (e < E) nt = (off[e + 1] - off[e] + QBM - 1) / QBM;
  if (e < E) s_first[e + 1] = nt;
  if (threadIdx.x == 0) s_first[0] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i <= E; ++i) s_first[i] += s_first[i - 1];
    *ntiles = min(s_first[E], max_tiles);
  }
  __syncthreads();
  if (e < E) {
    const int base = s_first[e];
    for (int t = 0; t < nt && base + t < max_tiles; ++t) {
      tiles[2 * (base + t)] = e;
      tiles[2 * (base + t) + 1] = off[e] + t * QBM;
    }
  }
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

// One operand tile of `nrows` rows (128 or 256) x QBK contraction values.
struct TileSrc {
  int kind;
  const uint16_t* bf;          // bf16 source base
  int64_t ld;                  // row stride of the source (elements)
  const int32_t* row_map;      // LD_ROWS / LD_ROWS_T: source row of local row / contraction index
  int row_map_div;             // divide row_map values (sorted pair -> token)
  int64_t row_base;            // first output row (LD_ROWS) or first contraction index (LD_ROWS_T)
  int64_t row_end;             // end of valid rows / contraction indices
  int64_t col_base;            // LD_ROWS_T / LD_FP4_T: first output column in the source
  int64_t col_end;             // valid columns end
  const uint8_t* codes;        // LD_FP4 / LD_FP4_T: weight codes of the expert [N, K/2]
  const uint8_t* scales;       // [N, K/16]
  int64_t wK;                  // weight K
  int64_t wN;                  // weight N
  int swap_nc;                 // unused (reserved)
  const int32_t* nmap;         // LD_FP4: weight row of local row (nullptr: identity from col_base)
};

__device__ __forceinline__ int64_t src_row(const TileSrc& s, int64_t i) {
  if (!s.row_map) return i;
  const int64_t v = s.row_map[i];
  return s.row_map_div > 0 ? v / s.row_map_div : v;
}

// Fill tile `dst` ([QQ][nrows][8] bf16) for contraction step ks.
template <int kRows>
__device__ __forceinline__ void fill_tile(const TileSrc& s, int ks, uint16_t* dst, int t) {
  const int64_t k0 = (int64_t)ks * QBK;
  if (s.kind == LD_ROWS) {
    // rows of the tile are output rows; 8 threads per row, 16 B each
    constexpr int kChunks = kRows * QQ;
#pragma unroll
    for (int u = 0; u < kChunks / QT; ++u) {
      const int c = t + QT * u;
      const int r = c / QQ, q = c % QQ;
      const int64_t gr = s.row_base + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gr < s.row_end) v = *reinterpret_cast<const uint4*>(s.bf + src_row(s, gr) * s.ld + k0 + q * 8);
      *reinterpret_cast<uint4*>(dst + ((size_t)q * kRows + r) * 8) = v;
    }
  } else if (s.kind == LD_ROWS_T) {
    // tile row = source column (col_base + r); contraction = source rows
    // (k0 + 4j .. +4).  Task = 4 source rows x 8 columns, transposed.
    constexpr int kTasks = (QBK / 4) * (kRows / 8);
#pragma unroll
    for (int u = 0; u < kTasks / QT; ++u) {
      const int task = t + QT * u;
      const int cg = task % (kRows / 8), pg = task / (kRows / 8);
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t p = k0 + 4 * pg + i;
        v[i] = make_uint4(0, 0, 0, 0);
        if (p < s.row_end - s.row_base && s.col_base + 8 * cg < s.col_end)
          v[i] = *reinterpret_cast<const uint4*>(s.bf + src_row(s, s.row_base + p) * s.ld + s.col_base + 8 * cg);
      }
      const int q = (4 * pg) / 8, off4 = (4 * pg) % 8;
      const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
      const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
      const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
      const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // columns 2j (low halves) and 2j+1 (high halves)
        const uint2 lo = make_uint2(pack_lo(w0[j], w1[j]), pack_lo(w2[j], w3[j]));
        const uint2 hi = make_uint2(pack_hi(w0[j], w1[j]), pack_hi(w2[j], w3[j]));
        *reinterpret_cast<uint2*>(dst + ((size_t)q * kRows + 8 * cg + 2 * j) * 8 + off4) = lo;
        *reinterpret_cast<uint2*>(dst + ((size_t)q * kRows + 8 * cg + 2 * j + 1) * 8 + off4) = hi;
      }
    }
  } else if (s.kind == LD_FP4) {
    // tile row = weight row n; contraction = weight K.  Task = one row x 32
    // values (16 B of codes, 2 block scales) -> 4 chunks of 8 bf16.
    const float st = 1.0f;  // tensor scale applied to the accumulators
    (void)st;
    constexpr int kTasks = kRows * (QBK / 32);
#pragma unroll
    for (int u = 0; u < kTasks / QT; ++u) {
      const int task = t + QT * u;
      const int r = task / (QBK / 32), hq = task % (QBK / 32);
      const int64_t n = s.nmap ? (int64_t)s.nmap[r] : s.col_base + r;
      uint4 o0 = make_uint4(0, 0, 0, 0), o1 = o0, o2 = o0, o3 = o0;
      if (n >= 0 && n < s.wN) {
        const int64_t kk = k0 + 32 * hq;
        const uint4 cw = *reinterpret_cast<const uint4*>(s.codes + n * (s.wK >> 1) + (kk >> 1));
        const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(s.scales + n * (s.wK >> 4) + (kk >> 4));
        const float sb0 = e4m3_to_f32(sc2 & 0xFFu), sb1 = e4m3_to_f32(sc2 >> 8);
        o0 = fp4x8_to_bf16(cw.x, sb0);
        o1 = fp4x8_to_bf16(cw.y, sb0);
        o2 = fp4x8_to_bf16(cw.z, sb1);
        o3 = fp4x8_to_bf16(cw.w, sb1);
      }
      const int q0 = 4 * hq;
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 0) * kRows + r) * 8) = o0;
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 1) * kRows + r) * 8) = o1;
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 2) * kRows + r) * 8) = o2;
      *reinterpret_cast<uint4*>(dst + ((size_t)(q0 + 3) * kRows + r) * 8) = o3;
    }
  } else {  // LD_FP4_T
    // tile row = weight column c (col_base + r); contraction = weight rows n
    // (k0 ..).  Task = 4 weight rows x 16 columns (one block), transposed.
    constexpr int kTasks = (QBK / 4) * (kRows / 16);
#pragma unroll
    for (int u = 0; u < kTasks / QT; ++u) {
      const int task = t + QT * u;
      const int cb = task % (kRows / 16), ng = task / (kRows / 16);
      const int64_t c0 = s.col_base + 16 * cb;
      uint32_t rowv[4][8];  // [weight row][column pair] packed bf16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = k0 + 4 * ng + i;
#pragma unroll
        for (int j = 0; j < 8; ++j) rowv[i][j] = 0u;
        if (n < s.wN && c0 < s.col_end) {
          const uint2 cw = *reinterpret_cast<const uint2*>(s.codes + n * (s.wK >> 1) + (c0 >> 1));
          const float sb = e4m3_to_f32(s.scales[n * (s.wK >> 4) + (c0 >> 4)]);
          const uint4 a = fp4x8_to_bf16(cw.x, sb), b = fp4x8_to_bf16(cw.y, sb);
          rowv[i][0] = a.x; rowv[i][1] = a.y; rowv[i][2] = a.z; rowv[i][3] = a.w;
          rowv[i][4] = b.x; rowv[i][5] = b.y; rowv[i][6] = b.z; rowv[i][7] = b.w;
        }
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
}

// Output tile QBM x QBN = (rows of A) x (rows of B); contraction nk stages.
template <int kMode>
__global__ __launch_bounds__(QT) void k_qat_gemm(QatParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][QQ * QBM * 8];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][QQ * QBN * 8];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, l32 = lane & 31, h = lane >> 5;

  TileSrc A, B;
  A.row_map = nullptr; A.row_map_div = 0; A.nmap = nullptr;
  B.row_map = nullptr; B.row_map_div = 0; B.nmap = nullptr;
  int e;
  int64_t out_r0, out_r_end, out_c0, out_c_end, nk;
  __shared__ int32_t s_nmap[QBN];

  if (kMode == NVQ_QAT_WGRAD) {
    // grid: E x n_tiles_m (over N) x n_tiles_n (over K); XCD-aware
    const int G = gridDim.x, per = G >> 3;
    const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    const int per_e = p.n_tiles_m * p.n_tiles_n;
    e = logical / per_e;
    if (e >= p.E) return;
    const int rem = logical % per_e;
    const int mt = rem % p.n_tiles_m, nt = rem / p.n_tiles_m;
    const int64_t pe0 = p.off[e], pe1 = p.off[e + 1];
    out_r0 = (int64_t)mt * QBM; out_r_end = p.N;
    out_c0 = (int64_t)nt * QBN; out_c_end = p.K;
    nk = (pe1 - pe0 + QBK - 1) / QBK;
    A.kind = LD_ROWS_T; A.bf = p.dy; A.ld = p.N; A.row_base = pe0; A.row_end = pe1;
    A.col_base = out_r0; A.col_end = p.N;
    B.kind = LD_ROWS_T; B.bf = p.x; B.ld = p.K; B.row_base = pe0; B.row_end = pe1;
    B.col_base = out_c0; B.col_end = p.K; B.row_map = p.a_row; B.row_map_div = p.a_row ? 0 : 0;
  } else {
    const int G = gridDim.x, per = G >> 3;
    const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    const int mt = logical % p.max_tiles, nt = logical / p.max_tiles;
    if (nt >= p.n_tiles_n || mt >= *p.ntiles) return;
    e = p.tiles[2 * mt];
    out_r0 = p.tiles[2 * mt + 1];
    out_r_end = p.off[e + 1];
    out_c0 = (int64_t)nt * QBN;
    const uint8_t* wc = p.w_codes + (int64_t)e * p.N * (p.K >> 1);
    const uint8_t* ws = p.w_scales + (int64_t)e * p.N * (p.K >> 4);
    if (kMode == NVQ_QAT_FWD) {
      out_c_end = p.N;
      nk = p.K / QBK;
      A.kind = LD_ROWS; A.bf = p.x; A.ld = p.K; A.row_map = p.a_row; A.row_base = out_r0;
      A.row_end = out_r_end;
      B.kind = LD_FP4; B.codes = wc; B.scales = ws; B.wK = p.K; B.wN = p.N; B.col_base = out_c0;
      B.col_end = p.N;
    } else {  // DGRAD
      out_c_end = p.K;
      nk = p.N / QBK;
      A.kind = LD_ROWS; A.bf = p.dy; A.ld = p.N; A.row_base = out_r0; A.row_end = out_r_end;
      B.kind = LD_FP4_T; B.codes = wc; B.scales = ws; B.wK = p.K; B.wN = p.N; B.col_base = out_c0;
      B.col_end = p.K;
    }
  }
  (void)s_nmap;

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  if (nk > 0) {
    fill_tile<QBM>(A, 0, sA[0], t);
    fill_tile<QBN>(B, 0, sB[0], t);
  }
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
#pragma unroll
    for (int s = 0; s < QBK / 16; ++s) {
      const int q = 2 * s + h;
      bf16x8_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sA[buf][((size_t)q * QBM + 32 * i + l32) * 8]);
        __builtin_memcpy(&af[i], &v, 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v =
            *reinterpret_cast<const uint4*>(&sB[buf][((size_t)q * QBN + 128 * wave + 32 * j + l32) * 8]);
        __builtin_memcpy(&bf[j], &v, 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) {
      // the other buffer was last read one step ago; everyone has passed the
      // barrier at the end of that step
      fill_tile<QBM>(A, ks + 1, sA[buf ^ 1], t);
      fill_tile<QBN>(B, ks + 1, sB[buf ^ 1], t);
    }
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
  if (a->K % QBK != 0 || a->N % QBK != 0) return NVQ_ESHAPE;  // 64-element contraction stages
  const bool wgrad = a->mode == NVQ_QAT_WGRAD;
  if (a->mode != NVQ_QAT_DGRAD && !a->x) return NVQ_EINVAL;
  if (a->mode != NVQ_QAT_FWD && !a->dy) return NVQ_EINVAL;
  if (!wgrad && (!a->w_codes || !a->w_scales || !a->w_tensor_scale)) return NVQ_EINVAL;
  if (!wgrad && !a->out_bf16 && !a->out_f32) return NVQ_EINVAL;
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
    p.n_tiles_m = (int)((a->N + QBM - 1) / QBM);
    p.n_tiles_n = (int)((a->K + QBN - 1) / QBN);
    const int64_t G0 = a->E * p.n_tiles_m * p.n_tiles_n;
    const int64_t G = (G0 + 7) / 8 * 8;
    hipLaunchKernelGGL(k_qat_gemm<NVQ_QAT_WGRAD>, dim3((unsigned)G), dim3(QT), 0, s, p);
    return last_launch();
  }
  if (a->rows == 0) return NVQ_OK;
  hipLaunchKernelGGL(k_qat_tile_table, dim3(1), dim3(1024), 0, s, a->expert_offsets, (int)a->E,
                     L.tiles, L.ntiles, L.max_tiles);
  if (int rc = last_launch()) return rc;
  p.n_tiles_m = 0;
  const int64_t cols = (a->mode == NVQ_QAT_FWD) ? a->N : a->K;
  p.n_tiles_n = (int)((cols + QBN - 1) / QBN);
  const int64_t G0 = (int64_t)L.max_tiles * p.n_tiles_n;
  const int64_t G = (G0 + 7) / 8 * 8;
  if (a->mode == NVQ_QAT_FWD)
    hipLaunchKernelGGL(k_qat_gemm<NVQ_QAT_FWD>, dim3((unsigned)G), dim3(QT), 0, s, p);
  else
    hipLaunchKernelGGL(k_qat_gemm<NVQ_QAT_DGRAD>, dim3((unsigned)G), dim3(QT), 0, s, p);
  return last_launch();
}

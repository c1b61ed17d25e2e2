// W4A4 MoE grouped GEMM with residual activation compensation (gfx950).
//
// Method: QUADS explainer §1 (native NVFP4 W4A4 GEMMs for the rollout) and
// §2.2-B (a correction computed on the highest-residual channels is added to
// the quantized output).  For sorted row p of expert e and token t = a_row[p]:
//   Y[p, n] = s_tA s_tW sum_c (G_A s_bA)[t, c] (G_W s_bW)[e, n, c]
//           + s_tW sum_j bf16(r[t, S_j]) (G_W s_bW)[e, n, S_j]
//
// Path DEQ16 (the one used): the NVFP4 E4M3-per-16 block scales do not fit the
// E8M0-per-32 scaled FP4 MFMA, so each FP4 fragment is dequantized exactly to
// fp16 in registers -- G * s_b has at most 6 significant bits and lies in
// [2^-10, 2688] -- and fed to v_mfma_f32_32x32x16_f16.  The hardware FP4->fp16
// conversion applies only the exponent of its scale argument, so it yields
// G * 2^8 and one v_pk_mul_f16 by the fp16 pattern (code << 7) = s_b * 2^-8
// (an fp16 subnormal for subnormal E4M3 codes) completes the product.  The
// tensor scales are applied to the fp32 accumulators; the compensation term
// runs as extra bf16 MFMA steps into the same accumulators between the
// s_tA and s_tW scalings.
//
// Tiling: workgroup = 2 waves = 128 rows x 256 columns; wave = 128 x 128
// (4 x 4 MFMA 32x32 tiles, accumulators in AGPRs); K staged through LDS in
// 128-element steps, double buffered: FP4 codes and raw E4M3 scale bytes only
// (4.5 bits/element), never dequantized 16-bit tiles.  A rows are gathered
// through a_row (token index).  Within a 128-element K step, lane half h owns
// elements [64h, 64h + 64) and MFMA step s takes elements 64h + 8s .. +8 from
// each half: any fixed K assignment works because A and B share it and every
// element carries its own block scale into the fragment.
//
// Workgroups map to tiles XCD-aware: consecutive logical tiles (same expert
// and column tile, consecutive row tiles) share their weight tile and land on
// the same XCD, so the second and third readers hit that XCD's L2.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "nvq.h"
#include "nvq_device.h"
#include "nvq_internal.h"

namespace nvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128;       // rows per workgroup
constexpr int BN = 256;       // columns per workgroup (2 waves x 128)
constexpr int BK = 128;       // K elements per LDS stage
constexpr int NTHR = 128;     // threads per workgroup
constexpr int KQ = BK / 32;   // 16-byte code chunks per row per stage (4)
constexpr int KB = BK / 16;   // scale bytes per row per stage (8)

struct GemmParams {
  int64_t rows, K, N, E, a_rows;
  const int32_t* a_row;
  int a_row_div;
  const int32_t* off;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_st;
  const uint16_t* a_resid;
  const int32_t* comp_idx;
  int k;
  int kpad;                 // k rounded up to 16 (row stride of wcomp)
  const uint16_t* wcomp;    // [E, N, kpad] bf16: dequantized weight at the selected channels
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_st;
  uint16_t* out_bf16;
  float* out_f32;
  const int32_t* tiles;   // [max_tiles][2]: expert, first row
  const int32_t* ntiles;  // [1]
  int max_tiles;
  int n_tiles_n;
  int swiglu;             // 1: gate/up fused weight, epilogue h = silu(gate) * up
};

// Tile table: expert e's rows [off[e], off[e+1]) split into BM-row tiles.
__global__ __launch_bounds__(1024) void k_tile_table(const int32_t* __restrict__ off, int E,
                                                    int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ ntiles, int max_tiles) {
  __shared__ int32_t s_first[1025];
  const int e = threadIdx.x;
  int nt = 0;
  if (e < E) nt = (off[e + 1] - off[e] + BM - 1) / BM;
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
      tiles[2 * (base + t) + 1] = off[e] + t * BM;
    }
  }
}

// Row of the A record (token) feeding sorted row pr.
__device__ __forceinline__ int64_t a_source_row(const GemmParams& p, int64_t pr) {
  if (!p.a_row) return pr;
  const int64_t v = p.a_row[pr];
  return p.a_row_div > 0 ? v / p.a_row_div : v;
}

// Weight row (column n of Y) held at local B row r of a workgroup.  With the
// SwiGLU epilogue each wave holds 64 gate rows then the 64 matching up rows.
__device__ __forceinline__ int64_t b_row_to_n(int r, int nt, int swiglu, int64_t N) {
  if (!swiglu) return (int64_t)nt * BN + r;
  const int w = r >> 7, q = r & 127;
  const int64_t I = N >> 1;
  const int64_t g0 = (int64_t)nt * (BN / 2) + 64 * w;
  return (q < 64) ? g0 + q : I + g0 + (q - 64);
}

// 8 FP4 codes (one dword) times one E4M3 scale -> 8 exact fp16 values.
__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t sc2) {
  half2_t s;
  __builtin_memcpy(&s, &sc2, 4);
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// E4M3 code byte b (0..3) of a dword -> fp16x2 pattern (code << 7) in both
// halves, i.e. s_b * 2^-8 twice.
__device__ __forceinline__ uint32_t scale_pair(uint32_t four, int b) {
  const uint32_t sel = (uint32_t)b | (0x0Cu << 8) | ((uint32_t)b << 16) | (0x0Cu << 24);
  return __builtin_amdgcn_perm(0u, four, sel) << 7;
}

// bf16 bits of the exact dequantized weight value G * s_b (<= 6 significant bits).
__device__ __forceinline__ uint32_t w_comp_bf16(const uint8_t* codes_row, const uint8_t* scales_row,
                                                int c) {
  const uint32_t byte = codes_row[c >> 1];
  const uint32_t nib = (c & 1) ? (byte >> 4) : (byte & 15u);
  const float v = e2m1_mag(nib & 7u) * e4m3_to_f32(scales_row[c >> 4]);
  return (__float_as_uint(v) >> 16) | ((nib & 8u) << 12);
}

// Packs the selected weight columns once per call: wcomp[e, n, j] = bf16 of
// the exact dequantized weight G * s_b at channel idx[j] (0 for j >= k).  One
// wave per weight row; the row's code bytes are fetched once and then hit L2.
__global__ __launch_bounds__(256) void k_gather_wcomp(const uint8_t* __restrict__ w_codes,
                                                     const uint8_t* __restrict__ w_scales,
                                                     int64_t rows_total, int64_t K,
                                                     const int32_t* __restrict__ idx, int k, int kpad,
                                                     uint16_t* __restrict__ wcomp) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows_total) return;
  const uint8_t* cr = w_codes + row * (K >> 1);
  const uint8_t* sr = w_scales + row * (K >> 4);
  for (int j = threadIdx.x & 63; j < kpad; j += 64)
    wcomp[row * kpad + j] = (uint16_t)((j < k) ? w_comp_bf16(cr, sr, idx[j]) : 0u);
}

template <int kSwiglu>
__global__ __launch_bounds__(NTHR) void k_moe_gemm_deq16(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][KQ][BM][16];
  __shared__ __attribute__((aligned(16))) uint8_t sAs[2][BM][KB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][KQ][BN][16];
  __shared__ __attribute__((aligned(16))) uint8_t sBs[2][BN][KB];

  // XCD-aware tile order (the grid is a multiple of 8 workgroups).
  const int G = gridDim.x;
  const int per = G >> 3;
  const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int mt = logical % p.max_tiles;
  const int nt = logical / p.max_tiles;
  if (nt >= p.n_tiles_n || mt >= *p.ntiles) return;
  const int e = p.tiles[2 * mt];
  const int64_t row0 = p.tiles[2 * mt + 1];
  const int64_t row_end = p.off[e + 1];
  const int64_t K = p.K, N = p.N;
  const int64_t Kh = K >> 1, Kb = K >> 4;

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int l32 = lane & 31, h = lane >> 5;

  // ---- loader state: each thread stages 4 A chunks, 8 B chunks, 1 A and 2 B scale rows
  const uint8_t* a_src[4];
  bool a_ok[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (t >> 2) + 32 * u;
    const int64_t pr = row0 + r;
    a_ok[u] = pr < row_end;
    const int64_t ar = a_ok[u] ? a_source_row(p, pr) : 0;
    a_src[u] = p.a_codes + ar * Kh + (t & 3) * 16;
  }
  const uint8_t* as_src;
  bool as_ok;
  {
    const int64_t pr = row0 + t;
    as_ok = pr < row_end;
    const int64_t ar = as_ok ? a_source_row(p, pr) : 0;
    as_src = p.a_scales + ar * Kb;
  }
  const uint8_t* wcodes_e = p.w_codes + (int64_t)e * N * Kh;
  const uint8_t* wscales_e = p.w_scales + (int64_t)e * N * Kb;
  const uint8_t* b_src[8];
  bool b_ok[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = (t >> 2) + 32 * u;
    const int64_t n = b_row_to_n(r, nt, kSwiglu, N);
    b_ok[u] = n < N;
    b_src[u] = wcodes_e + (b_ok[u] ? n : 0) * Kh + (t & 3) * 16;
  }
  const uint8_t* bs_src[2];
  bool bs_ok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t n = b_row_to_n(t + 128 * u, nt, kSwiglu, N);
    bs_ok[u] = n < N;
    bs_src[u] = wscales_e + (bs_ok[u] ? n : 0) * Kb;
  }

  uint4 ra[4], rb[8];
  uint2 ras, rbs[2];
  auto gload = [&](int kstep) {
    const int64_t kc = (int64_t)kstep * (BK / 2), ks = (int64_t)kstep * KB;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ra[u] = a_ok[u] ? *reinterpret_cast<const uint4*>(a_src[u] + kc) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      rb[u] = b_ok[u] ? *reinterpret_cast<const uint4*>(b_src[u] + kc) : make_uint4(0, 0, 0, 0);
    ras = as_ok ? *reinterpret_cast<const uint2*>(as_src + ks) : make_uint2(0, 0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      rbs[u] = bs_ok[u] ? *reinterpret_cast<const uint2*>(bs_src[u] + ks) : make_uint2(0, 0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(&sA[buf][t & 3][(t >> 2) + 32 * u][0]) = ra[u];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      *reinterpret_cast<uint4*>(&sB[buf][t & 3][(t >> 2) + 32 * u][0]) = rb[u];
    *reinterpret_cast<uint2*>(&sAs[buf][t][0]) = ras;
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<uint2*>(&sBs[buf][t + 128 * u][0]) = rbs[u];
  };

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (int)(K / BK);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    // scale bytes of this lane's 4 blocks (lane half h owns blocks 4h .. 4h+3)
    uint32_t asc[4], bsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      asc[i] = *reinterpret_cast<const uint32_t*>(&sAs[buf][32 * i + l32][4 * h]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bsc[j] = *reinterpret_cast<const uint32_t*>(&sBs[buf][128 * wave + 32 * j + l32][4 * h]);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 ac[4], bc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ac[i] = *reinterpret_cast<const uint4*>(&sA[buf][2 * h + half][32 * i + l32][0]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bc[j] = *reinterpret_cast<const uint4*>(&sB[buf][2 * h + half][128 * wave + 32 * j + l32][0]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int sb = 2 * half + (s >> 1);  // block within this lane half's 4
        half8_t af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = s == 0 ? ac[i].x : s == 1 ? ac[i].y : s == 2 ? ac[i].z : ac[i].w;
          af[i] = dequant8(w, scale_pair(asc[i], sb));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = s == 0 ? bc[j].x : s == 1 ? bc[j].y : s == 2 ? bc[j].z : bc[j].w;
          bf[j] = dequant8(w, scale_pair(bsc[j], sb));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) {
      __syncthreads();  // everyone is done reading buf ^ 1 from the previous step
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- s_tA, then the compensation steps, then s_tW
  const float sta = *p.a_st;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] *= sta;

  if (p.k > 0) {
    const int nsteps = (p.k + 15) / 16;
    int64_t arow_i[4];
    bool arow_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t pr = row0 + 32 * i + l32;
      arow_ok[i] = pr < row_end;
      arow_i[i] = arow_ok[i] ? a_source_row(p, pr) : 0;
    }
    const uint16_t* wrow[4];
    bool wok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = b_row_to_n(128 * wave + 32 * j + l32, nt, kSwiglu, N);
      wok[j] = n < N;
      wrow[j] = p.wcomp + ((int64_t)e * N + (wok[j] ? n : 0)) * p.kpad;
    }
    for (int st = 0; st < nsteps; ++st) {
      const int c0 = 16 * st + 8 * h;  // this lane's 8 compensation channels (k % 8 == 0)
      bf16x8_t af[4], bf[4];
      const bool cin = c0 < p.k;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (arow_ok[i] && cin) v = *reinterpret_cast<const uint4*>(p.a_resid + arow_i[i] * p.k + c0);
        __builtin_memcpy(&af[i], &v, 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (wok[j]) v = *reinterpret_cast<const uint4*>(wrow[j] + c0);
        __builtin_memcpy(&bf[j], &v, 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  const float stw = p.w_st[e];
  // ---- epilogue.  acc[i][j][v]: row 32i + 8(v/4) + 4h + v%4, column 32j + l32 of the wave tile.
  if (!kSwiglu) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t pr = row0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (pr >= row_end) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t n = (int64_t)nt * BN + 128 * wave + 32 * j + l32;
          if (n >= N) continue;
          const float y = acc[i][j][v] * stw;
          if (p.out_f32) p.out_f32[pr * N + n] = y;
          if (p.out_bf16) p.out_bf16[pr * N + n] = (uint16_t)f32_to_bf16_rne(y);
        }
      }
  } else {
    const int64_t I = N >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t pr = row0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (pr >= row_end) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t ng = (int64_t)nt * (BN / 2) + 64 * wave + 32 * j + l32;
          if (ng >= I) continue;
          const float g = acc[i][j][v] * stw;
          const float u = acc[i][j + 2][v] * stw;
          if (p.out_f32) {
            p.out_f32[pr * N + ng] = g;
            p.out_f32[pr * N + I + ng] = u;
          }
          const float hv = g / (1.0f + __expf(-g)) * u;
          if (p.out_bf16) p.out_bf16[pr * I + ng] = (uint16_t)f32_to_bf16_rne(hv);
        }
      }
  }
}

struct MoeLayout {
  int max_tiles;
  int kpad;
  int32_t* tiles;
  int32_t* ntiles;
  uint16_t* wcomp;
  size_t bytes;
};

MoeLayout moe_layout(void* ws, int64_t rows, int64_t E, int64_t N, int64_t k) {
  MoeLayout L;
  L.max_tiles = (int)((rows + BM - 1) / BM + E);
  L.kpad = (int)((k + 15) / 16 * 16);
  WsCarve c(ws);
  L.tiles = c.take<int32_t>((size_t)L.max_tiles * 2);
  L.ntiles = c.take<int32_t>(1);
  L.wcomp = c.take<uint16_t>((size_t)(E * N * L.kpad));
  L.bytes = c.off;
  return L;
}

}  // namespace
}  // namespace nvq

using namespace nvq;

extern "C" size_t moe_gemm_workspace_bytes(int64_t rows, int64_t E, int64_t N, int32_t k) {
  if (rows < 0 || E < 1 || N < 1 || k < 0) return kAlign;
  return moe_layout(nullptr, rows, E, N, k).bytes;
}

extern "C" int moe_grouped_gemm_w4a4_comp(const nvq_moe_gemm_args* a, void* stream) {
  if (!a || a->struct_size < sizeof(nvq_moe_gemm_args)) return NVQ_EINVAL;
  if (!a->expert_offsets || !a->a_codes || !a->a_scales || !a->a_tensor_scale || !a->w_codes ||
      !a->w_scales || !a->w_tensor_scale || !a->ws)
    return NVQ_EINVAL;
  if (!a->out_bf16 && !a->out_f32) return NVQ_EINVAL;
  if (a->epilogue != NVQ_EPI_NONE && a->epilogue != NVQ_EPI_SWIGLU) return NVQ_EINVAL;
  if (a->path != NVQ_GEMM_AUTO && a->path != NVQ_GEMM_DEQ16 && a->path != NVQ_GEMM_FP8_BLOCK)
    return NVQ_EINVAL;
  if (a->path == NVQ_GEMM_FP8_BLOCK) return NVQ_EUNSUPPORTED;
  if (a->rows < 0 || a->E < 1 || a->E > 1024 || a->N <= 0 || a->K <= 0) return NVQ_ESHAPE;
  if (a->K % BK != 0) return NVQ_ESHAPE;  // the FP4 stage is 128 elements of K
  if (a->epilogue == NVQ_EPI_SWIGLU && (a->N % 2 != 0)) return NVQ_ESHAPE;
  if (a->k < 0 || a->k > a->K || (a->k & 7)) return NVQ_ESHAPE;
  if (a->k > 0 && (!a->a_resid || !a->comp_idx)) return NVQ_EINVAL;
  if (a->a_row_div < 0) return NVQ_EINVAL;
  if (((uintptr_t)a->a_codes & 15u) || ((uintptr_t)a->w_codes & 15u) ||
      (a->k > 0 && ((uintptr_t)a->a_resid & 15u)) ||
      ((uintptr_t)a->a_scales & 7u) || ((uintptr_t)a->w_scales & 7u))
    return NVQ_EALIGN;
  if (!aligned256(a->ws)) return NVQ_EALIGN;
  MoeLayout L = moe_layout(a->ws, a->rows, a->E, a->N, a->k);
  if (a->ws_bytes < L.bytes) return NVQ_EWORKSPACE;
  if (a->rows == 0) return NVQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_tile_table, dim3(1), dim3(1024), 0, s, a->expert_offsets, (int)a->E, L.tiles,
                     L.ntiles, L.max_tiles);
  if (int rc = last_launch()) return rc;
  GemmParams p;
  p.rows = a->rows; p.K = a->K; p.N = a->N; p.E = a->E; p.a_rows = a->a_rows;
  p.a_row = a->a_row; p.a_row_div = a->a_row_div; p.off = a->expert_offsets;
  p.a_codes = a->a_codes; p.a_scales = a->a_scales; p.a_st = a->a_tensor_scale;
  p.a_resid = a->a_resid; p.comp_idx = a->comp_idx; p.k = a->k;
  p.kpad = L.kpad; p.wcomp = L.wcomp;
  if (a->k > 0) {
    const int64_t wrows = a->E * a->N;
    hipLaunchKernelGGL(k_gather_wcomp, dim3((unsigned)((wrows + 3) / 4)), dim3(256), 0, s, a->w_codes,
                       a->w_scales, wrows, a->K, a->comp_idx, (int)a->k, L.kpad, L.wcomp);
    if (int rc = last_launch()) return rc;
  }
  p.w_codes = a->w_codes; p.w_scales = a->w_scales; p.w_st = a->w_tensor_scale;
  p.out_bf16 = a->out_bf16; p.out_f32 = a->out_f32;
  p.tiles = L.tiles; p.ntiles = L.ntiles; p.max_tiles = L.max_tiles;
  const bool swiglu = a->epilogue == NVQ_EPI_SWIGLU;
  p.swiglu = swiglu ? 1 : 0;
  p.n_tiles_n = swiglu ? (int)((a->N / 2 + BN / 2 - 1) / (BN / 2)) : (int)((a->N + BN - 1) / BN);
  const int64_t G0 = (int64_t)L.max_tiles * p.n_tiles_n;
  const int64_t G = (G0 + 7) / 8 * 8;
  if (swiglu)
    hipLaunchKernelGGL(k_moe_gemm_deq16<1>, dim3((unsigned)G), dim3(NTHR), 0, s, p);
  else
    hipLaunchKernelGGL(k_moe_gemm_deq16<0>, dim3((unsigned)G), dim3(NTHR), 0, s, p);
  return last_launch();
}

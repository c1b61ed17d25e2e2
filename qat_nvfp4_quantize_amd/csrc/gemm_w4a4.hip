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
// Tiling: workgroup = 4 waves = 128 rows x 256 columns, two workgroups per
// CU (each wave keeps its 128 x 64 accumulators in VGPRs, at most 256
// registers, so two waves share a SIMD and one covers the other's barrier
// and memory waits).  K advances 128 elements per step.  The A tile (128
// rows, shared by the four waves) is dequantized once per workgroup to exact
// fp16 into a double-buffered LDS tile (272-byte rows: the 16-byte fragment
// reads of consecutive rows hit distinct banks).  Each wave's 64 weight rows
// are used by that wave only, so they skip LDS: they are loaded straight into
// registers in MFMA fragment order, two steps ahead, and dequantized there.
// Within a 128-element step, lane half h owns elements [64h, 64h + 64) and
// MFMA sub-step d takes its elements 64h + 8d .. +8: any fixed K assignment
// works because A and B share it and every element carries its own block
// scale into the fragment.  A rows are gathered through a_row (token index).
// The compensation runs as extra bf16 steps of 128 channels through the same
// LDS tile (residual columns) and registers (packed weight columns).
//
// Workgroups map to tiles XCD-aware: each XCD walks a contiguous range of
// logical tiles, ordered by groups of 4 row tiles, then column tile, then row
// tile within the group, so the workgroups resident on one XCD share a few
// A and B tiles in that XCD's L2.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "nvq.h"
#include "nvq_device.h"
#include "nvq_internal.h"
#include "nvq_scan.h"

namespace nvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int NTHR = 256;     // threads per workgroup (4 waves)
constexpr int BM = 128;       // rows per workgroup
constexpr int BN = 256;       // columns per workgroup (4 waves x 64)
constexpr int WN = 64;        // columns per wave
constexpr int SE = 128;       // K elements per step
constexpr int LROW = 272;     // LDS bytes per A tile row (256 data + 16 pad)

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
  int bm;                 // row tile of the tile table
  uint32_t* h_amax;       // SwiGLU: max |h| over the stored bf16 h, as fp32 bits; or NULL
  int bf16_rows16;        // out_bf16 rows may be written in 16-byte pieces (N % 8 == 0, aligned)
  int h_rows16;           // SwiGLU: rows of h (N / 2 wide) may be written in 16-byte pieces
  // fused combine (NULL comb_out: none)
  const int32_t* comb_pair;
  const int32_t* comb_pos;
  const float* comb_w;
  int comb_topk;
  uint16_t* comb_out;
  uint32_t* comb_cnt;     // [T, n_tiles_n] arrival counters, zero at launch
};

// Before a GEMM with the fused combine: clears the arrival counters, and
// writes the output row of every token none of whose pairs has a row (all
// dropped by the permutation): its combine is the empty sum, 0.
__global__ __launch_bounds__(256) void k_comb_prep(uint32_t* __restrict__ cnt, int64_t n_cnt,
                                                  const int32_t* __restrict__ pos, int64_t T, int topk,
                                                  uint16_t* __restrict__ out, int64_t N) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_cnt; i += stride) cnt[i] = 0u;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < T; t += stride) {
    bool any = false;
    for (int j = 0; j < topk; ++j) any = any || pos[t * topk + j] >= 0;
    if (any) continue;
    for (int64_t c = 0; c < N; c += 8) *reinterpret_cast<uint4*>(out + t * N + c) = make_uint4(0, 0, 0, 0);
  }
}

// Tile table: expert e's rows [off[e], off[e+1]) split into BM-row tiles.
// Also clears the h amax word, ahead of the GEMM on the same stream.
__global__ __launch_bounds__(1024) void k_tile_table(const int32_t* __restrict__ off, int E, int BM,
                                                    int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ ntiles, int max_tiles,
                                                    uint32_t* __restrict__ h_amax) {
  __shared__ int32_t s_wave[16];
  if (h_amax && threadIdx.x == 0) *h_amax = 0u;
  __shared__ int32_t s_incl[1024];
  build_tile_table(off, E, BM, tiles, ntiles, max_tiles, s_wave, s_incl);
}

__global__ void k_clear_word(uint32_t* w) { *w = 0u; }

// Row of the A record (token) feeding sorted row pr.
__device__ __forceinline__ int64_t a_source_row(const GemmParams& p, int64_t pr) {
  if (!p.a_row) return pr;
  const int64_t v = p.a_row[pr];
  return p.a_row_div > 0 ? v / p.a_row_div : v;
}

// Weight row (column n of Y) held at local B row r (0..255) of column tile
// nt.  With the SwiGLU epilogue each wave's 64 rows are 32 gate rows then the
// 32 matching up rows, so a lane holds gate and up of the same column.
__device__ __forceinline__ int64_t b_row_to_n(int r, int nt, int swiglu, int64_t N) {
  if (!swiglu) return (int64_t)nt * BN + r;
  const int w = r >> 6, q = r & 63;
  const int64_t I = N >> 1;
  const int64_t g0 = (int64_t)nt * (BN / 2) + 32 * w;
  return (q < 32) ? g0 + q : I + g0 + (q - 32);
}

// E4M3 code byte b (0..3) of a dword -> fp16x2 pattern (code << 7) in both
// halves, i.e. s_b * 2^-8 twice.
__device__ __forceinline__ uint32_t scale_pair(uint32_t four, int b) {
  const uint32_t sel = (uint32_t)b | (0x0Cu << 8) | ((uint32_t)b << 16) | (0x0Cu << 24);
  return __builtin_amdgcn_perm(0u, four, sel) << 7;
}

// 8 FP4 codes (one dword) times the fp16x2 scale pattern -> 8 exact fp16 values.
__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t pat) {
  half2_t s;
  __builtin_memcpy(&s, &pat, 4);
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

__device__ __forceinline__ uint32_t dword_of(const uint4 (&c)[2], int d) {
  const uint4& v = c[d >> 2];
  return (d & 3) == 0 ? v.x : (d & 3) == 1 ? v.y : (d & 3) == 2 ? v.z : v.w;
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

// Channel-major copy of a weight record.  Codes: a 64 x 64 (rows n x
// columns c) tile through LDS; output byte (c, m) packs rows 2m (low nibble)
// and 2m + 1.  N and K are multiples of 16, so every 16-row or 16-column
// group is wholly inside or outside the matrix.
__global__ __launch_bounds__(256) void k_codes_cm(const uint8_t* __restrict__ codes, int64_t N, int64_t K,
                                                 uint8_t* __restrict__ codes_cm) {
  __shared__ uint32_t tile[64][9];  // row n: 32 code bytes (64 columns) + pad
  const int64_t b = blockIdx.z, n0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int t = threadIdx.x;
  {
    const int r = t >> 2, q = t & 3;  // row n0 + r, code bytes 8q .. 8q + 7 (columns c0 + 16q ..)
    uint2 v = make_uint2(0u, 0u);
    if (n0 + r < N && c0 + 16 * q < K)
      v = *reinterpret_cast<const uint2*>(codes + (b * N + n0 + r) * (K >> 1) + (c0 >> 1) + 8 * q);
    tile[r][2 * q] = v.x;
    tile[r][2 * q + 1] = v.y;
  }
  __syncthreads();
  const int c = t >> 2, q = t & 3;  // column c0 + c, output bytes 8q .. 8q + 7 (rows n0 + 16q ..)
  if (c0 + c >= K || n0 + 16 * q >= N) return;
  const int sh = 4 * (c & 7);  // nibble of column c in its word
  uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int n = 16 * q + 2 * m;
    const uint32_t lo = (tile[n][c >> 3] >> sh) & 15u, hi = (tile[n + 1][c >> 3] >> sh) & 15u;
    const uint32_t byte = (lo | (hi << 4)) << (8 * (m & 3));
    if (m < 4) w0 |= byte; else w1 |= byte;
  }
  *reinterpret_cast<uint2*>(codes_cm + (b * K + c0 + c) * (N >> 1) + (n0 >> 1) + 8 * q) = make_uint2(w0, w1);
}

// Scales [b, N, K/16] -> [b, K/16, N]: a 64 x 64 byte transpose through LDS.
__global__ __launch_bounds__(256) void k_scales_cm(const uint8_t* __restrict__ scales, int64_t N, int64_t KB,
                                                  uint8_t* __restrict__ scales_cm) {
  __shared__ uint8_t tile[64][65];
  const int64_t b = blockIdx.z, n0 = (int64_t)blockIdx.y * 64, s0 = (int64_t)blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, cc = i & 63;
    tile[r][cc] = (n0 + r < N && s0 + cc < KB) ? scales[(b * N + n0 + r) * KB + s0 + cc] : (uint8_t)0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i >> 6, r = i & 63;
    if (s0 + cc < KB && n0 + r < N) scales_cm[(b * KB + s0 + cc) * N + n0 + r] = tile[r][cc];
  }
}

// bf16 bits of G * s_b for code nibble nib and E4M3 scale byte sc (exact).
__device__ __forceinline__ uint32_t wq_bf16(uint32_t nib, uint32_t sc) {
  const float v = e2m1_mag(nib & 7u) * e4m3_to_f32(sc);
  return (__float_as_uint(v) >> 16) | ((nib & 8u) << 12);
}

// The compensation weights from the channel-major record: wcomp[e, n, j] =
// bf16 of G * s_b at channel idx[j] (0 for j >= k).  Workgroup = 64 weight
// rows x one 64-channel slice of wcomp (blockIdx.y) of one expert.  Thread t
// takes rows 2 (t % 32), + 1 and channels 8 (t / 32) .. + 7 of the slice:
// eight independent (code byte, two scale bytes) loads from those channels'
// contiguous rows (lanes along the rows, so each load instruction reads
// consecutive bytes; k is a multiple of 8, so a group of 8 channels is wholly
// below k or past it), decoded branch-free (the hardware FP4 conversion gives
// both rows' G, signed; G * s_b has at most 6 significant bits, so its bf16
// is exact) into an LDS tile.  Then each group of 8 threads stores one row's
// 128 slice bytes as 16-byte pieces, so every output line is written whole
// by one workgroup.  With tiles set, the grid has one more z slice whose
// first workgroup builds the GEMM's tile table (and clears h_amax) while
// the others gather: one launch less per call.
constexpr int kWcRows = 64, kWcCh = 64, kWcPitch = kWcCh + 8;  // tile pitch in bf16 (+16 bytes)
__global__ __launch_bounds__(256) void k_gather_wcomp_rows(const uint8_t* __restrict__ codes_cm,
                                                          const uint8_t* __restrict__ scales_cm, int64_t N,
                                                          int64_t K, const int32_t* __restrict__ idx, int k,
                                                          int kpad, uint16_t* __restrict__ wcomp,
                                                          const int32_t* __restrict__ off, int E, int bm,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles, int max_tiles,
                                                          uint32_t* __restrict__ h_amax) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kWcRows][kWcPitch];
  static_assert(sizeof(tile) >= (1024 + 16) * sizeof(int), "tile table prefixes alias the tile");
  if (tiles && blockIdx.z == (unsigned)E) {  // the extra slice (uniform over the workgroup)
    if (blockIdx.x | blockIdx.y) return;
    if (h_amax && threadIdx.x == 0) *h_amax = 0u;
    int* s_wave = reinterpret_cast<int*>(&tile[0][0]);
    build_tile_table(off, E, bm, tiles, ntiles, max_tiles, s_wave, s_wave + 16);
    return;
  }
  const int64_t e = blockIdx.z;
  const int64_t n0 = (int64_t)blockIdx.x * kWcRows;
  const int c0 = kWcCh * (int)blockIdx.y;
  const int t = threadIdx.x, q = t >> 5, rp = t & 31;
  const int j0 = c0 + 8 * q;
  const int64_t n = n0 + 2 * rp;
  if (j0 < kpad) {
    uint4 o0 = make_uint4(0, 0, 0, 0), o1 = make_uint4(0, 0, 0, 0);
    if (j0 < k && n < N) {
      const uint8_t* cb = codes_cm + e * K * (N >> 1) + (n >> 1);
      const uint8_t* sb = scales_cm + e * (K >> 4) * N + n;
      int64_t ch[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ch[u] = idx[j0 + u];
      uint32_t byte[8], sc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        byte[u] = cb[ch[u] * (N >> 1)];
        sc[u] = *reinterpret_cast<const uint16_t*>(sb + (ch[u] >> 4) * N);
      }
      auto e4m3 = [](uint32_t c) {  // c <= 0x7E
        const float nrm = __uint_as_float(((c & 0x7Fu) << 20) + (120u << 23));
        const float sub = (float)(c & 7u) * 0x1p-9f;
        return (c & 0x78u) ? nrm : sub;
      };
      uint32_t r0[4], r1[4];
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        uint32_t lo[2], hi[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte[u + v], 1.0f, 0);
          lo[v] = __float_as_uint(g[0] * e4m3(sc[u + v] & 0xFFu)) >> 16;
          hi[v] = __float_as_uint(g[1] * e4m3(sc[u + v] >> 8)) >> 16;
        }
        r0[u >> 1] = lo[0] | (lo[1] << 16);
        r1[u >> 1] = hi[0] | (hi[1] << 16);
      }
      o0 = make_uint4(r0[0], r0[1], r0[2], r0[3]);
      o1 = make_uint4(r1[0], r1[1], r1[2], r1[3]);
    }
    *reinterpret_cast<uint4*>(&tile[2 * rp][8 * q]) = o0;
    *reinterpret_cast<uint4*>(&tile[2 * rp + 1][8 * q]) = o1;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (t >> 3) + 32 * h, cq = t & 7;
    const int64_t nr = n0 + r;
    if (nr < N && c0 + 8 * cq < kpad)
      *reinterpret_cast<uint4*>(wcomp + (e * N + nr) * kpad + c0 + 8 * cq) =
          *reinterpret_cast<const uint4*>(&tile[r][8 * cq]);
  }
}

// The tile of this workgroup.  XCD-aware order: the grid is sized for the
// most row tiles the offsets allow and the real count comes from the tile
// table.  Workgroups are dealt to the 8 XCDs round-robin, so XCD x =
// blockIdx % 8 takes the contiguous logical range [x * per, (x + 1) * per)
// of the real tiles, in groups of kGroupM row tiles x all column tiles (the
// row tiles of a group, consecutive in the order, read the same weight tile
// at about the same time); surplus workgroups get valid == false.
constexpr int kGroupM = 8;
struct TileCtx {
  bool valid;
  int e, nt;
  int64_t row0, row_end;
};
template <int kGM = kGroupM>
__device__ __forceinline__ TileCtx tile_of_block(const GemmParams& p) {
  TileCtx c;
  c.valid = false;
  const int n_mt = min(*p.ntiles, p.max_tiles);
  const int n_groups = (n_mt + kGM - 1) / kGM;
  const int total = n_groups * kGM * p.n_tiles_n;
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  if (slot >= per) return c;
  const int logical = (blockIdx.x & 7) * per + slot;
  if (logical >= total) return c;
  const int group_span = kGM * p.n_tiles_n;
  const int grp = logical / group_span, rem = logical - grp * group_span;
  const int mt = kGM * grp + (rem % kGM);
  if (mt >= n_mt) return c;
  c.valid = true;
  c.nt = rem / kGM;
  c.e = p.tiles[2 * mt];
  c.row0 = p.tiles[2 * mt + 1];
  c.row_end = p.off[c.e + 1];
  return c;
}

// Token row of A loader row ar (clamped to the expert's last row) and the
// weight rows of this lane's two B fragments (clamped to N - 1): rows past
// the ends are read but never stored, so every load is unconditional.
__device__ __forceinline__ int64_t loader_a_token(const GemmParams& p, const TileCtx& c, int ar) {
  return a_source_row(p, min<int64_t>(c.row0 + ar, c.row_end - 1));
}
template <int kSwiglu>
__device__ __forceinline__ int64_t loader_b_row(const GemmParams& p, const TileCtx& c, int wave, int j,
                                                int l32) {
  return min<int64_t>(b_row_to_n(WN * wave + 32 * j + l32, c.nt, kSwiglu, p.N), p.N - 1);
}

// Direct global -> LDS load of 16 bytes per lane: lane l lands at LDS byte
// lds_addr + 16 l (lds_addr wave-uniform, read from the first lane).  Issued
// from inline assembly, so the compiler places no wait for it in front of
// unrelated LDS reads; the reader waits (vmcnt) and synchronizes itself.
#define NVQ_LDS_U8 __attribute__((address_space(3))) uint8_t
__device__ __forceinline__ void dma16_lds(const void* g, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}

// The compensation operands of the first 128-channel step, fetched while
// the last main-loop MFMAs run (path DEQ16): the residual rows of the tile go
// global -> LDS with direct loads into a compact tile of S = 8 (k <= 64) or
// 16 slots of 16 bytes per row, slot s of row r stored at s ^ (r & (S - 1));
// the weight fragments of its first kD sub-steps (16 channels each) go into
// registers: 4 for the down projection, 3 with the SwiGLU epilogue (a fourth
// would spill there).  s_tok[r]: the A source row of tile row r.
template <int kD>
struct CompPre {
  uint4 w[2][kD];
  int S;
};
template <int kD>
__device__ __forceinline__ void comp_prefetch(const GemmParams& p, uint32_t lds0, const int64_t* s_tok,
                                              const TileCtx& c, const int64_t (&b_n)[2], CompPre<kD>& cp) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, h = lane >> 5;
  const int rem = min(p.k, SE);
  cp.S = rem > 64 ? 16 : 8;
  const int S = cp.S, nld = S / 2;  // 1 KB loads per wave: 128 rows x S slots / 4 waves
  const int rl = lane / S, ps = lane & (S - 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < nld) {
      const int g = nld * wave + i;  // load g covers tile rows (64 / S) g ..
      const int r = (64 / S) * g + rl;
      const int ls = ps ^ (r & (S - 1));
      dma16_lds(p.a_resid + s_tok[r] * p.k + min(8 * ls, p.k - 8), lds0 + 1024u * g);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint16_t* w_src = p.wcomp + ((int64_t)c.e * p.N + b_n[j]) * p.kpad;
#pragma unroll
    for (int d = 0; d < kD; ++d)
      if (16 * d < rem) cp.w[j][d] = *reinterpret_cast<const uint4*>(w_src + min(16 * d + 8 * h, p.kpad - 8));
  }
}

// acc *= s_tA, then the compensation: 128-channel bf16 steps with the
// residual rows through the LDS tile and the packed weight columns loaded in
// fragment order.  Channels past k (kpad) read as zero.  With kPre, the first
// step's operands were fetched by comp_prefetch into pre (residual tile at
// the start of lds), and the caller has waited for them and synchronized the
// workgroup; later steps load their own.  kNI: the live 32-row sub-tiles
// (the MFMAs of the others are skipped).
template <bool kPre, int kD, int kNI = 4>
__device__ __forceinline__ void comp_phase(const GemmParams& p, const TileCtx& c,
                                           floatx16_t (&acc)[4][2], uint8_t (*lds)[LROW],
                                           int64_t a_tok, const int64_t (&b_n)[2], const CompPre<kD>& pre) {
  const float sta = *p.a_st;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] *= sta;
  if (p.k <= 0) return;
  const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, h = lane >> 5;
  const int ar = t >> 1, ahh = t & 1;
  const uint16_t* r_src = p.a_resid + a_tok * p.k;
  const uint16_t* w_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) w_src[j] = p.wcomp + ((int64_t)c.e * p.N + b_n[j]) * p.kpad;
  const int ncs = (p.k + SE - 1) / SE;
  // Sub-step d of a 128-channel step covers channels 16 d .. 16 d + 15 (lane
  // half h: 16 d + 8 h ..), so the sub-steps past k are skipped wave-uniformly
  // (k = 64 runs half the MFMAs of a step).  Every load of a step is issued
  // before the first wait: addresses are clamped into the row (k and kpad are
  // multiples of 8) and channels past k are zeroed by a select afterwards.  A
  // load under a per-lane condition would be followed by its own wait, one
  // memory round trip each.
  auto keep = [](bool live, uint4 v) {
    const uint32_t m = live ? 0xFFFFFFFFu : 0u;
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
  };
  int cs = 0;
  if (kPre) {
    // the prefetched first step: the caller waited for its loads and met
    // the other waves at a barrier, so every wave's direct loads have landed
    const int rem = min(p.k, SE), S = pre.S;
    const uint8_t* tile = &lds[0][0];
    uint4 wl[2][8 - kD];  // sub-steps kD.., loaded now
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint16_t* w_src = p.wcomp + ((int64_t)c.e * p.N + b_n[j]) * p.kpad;
#pragma unroll
      for (int d = kD; d < 8; ++d)
        if (16 * d < rem) wl[j][d - kD] = *reinterpret_cast<const uint4*>(w_src + min(16 * d + 8 * h, p.kpad - 8));
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      if (16 * d >= rem) break;
      bf16x8_t af[kNI], bf[2];
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        const int r = 32 * i + l32;
        af[i] = *reinterpret_cast<const bf16x8_t*>(tile + 16 * (S * r + ((2 * d + h) ^ (r & (S - 1)))));
      }
      const bool live = 16 * d + 8 * h < rem;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 v = keep(live, d < kD ? pre.w[j][d < kD ? d : 0] : wl[j][d < kD ? 0 : d - kD]);
        __builtin_memcpy(&bf[j], &v, 16);
      }
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    cs = 1;
  }
  for (; cs < ncs; ++cs) {
    const int rem = p.k - SE * cs;  // channels left, uniform
    uint4 rv[8], wv[2][8];
#pragma unroll
    for (int q = 0; q < 8; ++q)  // residual channels 16 q + 8 ahh .. + 7
      if (16 * q < rem) rv[q] = *reinterpret_cast<const uint4*>(r_src + min(SE * cs + 16 * q + 8 * ahh, p.k - 8));
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (16 * d < rem)
          wv[j][d] = *reinterpret_cast<const uint4*>(w_src[j] + min(SE * cs + 16 * d + 8 * h, p.kpad - 8));
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (16 * q < rem)
        *reinterpret_cast<uint4*>(&lds[ar][32 * q + 16 * ahh]) = keep(16 * q + 8 * ahh < rem, rv[q]);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      if (16 * d >= rem) break;
      bf16x8_t af[kNI], bf[2];
#pragma unroll
      for (int i = 0; i < kNI; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&lds[32 * i + l32][32 * d + 16 * h]);
      const bool live = 16 * d + 8 * h < rem;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 v = keep(live, wv[j][d]);
        __builtin_memcpy(&bf[j], &v, 16);
      }
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
}

// acc + w * y with two roundings (no fused multiply-add), as the separate
// combine computes it.
__device__ __forceinline__ float mul_add_unfused(float acc, float w, float y) {
#pragma clang fp contract(off)
  return acc + w * y;
}

// The layer's combine fused after the down projection's stores (the
// "last workgroup" pattern): every workgroup makes its output rows visible
// device-wide (__threadfence), then counts, for each of its rows, one arrival
// of that row's token at this column tile.  The workgroup whose arrival
// completes a token's count (the number of its pairs the permutation kept)
// sums the token's pair rows over this column tile, j ascending, in fp32, as
// nvq_moe_combine does on the same bf16 rows: the result does not depend on
// which workgroup is last.  lds: the kernel's LDS tiles, free by now.
__device__ __forceinline__ void fused_combine(const GemmParams& p, const TileCtx& c, uint8_t* lds) {
  const int t = threadIdx.x;
  int32_t* s_list = reinterpret_cast<int32_t*>(lds);      // tokens completed here (<= BM)
  int32_t* s_n = reinterpret_cast<int32_t*>(lds + 4 * BM);
  __threadfence();  // this thread's output rows are visible to every workgroup
  __syncthreads();  // ... and every thread of this workgroup is past its stores
  if (t == 0) *s_n = 0;
  __syncthreads();
  const int topk = p.comb_topk;
  if (t < BM && c.row0 + t < c.row_end) {
    const int64_t tok = p.comb_pair[c.row0 + t] / topk;
    int nvalid = 0;
    for (int j = 0; j < topk; ++j) nvalid += p.comb_pos[tok * topk + j] >= 0 ? 1 : 0;
    const uint32_t before = atomicAdd(&p.comb_cnt[tok * p.n_tiles_n + c.nt], 1u);
    if (before + 1u == (uint32_t)nvalid) s_list[atomicAdd(s_n, 1)] = (int32_t)tok;
  }
  __syncthreads();
  const int nlast = *s_n;
  if (nlast == 0) return;
  __threadfence();  // the other workgroups' rows of these tokens are visible here
  const int64_t N = p.N;
  constexpr int kVecs = BN / 8;  // 8-column pieces of a column tile
  for (int idx = t; idx < nlast * kVecs; idx += NTHR) {
    const int64_t tok = s_list[idx / kVecs];
    const int64_t col = (int64_t)c.nt * BN + 8 * (idx % kVecs);
    if (col >= N) continue;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < topk; ++j) {
      const int32_t pj = p.comb_pos[tok * topk + j];
      if (pj < 0) continue;
      const float wj = p.comb_w[tok * topk + j];
      const uint4 q = *reinterpret_cast<const uint4*>(p.out_bf16 + (int64_t)pj * N + col);
      const uint32_t q4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int h2 = 0; h2 < 4; ++h2) {
        acc[2 * h2] = mul_add_unfused(acc[2 * h2], wj, bf16_lo(q4[h2]));
        acc[2 * h2 + 1] = mul_add_unfused(acc[2 * h2 + 1], wj, bf16_hi(q4[h2]));
      }
    }
    uint4 o;
    o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(p.comb_out + tok * N + col) = o;
  }
}

// Scale by s_tW and store.  acc[i][j][v]: row 32i + 8(v/4) + 4h + v%4, local
// column 64 wave + 32 j + l32; with SwiGLU fragment 0 is the gate and
// fragment 1 the up column of the same output column.  lds: the kernel's
// LDS tiles, no longer read (a 16 KB region per wave for the bf16 stores).
template <int kSwiglu>
__device__ __forceinline__ void epilogue(const GemmParams& p, const TileCtx& c,
                                         const floatx16_t (&acc)[4][2], uint8_t* lds) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, l32 = lane & 31, h = lane >> 5;
  const int64_t N = p.N;
  const float stw = p.w_st[c.e];
  // Tiles wholly inside the output take the unguarded store path: per-element
  // guards become exec-mask branches whose waits serialize the stores.
  const bool rows_full = c.row0 + BM <= c.row_end;
  if (!kSwiglu) {
    const bool cols_full = (int64_t)c.nt * BN + WN * (wave + 1) <= N;
    // bf16 through LDS when the wave's 64 columns are inside the output
    const bool bf16_lds = p.out_bf16 && p.bf16_rows16 && cols_full;
    auto emit = [&](bool check, bool f32, bool bf16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t pr = c.row0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          if (check && pr >= c.row_end) continue;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int64_t n = (int64_t)c.nt * BN + WN * wave + 32 * j + l32;
            if (check && n >= N) continue;
            const float y = acc[i][j][v] * stw;
            if (f32) p.out_f32[pr * N + n] = y;
            if (bf16) p.out_bf16[pr * N + n] = (uint16_t)f32_to_bf16_rne(y);
          }
        }
    };
    const bool f32 = p.out_f32 != nullptr, bf16_direct = p.out_bf16 && !bf16_lds;
    if (f32 || bf16_direct) {
      if (rows_full && cols_full)
        emit(false, f32, bf16_direct);
      else
        emit(true, f32, bf16_direct);
    }
    if (bf16_lds)
      store_tile_bf16_lds(acc, stw, lds + 16384 * wave, p.out_bf16 + c.row0 * N + (int64_t)c.nt * BN + WN * wave,
                          N, (int)min<int64_t>(BM, c.row_end - c.row0));
    if (p.comb_out) fused_combine(p, c, lds);
  } else {
    const int64_t I = N >> 1;
    const int64_t ng0 = (int64_t)c.nt * (BN / 2);  // first h column of the tile
    const int64_t ng = ng0 + 32 * wave + l32;
    uint32_t hmax = 0;  // largest |h| stored by this lane, as bf16 bits
    // A tile whose 128 h columns lie inside H stages them in LDS (128 rows x
    // 256 bytes; 16-byte chunk q of row r at slot q ^ 4 s, s = (r & 1) | ((r
    // >> 2) & 1) << 1, so the four rows one write instruction touches fill
    // distinct banks) and stores 16-byte pieces, 16 lanes per row, instead of
    // one 2-byte store per element.
    const bool h_lds = p.out_bf16 && p.h_rows16 && ng0 + BN / 2 <= I;
    auto swz = [](int r) { return 4 * ((r & 1) | (((r >> 2) & 1) << 1)); };
    auto emit = [&](bool check, bool to_lds) {
      const bool odd = (l32 & 1) != 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          uint32_t hb2[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int64_t pr = c.row0 + 32 * i + 8 * (v >> 2) + 4 * h + ((v + s) & 3);
            const bool live = !check || (pr < c.row_end && ng < I);
            const float g = acc[i][0][v + s] * stw;
            const float u = acc[i][1][v + s] * stw;
            if (p.out_f32 && live) {
              p.out_f32[pr * N + ng] = g;
              p.out_f32[pr * N + I + ng] = u;
            }
            // silu(g) u; the result is rounded to bf16, so an rcp suffices
            const float hv = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
            const uint32_t hb = f32_to_bf16_rne(hv);
            if (live) {
              if (p.out_bf16 && !to_lds) p.out_bf16[pr * I + ng] = (uint16_t)hb;
              hmax = max(hmax, hb & 0x7FFFu);
            }
            hb2[s] = hb;
          }
          if (to_lds) {
            // rows r, r + 1 of column l32: the even lane keeps row r and sends
            // row r + 1 to its odd neighbour, which keeps row r + 1
            const uint32_t send = odd ? hb2[0] : hb2[1];
            const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);
            const uint32_t lo = odd ? recv : hb2[0], hi = odd ? hb2[1] : recv;
            const int row = 32 * i + 8 * (v >> 2) + 4 * h + (v & 3) + (odd ? 1 : 0);
            const int col = 32 * wave + l32 - (odd ? 1 : 0);  // even column of the pair
            *reinterpret_cast<uint32_t*>(lds + row * 256 + (((col >> 3) ^ swz(row)) << 4) + (col & 7) * 2) =
                lo | (hi << 16);
          }
        }
    };
    if (h_lds) {
      emit(!rows_full, true);
      __syncthreads();  // the tile's h is in LDS
      const int nrows = (int)min<int64_t>(BM, c.row_end - c.row0), q = t & 15;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int row = (t >> 4) + 16 * m;
        if (row < nrows)
          *reinterpret_cast<uint4*>(p.out_bf16 + (c.row0 + row) * I + ng0 + 8 * q) =
              *reinterpret_cast<const uint4*>(lds + row * 256 + ((q ^ swz(row)) << 4));
      }
    } else if (rows_full && ng0 + 32 * (wave + 1) <= I) {
      emit(false, false);
    } else {
      emit(true, false);
    }
    // amax of H for its quantization: bit patterns of non-negative values
    // order as the values; one device-scope atomic per wave.
    if (p.h_amax) {
      const uint32_t m = wave_max_u32(hmax);
      if (lane == 0 && m != 0u) atomicMax(p.h_amax, m << 16);
    }
  }
}

// Per-thread register stage of one 128-element K step: this thread's A half
// row (32 code bytes, 4 scale bytes) and, for each of its two B fragments,
// the lane half (32 + 4 bytes) or, for path FP8_BLOCK, one code dword of
// each of the 8 blocks (the lane half's 8 elements of the block) and the
// 8 scale bytes.
template <bool kFp8>
struct Stage {
  uint4 a[2];
  uint32_t as;
  uint4 b[2][2];
  uint32_t bs[2][kFp8 ? 2 : 1];
};

// ------------------------------------------------------------ path DEQ16 --
template <int kSwiglu>
__global__ __launch_bounds__(NTHR, 2) void k_moe_gemm_deq16(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM][LROW];
  __shared__ int64_t s_tok[BM];  // A source row of each tile row (compensation prefetch)
  const TileCtx c = tile_of_block(p);
  if (!c.valid) return;
  const int64_t K = p.K, N = p.N;
  const int64_t Kh = K >> 1, Kb = K >> 4;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int l32 = lane & 31, h = lane >> 5;

  // A loader: row ar = t / 2, lane half ahh = t % 2 (elements [64 ahh, 64 ahh
  // + 64) of each step).  B: fragment j = local row 64 wave + 32 j + l32, lane
  // half h.
  const int ar = t >> 1, ahh = t & 1;
  const int64_t a_tok = loader_a_token(p, c, ar);
  if (ahh == 0) s_tok[ar] = a_tok;  // read after the prologue's barrier
  const uint8_t* a_src = p.a_codes + a_tok * Kh + 32 * ahh;
  const uint8_t* a_ssrc = p.a_scales + a_tok * Kb + 4 * ahh;
  const uint8_t* b_src[2];
  const uint8_t* b_ssrc[2];
  int64_t b_n[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    b_n[j] = loader_b_row<kSwiglu>(p, c, wave, j, l32);
    b_src[j] = p.w_codes + ((int64_t)c.e * N + b_n[j]) * Kh + 32 * h;
    b_ssrc[j] = p.w_scales + ((int64_t)c.e * N + b_n[j]) * Kb + 4 * h;
  }
  const int nst = (int)(K / SE);
  auto gload = [&](Stage<false>& S, int step) {
    const int64_t sc = min(step, nst - 1);  // past the end: a valid step, zero-scaled later
    S.a[0] = *reinterpret_cast<const uint4*>(a_src + sc * 64);
    S.a[1] = *reinterpret_cast<const uint4*>(a_src + sc * 64 + 16);
    S.as = *reinterpret_cast<const uint32_t*>(a_ssrc + sc * 8);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S.b[j][0] = *reinterpret_cast<const uint4*>(b_src[j] + sc * 64);
      S.b[j][1] = *reinterpret_cast<const uint4*>(b_src[j] + sc * 64 + 16);
      S.bs[j][0] = *reinterpret_cast<const uint32_t*>(b_ssrc[j] + sc * 8);
    }
  };
  // This thread's 64 A elements of a step -> exact fp16 at LDS row ar, bytes
  // [128 ahh, 128 ahh + 128), 16-byte chunk d at slot d ^ 4 ahh: the two
  // halves of a row, stored by adjacent lanes, then fall in different banks
  // (their natural offsets differ by 128 bytes, one full turn of the 32
  // banks that a 16-byte store is served from).  live == false (a step past
  // K) writes zeros.
  auto a_store = [&](const Stage<false>& S, int buf, bool live) {
    uint8_t* dst = &lds[buf][ar][128 * ahh];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t pat = live ? scale_pair(S.as, d >> 1) : 0u;
      *reinterpret_cast<half8_t*>(dst + 16 * (d ^ (4 * ahh))) = dequant8(dword_of(S.a, d), pat);
    }
  };

  floatx16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // one step: 8 sub-steps; A fragments from LDS (rows 32 i + l32, chunk d of
  // half h), B fragments dequantized from registers (dword d).  Only
  // the first NI 32-row sub-tiles take part.
  auto mfma_step = [&](auto ni_c, const Stage<false>& S, int buf) {
    constexpr int NI = decltype(ni_c)::value;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      half8_t af[NI], bf[2];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(&lds[buf][32 * i + l32][128 * h + 16 * (d ^ (4 * h))]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = dequant8(dword_of(S.b[j], d), scale_pair(S.bs[j][0], d >> 1));
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Pipeline: while the waves run the MFMAs of step s from LDS buffer s & 1,
  // step s + 1 (in registers) is dequantized into the other buffer; each
  // register stage is loaded right after the barrier that frees it, about
  // one step before its A half is stored and its MFMAs run.  The
  // scheduling barriers pin the loads there: left to itself the compiler
  // sinks them into the next MFMA sequence (it reuses their registers as
  // dequantization temporaries first), and the A half then arrives late.
  // The loop covers step pairs; an odd step count adds one zero-scaled step.
  // The last pair is peeled: instead of loading past the end it fetches the
  // compensation operands, which then arrive under its last MFMAs.
  // NI = 1 serves a tile of at most 32 rows (an expert's ragged last tile):
  // a quarter of the MFMAs, and only wave 0 (A rows 0..31) dequantizes A;
  // the other rows' accumulators stay unused and are never stored.
  CompPre<kSwiglu ? 3 : 4> pre;
  auto run = [&](auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;
    const bool a_live = NI == 4 || wave < NI;  // this wave's A rows are 32 wave .. + 31
    Stage<false> X0, X1;
    gload(X0, 0);
    gload(X1, 1);
    if (a_live) a_store(X0, 0, true);
    __syncthreads();
    int st = 0;
    for (; st + 2 < nst; st += 2) {
      mfma_step(ni_c, X0, 0);
      if (a_live) a_store(X1, 1, st + 1 < nst);
      __syncthreads();
      gload(X0, st + 2);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(ni_c, X1, 1);
      if (a_live) a_store(X0, 0, st + 2 < nst);
      __syncthreads();
      gload(X1, st + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_step(ni_c, X0, 0);
    if (a_live) a_store(X1, 1, st + 1 < nst);
    __syncthreads();  // buffer 0 is free from here on
    if (p.k > 0) comp_prefetch(p, (uint32_t)(uintptr_t)(NVQ_LDS_U8*)&lds[0][0][0], s_tok, c, b_n, pre);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(ni_c, X1, 1);
    // past this barrier buffer 1 is free (the epilogue's LDS staging spans
    // both) and every wave's compensation prefetch has landed
    if (p.k > 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (kSwiglu != 0) {
      comp_phase<true, 3, NI>(p, c, acc, lds[0], a_tok, b_n, pre);
      epilogue<kSwiglu>(p, c, acc, &lds[0][0][0]);
    }
  };
  if (c.row_end - c.row0 <= 32)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 4>{});
  if constexpr (kSwiglu == 0) {
    comp_phase<true>(p, c, acc, lds[0], a_tok, b_n, pre);
    epilogue<kSwiglu>(p, c, acc, &lds[0][0][0]);
  }
}

// ------------------------------------------------ path DEQ16, wide tile --
// For experts with many rows: workgroup = 8 waves (two per SIMD) over a
// 256-row x 256-column tile; wave w owns rows 128 (w / 4) .. + 128 and
// columns 64 (w % 4) .. + 64 (4 x 2 MFMA tiles, 128 accumulator registers,
// as in the 128-row kernel).  K advances 64 elements per step.  Both operands
// are dequantized once per workgroup into a double-buffered fp16 LDS tile:
// thread t dequantizes half of A row t / 2 and half of B row t / 2 (one code
// uint4 and two scale bytes each), so every weight element is dequantized
// once per 256 rows, where the 128-row kernel dequantizes it once per wave
// of 128 rows.  The raw FP4 stages are loaded two steps ahead; one barrier
// per step.  LDS rows are 144 bytes (64 fp16 + 16 pad).  The compensation
// runs as bf16 steps of 64 channels through the same tiles after the
// tensor-scale multiply, as in the 128-row kernel.
constexpr int W_THR = 512;
constexpr int W_BM = 256;
constexpr int W_SE = 64;
constexpr int W_PITCH = 144;
constexpr int kGroupMW = 4;  // 256-row tiles per group of the XCD-aware order

struct WStage {
  uint4 a;
  uint32_t as;  // two scale bytes in the low half
  uint4 b;
  uint32_t bs;
};

template <int kSwiglu>
__global__ __launch_bounds__(W_THR, 1) void k_moe_gemm_deq16w(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][W_BM][W_PITCH];  // [buf][A, B][row][byte]
  const TileCtx c = tile_of_block<kGroupMW>(p);
  if (!c.valid) return;
  const int64_t K = p.K, N = p.N;
  const int64_t Kh = K >> 1, Kb = K >> 4;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int wr = wave >> 2, wc = wave & 3;  // wave's 128-row half and 64-column quarter

  // loader: row lr = t / 2 of A and of B, half hf = t % 2 of each step
  // (elements 32 hf .. 32 hf + 31); rows past the ends are clamped (loaded,
  // never stored)
  const int lr = t >> 1, hf = t & 1;
  const int64_t a_tok = a_source_row(p, min<int64_t>(c.row0 + lr, c.row_end - 1));
  const uint8_t* a_src = p.a_codes + a_tok * Kh + 16 * hf;
  const uint8_t* a_ssrc = p.a_scales + a_tok * Kb + 2 * hf;
  const int64_t bn = min<int64_t>(b_row_to_n(lr, c.nt, kSwiglu, N), N - 1);
  const uint8_t* b_src = p.w_codes + ((int64_t)c.e * N + bn) * Kh + 16 * hf;
  const uint8_t* b_ssrc = p.w_scales + ((int64_t)c.e * N + bn) * Kb + 2 * hf;
  const int nst = (int)(K / W_SE);  // even: K % 128 == 0

  auto gload = [&](WStage& S, int step) {
    const int64_t sc = min(step, nst - 1);  // past the end: a valid step, zero-scaled later
    S.a = *reinterpret_cast<const uint4*>(a_src + sc * 32);
    S.as = *reinterpret_cast<const uint16_t*>(a_ssrc + sc * 4);
    S.b = *reinterpret_cast<const uint4*>(b_src + sc * 32);
    S.bs = *reinterpret_cast<const uint16_t*>(b_ssrc + sc * 4);
  };
  auto dw = [](const uint4& v, int d) { return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w; };
  // this thread's halves of A and B rows lr -> exact fp16 in buffer buf;
  // live == false (a step past K) writes zeros
  auto stage_store = [&](const WStage& S, int buf, bool live) {
    uint8_t* da = &lds[buf][0][lr][64 * hf];
    uint8_t* db = &lds[buf][1][lr][64 * hf];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t pa = live ? scale_pair(S.as, d >> 1) : 0u;
      const uint32_t pb = live ? scale_pair(S.bs, d >> 1) : 0u;
      *reinterpret_cast<half8_t*>(da + 16 * d) = dequant8(dw(S.a, d), pa);
      *reinterpret_cast<half8_t*>(db + 16 * d) = dequant8(dw(S.b, d), pb);
    }
  };

  floatx16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // one step: 4 sub-steps of 16 elements; lane half h takes elements
  // 16 d + 8 h .. + 7 of A rows 128 wr + 32 i + l32 and B rows
  // 64 wc + 32 j + l32
  auto mfma_step = [&](int buf) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      half8_t af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(&lds[buf][0][128 * wr + 32 * i + l32][32 * d + 16 * h]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(&lds[buf][1][64 * wc + 32 * j + l32][32 * d + 16 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  WStage R0, R1;
  gload(R0, 0);
  gload(R1, 1);
  stage_store(R0, 0, true);
  gload(R0, 2);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    stage_store(R1, 1, st + 1 < nst);
    gload(R1, st + 3);
    mfma_step(0);
    __syncthreads();
    stage_store(R0, 0, st + 2 < nst);
    gload(R0, st + 4);
    mfma_step(1);
    __syncthreads();
  }

  // acc *= s_tA, then the compensation: bf16 steps of 64 channels, the
  // residual rows (A side) and packed weight columns (B side) copied into
  // buffer 0 (thread: channels 32 hf .. + 31 of row lr); channels past k
  // read as zero
  const float sta = *p.a_st;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] *= sta;
  if (p.k > 0) {
    auto keep = [](bool live, uint4 v) {
      const uint32_t m = live ? 0xFFFFFFFFu : 0u;
      return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
    };
    const uint16_t* r_row = p.a_resid + a_tok * p.k;
    const uint16_t* w_row = p.wcomp + ((int64_t)c.e * N + bn) * p.kpad;
    for (int kc = 0; kc < p.k; kc += W_SE) {
      const int rem = p.k - kc;  // channels left, uniform
      uint4 ra[4], wb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = 32 * hf + 8 * q;
        ra[q] = *reinterpret_cast<const uint4*>(r_row + min(kc + ch, p.k - 8));
        wb[q] = *reinterpret_cast<const uint4*>(w_row + min(kc + ch, p.kpad - 8));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = 32 * hf + 8 * q;
        *reinterpret_cast<uint4*>(&lds[0][0][lr][2 * ch]) = keep(ch < rem, ra[q]);
        *reinterpret_cast<uint4*>(&lds[0][1][lr][2 * ch]) = keep(ch < rem, wb[q]);
      }
      __syncthreads();
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if (16 * d >= rem) break;
        bf16x8_t af[4], bf[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(&lds[0][0][128 * wr + 32 * i + l32][32 * d + 16 * h]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bf[j] = *reinterpret_cast<const bf16x8_t*>(&lds[0][1][64 * wc + 32 * j + l32][32 * d + 16 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
    }
  }

  // epilogue: scale by s_tW and store.  acc[i][j][v]: row 128 wr + 32 i +
  // 8 (v / 4) + 4 h + v % 4, B row 64 wc + 32 j + l32 (with SwiGLU j = 0 is
  // the gate and j = 1 the up row of output column 32 wc + l32).
  const float stw = p.w_st[c.e];
  const int64_t rbase = c.row0 + 128 * wr;
  const bool rows_full = rbase + 128 <= c.row_end;
  if (!kSwiglu) {
    const int64_t nbase = (int64_t)c.nt * BN + WN * wc;
    auto emit = [&](bool check) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t pr = rbase + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          if (check && pr >= c.row_end) continue;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int64_t n = nbase + 32 * j + l32;
            if (check && n >= N) continue;
            const float y = acc[i][j][v] * stw;
            if (p.out_f32) p.out_f32[pr * N + n] = y;
            if (p.out_bf16) p.out_bf16[pr * N + n] = (uint16_t)f32_to_bf16_rne(y);
          }
        }
    };
    if (rows_full && nbase + WN <= N)
      emit(false);
    else
      emit(true);
  } else {
    const int64_t I = N >> 1;
    const int64_t ng = (int64_t)c.nt * (BN / 2) + 32 * wc + l32;
    uint32_t hmax = 0;  // largest |h| stored by this lane, as bf16 bits
    auto emit = [&](bool check) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t pr = rbase + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          if (check && (pr >= c.row_end || ng >= I)) continue;
          const float g = acc[i][0][v] * stw;
          const float u = acc[i][1][v] * stw;
          if (p.out_f32) {
            p.out_f32[pr * N + ng] = g;
            p.out_f32[pr * N + I + ng] = u;
          }
          // silu(g) u; the result is rounded to bf16, so an rcp suffices
          const float hv = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          const uint32_t hb = f32_to_bf16_rne(hv);
          if (p.out_bf16) p.out_bf16[pr * I + ng] = (uint16_t)hb;
          hmax = max(hmax, hb & 0x7FFFu);
        }
    };
    if (rows_full && (int64_t)c.nt * (BN / 2) + 32 * (wc + 1) <= I)
      emit(false);
    else
      emit(true);
    if (p.h_amax) {
      const uint32_t m = wave_max_u32(hmax);
      if (lane == 0 && m != 0u) atomicMax(p.h_amax, m << 16);
    }
  }
}

// -------------------------------------------------------- path FP8_BLOCK --
// E2M1 magnitude index -> FP8 E4M3 byte (0, 0.5, 1, 1.5, 2, 3, 4, 6), as two
// byte-select tables for v_perm.
constexpr uint32_t kFp8TabLo = 0x3C383000u;  // indices 0..3
constexpr uint32_t kFp8TabHi = 0x4C484440u;  // indices 4..7

// The 4 even (sel_odd = false) or odd nibbles of a code dword -> 4 FP8 bytes.
__device__ __forceinline__ uint32_t fp4_to_fp8_4(uint32_t w, bool sel_odd) {
  const uint32_t nib = sel_odd ? (w >> 4) : w;
  const uint32_t mag = __builtin_amdgcn_perm(kFp8TabHi, kFp8TabLo, nib & 0x07070707u);
  return mag | ((nib & 0x08080808u) << 4);
}

// Path FP8_BLOCK: per 16-element block, one v_mfma_f32_32x32x16_fp8_fp8 of
// the raw E2M1 magnitudes (exact in FP8 E4M3) into a zero accumulator gives
// the exact block dot products; the fp32 accumulator then adds them times
// s_bA s_bW.  Within block b, lane half h takes elements 8h .. 8h + 7 (even
// ones first, then odd), for A and B alike.  The A tile goes through LDS as FP8 with an
// fp32 table of its block scales; B stays in registers as in path DEQ16.
template <int kSwiglu>
__global__ __launch_bounds__(NTHR, 1) void k_moe_gemm_fp8blk(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM][LROW];  // FP8 tile uses 128 bytes a row
  __shared__ __attribute__((aligned(16))) float s_as[2][8][BM];       // A block scales [block][row]
  const TileCtx c = tile_of_block(p);
  if (!c.valid) return;
  const int64_t K = p.K, N = p.N;
  const int64_t Kh = K >> 1, Kb = K >> 4;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int ar = t >> 1, ahh = t & 1;
  const int64_t a_tok = loader_a_token(p, c, ar);
  const uint8_t* a_src = p.a_codes + a_tok * Kh + 32 * ahh;
  const uint8_t* a_ssrc = p.a_scales + a_tok * Kb + 4 * ahh;
  const uint8_t* b_src[2];
  const uint8_t* b_ssrc[2];
  int64_t b_n[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    b_n[j] = loader_b_row<kSwiglu>(p, c, wave, j, l32);
    b_src[j] = p.w_codes + ((int64_t)c.e * N + b_n[j]) * Kh;
    b_ssrc[j] = p.w_scales + ((int64_t)c.e * N + b_n[j]) * Kb;
  }
  const int nst = (int)(K / SE);
  auto gload = [&](Stage<true>& S, int step) {
    const int64_t sc = min(step, nst - 1);
    S.a[0] = *reinterpret_cast<const uint4*>(a_src + sc * 64);
    S.a[1] = *reinterpret_cast<const uint4*>(a_src + sc * 64 + 16);
    S.as = *reinterpret_cast<const uint32_t*>(a_ssrc + sc * 8);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t d[8];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        d[bb] = *reinterpret_cast<const uint32_t*>(b_src[j] + sc * 64 + 8 * bb + 4 * h);
      S.b[j][0] = make_uint4(d[0], d[1], d[2], d[3]);
      S.b[j][1] = make_uint4(d[4], d[5], d[6], d[7]);
      const uint2 sv = *reinterpret_cast<const uint2*>(b_ssrc[j] + sc * 8);
      S.bs[j][0] = sv.x;
      S.bs[j][1] = sv.y;
    }
  };
  // A blocks 4 ahh .. 4 ahh + 3 of a step -> FP8 at LDS row ar, bytes
  // [16 b, 16 b + 16): for each lane half h, the 8 elements 16 b + 8 h ..
  // as (even, odd) nibbles; and the block scales in fp32.
  auto a_store = [&](const Stage<true>& S, int buf, bool live) {
    const uint32_t w[8] = {S.a[0].x, S.a[0].y, S.a[0].z, S.a[0].w, S.a[1].x, S.a[1].y, S.a[1].z, S.a[1].w};
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int b = 4 * ahh + bb;
      uint4 o;
      o.x = fp4_to_fp8_4(w[2 * bb], false);
      o.y = fp4_to_fp8_4(w[2 * bb], true);
      o.z = fp4_to_fp8_4(w[2 * bb + 1], false);
      o.w = fp4_to_fp8_4(w[2 * bb + 1], true);
      *reinterpret_cast<uint4*>(&lds[buf][ar][16 * b]) = o;
      s_as[buf][b][ar] = live ? e4m3_to_f32((S.as >> (8 * bb)) & 0xFFu) : 0.0f;
    }
  };

  floatx16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto mfma_step = [&](const Stage<true>& S, int buf) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      int64_t af[4], bf[2];
      float sw[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const int64_t*>(&lds[buf][32 * i + l32][16 * b + 8 * h]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = dword_of(S.b[j], b);  // this lane half's 8 elements of block b
        const uint32_t lo = fp4_to_fp8_4(w, false), hi = fp4_to_fp8_4(w, true);
        bf[j] = (int64_t)(((uint64_t)hi << 32) | lo);
        sw[j] = e4m3_to_f32((S.bs[j][b >> 2] >> (8 * (b & 3))) & 0xFFu);
      }
      // 8 (i, j) tiles, i-major; the MFMA of tile k + 1 is issued before
      // tile k's scaled accumulate, and scheduling barriers keep at most two
      // block products live.
      float4 sa[4];
      auto load_sa = [&](int i) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sa[r] = *reinterpret_cast<const float4*>(&s_as[buf][b][32 * i + 8 * r + 4 * h]);
      };
      // The zero accumulator of each block product passes through an empty
      // volatile asm after the previous tile's accumulate, so the compiler
      // cannot hoist all eight products (8 x 16 registers) to the top.
      auto block_mfma = [&](int k) {
        floatx16_t z;
#pragma unroll
        for (int v = 0; v < 16; ++v) z[v] = 0.0f;
        asm volatile("" : "+v"(z));
        return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(af[k >> 1], bf[k & 1], z, 0, 0, 0);
      };
      auto accumulate = [&](int k, const floatx16_t& P) {
        const int i = k >> 1, j = k & 1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float4& s4 = sa[v >> 2];
          const float sav = (v & 3) == 0 ? s4.x : (v & 3) == 1 ? s4.y : (v & 3) == 2 ? s4.z : s4.w;
          acc[i][j][v] = __builtin_fmaf(P[v], sav * sw[j], acc[i][j][v]);
        }
        asm volatile("" : "+v"(acc[i][j]));
      };
      load_sa(0);
      floatx16_t P0 = block_mfma(0), P1;
#define NVQ_FP8_TILE(K)                       \
  P1 = block_mfma(K);                         \
  accumulate((K) - 1, P0);                    \
  if (((K) & 1) == 0) load_sa((K) >> 1);      \
  __builtin_amdgcn_sched_barrier(0);          \
  P0 = P1;
      NVQ_FP8_TILE(1) NVQ_FP8_TILE(2) NVQ_FP8_TILE(3) NVQ_FP8_TILE(4)
      NVQ_FP8_TILE(5) NVQ_FP8_TILE(6) NVQ_FP8_TILE(7)
#undef NVQ_FP8_TILE
      accumulate(7, P0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Stage<true> X0, X1;
  gload(X0, 0);
  gload(X1, 1);
  a_store(X0, 0, true);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    mfma_step(X0, 0);
    a_store(X1, 1, st + 1 < nst);
    __syncthreads();
    gload(X0, st + 2);
    mfma_step(X1, 1);
    a_store(X0, 0, st + 2 < nst);
    __syncthreads();
    gload(X1, st + 3);
  }
  comp_phase<false>(p, c, acc, lds[0], a_tok, b_n, CompPre<1>{});
  epilogue<kSwiglu>(p, c, acc, &lds[0][0][0]);
}

struct MoeLayout {
  int max_tiles;
  int kpad;
  int32_t* tiles;
  int32_t* ntiles;
  uint16_t* wcomp;
  int64_t n_cnt;
  uint32_t* cnt;
  size_t bytes;
};

MoeLayout moe_layout(void* ws, int64_t rows, int64_t E, int64_t N, int64_t k, int64_t comb_T = 0) {
  MoeLayout L;
  L.max_tiles = (int)((rows + BM - 1) / BM + E);
  L.kpad = (int)((k + 15) / 16 * 16);
  WsCarve c(ws);
  L.tiles = c.take<int32_t>((size_t)L.max_tiles * 2);
  L.ntiles = c.take<int32_t>(1);
  L.wcomp = c.take<uint16_t>((size_t)(E * N * L.kpad));
  L.n_cnt = comb_T * ((N + BN - 1) / BN);
  L.cnt = L.n_cnt > 0 ? c.take<uint32_t>((size_t)L.n_cnt) : nullptr;
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

extern "C" size_t moe_gemm_workspace_bytes_comb(int64_t rows, int64_t E, int64_t N, int32_t k,
                                                int64_t T) {
  if (rows < 0 || E < 1 || N < 1 || k < 0 || T < 0) return kAlign;
  return moe_layout(nullptr, rows, E, N, k, T).bytes;
}

extern "C" int moe_grouped_gemm_w4a4_comp(const nvq_moe_gemm_args* a, void* stream) {
  if (!a || a->struct_size < offsetof(nvq_moe_gemm_args, w_codes_cm)) return NVQ_EINVAL;
  const bool has_cm = a->struct_size >= offsetof(nvq_moe_gemm_args, w_scales_cm) + sizeof(void*) &&
                      a->w_codes_cm && a->w_scales_cm;
  uint32_t* h_amax = a->struct_size >= offsetof(nvq_moe_gemm_args, h_amax) + sizeof(void*)
                         ? reinterpret_cast<uint32_t*>(a->h_amax)
                         : nullptr;
  if (h_amax && a->epilogue != NVQ_EPI_SWIGLU) return NVQ_EINVAL;
  if (h_amax && ((uintptr_t)h_amax & 3u)) return NVQ_EALIGN;
  if (!a->expert_offsets || !a->w_codes || !a->w_scales || !a->w_tensor_scale || !a->ws) return NVQ_EINVAL;
  // the row buffers may be NULL when there are no rows
  if (a->rows != 0 && (!a->a_codes || !a->a_scales || !a->a_tensor_scale)) return NVQ_EINVAL;
  if (a->rows != 0 && !a->out_bf16 && !a->out_f32) return NVQ_EINVAL;
  if (a->epilogue != NVQ_EPI_NONE && a->epilogue != NVQ_EPI_SWIGLU) return NVQ_EINVAL;
  if (a->path != NVQ_GEMM_AUTO && a->path != NVQ_GEMM_DEQ16 && a->path != NVQ_GEMM_FP8_BLOCK &&
      a->path != NVQ_GEMM_DEQ16_WIDE)
    return NVQ_EINVAL;
  if (a->rows < 0 || a->E < 1 || a->E > 1024 || a->N <= 0 || a->K <= 0) return NVQ_ESHAPE;
  if (a->K % 128 != 0) return NVQ_ESHAPE;  // K steps of 32 elements; 128 keeps rows 64-byte aligned
  if (a->epilogue == NVQ_EPI_SWIGLU && (a->N % 2 != 0)) return NVQ_ESHAPE;
  if (a->k < 0 || a->k > a->K || (a->k & 7)) return NVQ_ESHAPE;
  if (a->rows != 0 && a->k > 0 && (!a->a_resid || !a->comp_idx)) return NVQ_EINVAL;
  if (a->a_row_div < 0) return NVQ_EINVAL;
  if (((uintptr_t)a->a_codes & 15u) || ((uintptr_t)a->w_codes & 15u) ||
      (a->k > 0 && ((uintptr_t)a->a_resid & 15u)) ||
      ((uintptr_t)a->a_scales & 7u) || ((uintptr_t)a->w_scales & 7u))
    return NVQ_EALIGN;
  if (!aligned256(a->ws)) return NVQ_EALIGN;
  const bool has_comb_fields = a->struct_size >= offsetof(nvq_moe_gemm_args, comb_out) + sizeof(void*);
  const bool comb = has_comb_fields && a->comb_out;
  if (comb) {
    if (a->epilogue != NVQ_EPI_NONE || a->path == NVQ_GEMM_DEQ16_WIDE || !a->out_bf16) return NVQ_EINVAL;
    if (!a->comb_pos || !a->comb_weights || (a->rows != 0 && !a->comb_pair)) return NVQ_EINVAL;
    if (a->comb_topk < 1 || a->comb_T < 0 || (a->N & 7)) return NVQ_ESHAPE;
    if (!aligned16(a->comb_out) || !aligned16(a->out_bf16)) return NVQ_EALIGN;
  }
  MoeLayout L = moe_layout(a->ws, a->rows, a->E, a->N, a->k, comb ? a->comb_T : 0);
  if (a->ws_bytes < L.bytes) return NVQ_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (comb && a->comb_T > 0) {  // counters start at zero (a kernel, not a memset: capture-safe)
    const int64_t nb = std::min<int64_t>((std::max(L.n_cnt, a->comb_T) + 255) / 256, 4096);
    hipLaunchKernelGGL(k_comb_prep, dim3((unsigned)nb), dim3(256), 0, s, L.cnt, L.n_cnt, a->comb_pos,
                       a->comb_T, (int)a->comb_topk, a->comb_out, a->N);
    if (int rc = last_launch()) return rc;
  }
  if (a->rows == 0) {
    if (!h_amax) return NVQ_OK;
    hipLaunchKernelGGL(k_clear_word, dim3(1), dim3(1), 0, s, h_amax);  // amax of no rows: 0
    return last_launch();
  }
  // Tile shape: 128-row tiles unless the 256-row kernel is asked for (it
  // measured slower on every layer here, also where experts average 2048
  // rows, so AUTO does not take it).
  const bool fp8 = a->path == NVQ_GEMM_FP8_BLOCK;
  const bool wide = a->path == NVQ_GEMM_DEQ16_WIDE;
  const int bm = wide ? W_BM : BM;
  const int max_tiles = wide ? (int)((a->rows + W_BM - 1) / W_BM + a->E) : L.max_tiles;
  const bool fused_table = a->k > 0 && has_cm;  // the gather's extra workgroup builds the table
  if (!fused_table) {
    hipLaunchKernelGGL(k_tile_table, dim3(1), dim3(1024), 0, s, a->expert_offsets, (int)a->E, bm, L.tiles,
                       L.ntiles, max_tiles, h_amax);
    if (int rc = last_launch()) return rc;
  }
  GemmParams p;
  p.rows = a->rows; p.K = a->K; p.N = a->N; p.E = a->E; p.a_rows = a->a_rows;
  p.a_row = a->a_row; p.a_row_div = a->a_row_div; p.off = a->expert_offsets;
  p.a_codes = a->a_codes; p.a_scales = a->a_scales; p.a_st = a->a_tensor_scale;
  p.a_resid = a->a_resid; p.comp_idx = a->comp_idx; p.k = a->k;
  p.kpad = L.kpad; p.wcomp = L.wcomp;
  if (fused_table) {
    hipLaunchKernelGGL(k_gather_wcomp_rows,
                       dim3((unsigned)((a->N + kWcRows - 1) / kWcRows), (unsigned)((L.kpad + kWcCh - 1) / kWcCh),
                            (unsigned)a->E + 1),
                       dim3(256), 0, s, a->w_codes_cm, a->w_scales_cm, a->N, a->K, a->comp_idx, (int)a->k, L.kpad,
                       L.wcomp, a->expert_offsets, (int)a->E, bm, L.tiles, L.ntiles, max_tiles, h_amax);
    if (int rc = last_launch()) return rc;
  } else if (a->k > 0) {
    const int64_t wrows = a->E * a->N;
    hipLaunchKernelGGL(k_gather_wcomp, dim3((unsigned)((wrows + 3) / 4)), dim3(256), 0, s, a->w_codes,
                       a->w_scales, wrows, a->K, a->comp_idx, (int)a->k, L.kpad, L.wcomp);
    if (int rc = last_launch()) return rc;
  }
  p.w_codes = a->w_codes; p.w_scales = a->w_scales; p.w_st = a->w_tensor_scale;
  p.out_bf16 = a->out_bf16; p.out_f32 = a->out_f32;
  p.bf16_rows16 = (a->N % 8 == 0 && aligned16(a->out_bf16)) ? 1 : 0;
  p.h_rows16 = (a->N % 16 == 0 && aligned16(a->out_bf16)) ? 1 : 0;
  p.comb_pair = comb ? a->comb_pair : nullptr;
  p.comb_pos = comb ? a->comb_pos : nullptr;
  p.comb_w = comb ? a->comb_weights : nullptr;
  p.comb_topk = comb ? a->comb_topk : 0;
  p.comb_out = comb ? a->comb_out : nullptr;
  p.comb_cnt = L.cnt;
  p.tiles = L.tiles; p.ntiles = L.ntiles; p.max_tiles = max_tiles;
  p.h_amax = h_amax;
  const bool swiglu = a->epilogue == NVQ_EPI_SWIGLU;
  p.swiglu = swiglu ? 1 : 0;
  p.bm = bm;
  p.n_tiles_n = swiglu ? (int)((a->N / 2 + BN / 2 - 1) / (BN / 2)) : (int)((a->N + BN - 1) / BN);
  const int gm = wide ? kGroupMW : kGroupM;
  const int n_groups = (max_tiles + gm - 1) / gm;
  const int64_t G0 = (int64_t)n_groups * gm * p.n_tiles_n;
  const int64_t G = (G0 + 7) / 8 * 8;
  if (G > 0x7FFFFFFF) return NVQ_ESHAPE;
  if (wide) {
    if (swiglu)
      hipLaunchKernelGGL(k_moe_gemm_deq16w<1>, dim3((unsigned)G), dim3(W_THR), 0, s, p);
    else
      hipLaunchKernelGGL(k_moe_gemm_deq16w<0>, dim3((unsigned)G), dim3(W_THR), 0, s, p);
  } else if (fp8) {
    if (swiglu)
      hipLaunchKernelGGL(k_moe_gemm_fp8blk<1>, dim3((unsigned)G), dim3(NTHR), 0, s, p);
    else
      hipLaunchKernelGGL(k_moe_gemm_fp8blk<0>, dim3((unsigned)G), dim3(NTHR), 0, s, p);
  } else {
    if (swiglu)
      hipLaunchKernelGGL(k_moe_gemm_deq16<1>, dim3((unsigned)G), dim3(NTHR), 0, s, p);
    else
      hipLaunchKernelGGL(k_moe_gemm_deq16<0>, dim3((unsigned)G), dim3(NTHR), 0, s, p);
  }
  return last_launch();
}

extern "C" int nvfp4_channel_major(const uint8_t* codes, const uint8_t* scales, int64_t batch, int64_t N,
                                   int64_t K, uint8_t* codes_cm, uint8_t* scales_cm, void* stream) {
  if (!codes || !scales || !codes_cm || !scales_cm) return NVQ_EINVAL;
  if (batch < 1 || N <= 0 || K <= 0 || (N % 16) || (K % 16)) return NVQ_ESHAPE;
  if (((uintptr_t)codes & 7u) || ((uintptr_t)codes_cm & 7u)) return NVQ_EALIGN;
  if (batch > 65535 || (N + 63) / 64 > 65535) return NVQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_codes_cm, dim3((unsigned)((K + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)batch),
                     dim3(256), 0, s, codes, N, K, codes_cm);
  if (int rc = last_launch()) return rc;
  const int64_t KB = K / 16;
  hipLaunchKernelGGL(k_scales_cm, dim3((unsigned)((KB + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)batch),
                     dim3(256), 0, s, scales, N, KB, scales_cm);
  return last_launch();
}

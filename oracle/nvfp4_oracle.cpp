// NVFP4 oracle -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
//
// A plain, slow, CPU-only reference of everything the NVFP4 hot path computes.
// Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
// may load this library.  It shares no code, header, table or helper with the
// HIP library: every constant below is written out here from the format and
// method definitions it cites.
//
// Sources (cited by page title and section; the pages carry no equations):
//  * QUADS explainer ("QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE
//    via QUantization-error Alignment across Dual Sides", gist.science, fr/es):
//      §1 Problem statement -- E2M1 grid, 8 magnitudes per sign.
//      §2.1 Error analysis  -- weights go through the same quantize/dequantize
//                              path on both sides; activations are quantized
//                              online and carry an error.
//      §2.2-A Asymmetric QAT -- trainer forward uses fake-quantized W4, A16.
//      §2.2-B Residual activation compensation -- channels with the largest
//                              quantization residual get a correction term added
//                              to the W4A4 output; a binary channel mask picks them.
//  * TRACE post ("TRACE : un entraînement conscient de la quantification guidé
//    par le rollout ...", sns.style), "Fonctionnement, côté ingénierie":
//      block scaling (a small group of values shares one scale, 4 bits each,
//      each value rounds to the grid point above or below); the trainer reuses
//      the rollout's recorded rounding.
//  * NVFP4 format details the pages leave open (public format definitions):
//      16-element blocks along K, one E4M3 scale per block, one FP32 scale per
//      tensor, E2M1 elements (OCP MX v1.0 FP4 E2M1), E4M3 "FN" scales (OCP FP8).
//
// Every reading taken where the pages are silent is listed in the repository's
// design notes; the ones that matter for the arithmetic are restated at each
// function.  Floating point is fp64 unless the definition fixes fp32; each
// place where fp64 is exact (not merely accurate) says why.
//
// Build:  g++ -O2 -std=c++17 -fPIC -shared -ffp-contract=off -pthread
// (no -ffast-math: the fp32 residual and score sums must be IEEE fp32, and
//  x86-64 evaluates float arithmetic in SSE single precision).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- formats ---

// E2M1 magnitudes indexed by the 3-bit field (e1 e0 m): exponent bias 1, one
// mantissa bit, index 0/1 subnormal (0, 0.5).  OCP MX v1.0, FP4 E2M1.
// QUADS explainer §1: 8 magnitudes per sign.
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

// E4M3 "FN" (OCP FP8): 4 exponent bits (bias 7), 3 mantissa bits, no
// infinities; 0x7F is NaN and is never produced.  Non-negative finite codes
// are 0x00..0x7E; 0x7E = 448 is the largest.
double e4m3_value(int code) {
  const int e = (code >> 3) & 0xF;
  const int m = code & 7;
  if (e == 0) return std::ldexp(m / 8.0, -6);      // subnormal: m/8 * 2^-6
  return std::ldexp(1.0 + m / 8.0, e - 7);         // normal: (1+m/8) * 2^(e-7)
}
const int kE4M3MaxCode = 0x7E;

// 6 * 448: the largest E2M1 magnitude times the largest E4M3 scale.
const double kTensorScaleDivisor = 2688.0;

float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round an fp32 value to bf16, round-to-nearest-even (finite inputs).
uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Round a real number held exactly in fp64 to bf16, round-to-nearest-even, in
// one step (no detour through fp32, which would round twice).  bf16 keeps 8
// significant bits over fp32's exponent range: normal values are multiples of
// 2^(e-7) in the binade [2^e, 2^(e+1)), e >= -126, and below 2^-126 the
// subnormal spacing is 2^-133.  The scaled value is rounded to an integer with
// ties to even (nearbyint in the default rounding mode), which is exact in
// fp64; a carry to the next binade gives the right value.  Magnitudes at or
// above the midpoint between the largest finite bf16 (2^127 * (2 - 2^-7)) and
// 2^128 round to infinity.  NaN maps to the canonical quiet NaN.
uint16_t double_to_bf16_rne(double v) {
  if (std::isnan(v)) return 0x7FC0u;
  const uint16_t sign = std::signbit(v) ? 0x8000u : 0u;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  const double kOverflow = std::ldexp(2.0 - std::ldexp(1.0, -8), 127);  // max + half ulp
  if (a >= kOverflow) return sign | 0x7F80u;
  int e2 = 0;
  std::frexp(a, &e2);           // a = f 2^e2, f in [0.5, 1): binade [2^(e2-1), 2^e2)
  int e = e2 - 1;               // a in [2^e, 2^(e+1))
  if (e < -126) e = -126;       // subnormal range: fixed spacing 2^-133
  const double q = std::nearbyint(std::ldexp(a, 7 - e));  // units of 2^(e-7)
  const float r = (float)std::ldexp(q, e - 7);  // exact: <= 8 significant bits in fp32 range
  uint32_t u;
  std::memcpy(&u, &r, 4);
  return (uint16_t)(sign | (u >> 16));
}

// Element (r, c) of a row-major [rows, ld] tensor of dtype 0 = f32, 1 = bf16,
// returned as float (bf16 -> f32 is exact).
float load_elem(const void* x, int dtype, int64_t r, int64_t ld, int64_t c) {
  if (dtype == 0) return static_cast<const float*>(x)[r * ld + c];
  return bf16_bits_to_float(static_cast<const uint16_t*>(x)[r * ld + c]);
}

int oracle_threads() {
  const char* s = std::getenv("ORACLE_THREADS");
  if (s && std::atoi(s) > 0) return std::atoi(s);
  unsigned n = std::thread::hardware_concurrency();
  return n ? (int)n : 1;
}

// Run fn(i) for i in [0, n) on the host cores.  Each i is independent, so
// the split changes no result.
template <class F>
void parallel_for(int64_t n, F fn) {
  int nt = oracle_threads();
  if (n < 2 || nt == 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  if (nt > n) nt = (int)n;
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([=] {
      for (int64_t i = t; i < n; i += nt) fn(i);
    });
  }
  for (auto& th : pool) th.join();
}

// ------------------------------------------------------------ quantizer ----

// Q3.  The E4M3 scale code nearest the real number amax_b / (6 s_t), ties to
// the even code, saturating at 448.  Exhaustive search over the 127 finite
// non-negative codes, minimising |amax_b - v * 6 * s_t| (the same argmin, as
// 6 s_t > 0).  v * 6 * s_t has at most 4 + 2 + 24 significant bits and is
// exact in fp64; the distances of the two codes that bracket the target are
// differences of numbers within a few binades of each other with <= 30 bits,
// hence exact, so ties and near-ties are decided exactly.
int e4m3_scale_code_search(double amax_b, double s_t) {
  int best = 0;
  double best_d = INFINITY;
  for (int v = 0; v <= kE4M3MaxCode; ++v) {
    const double d = std::fabs(amax_b - e4m3_value(v) * 6.0 * s_t);
    if (d < best_d || (d == best_d && (v & 1) == 0)) {
      best = v;
      best_d = d;
    }
  }
  return best;
}

// Q4.  The E2M1 magnitude index whose grid value G[i] * s_b * s_t is nearest
// |x|, ties to the even index (even mantissa bit).  Values beyond 6 s_b s_t
// land on index 7.  G[i] * s_b * s_t has <= 2 + 4 + 24 significant bits: exact.
int e2m1_index_search(double ax, double s_b, double s_t) {
  int best = 0;
  double best_d = INFINITY;
  for (int i = 0; i < 8; ++i) {
    const double d = std::fabs(ax - kE2M1[i] * s_b * s_t);
    if (d < best_d || (d == best_d && (i & 1) == 0)) {
      best = i;
      best_d = d;
    }
  }
  return best;
}

// Threshold form of Q3/Q4 (a second, independent formulation used only to
// cross-check the search form): the code is the number of decision midpoints
// that lie below the target, where a target exactly on a midpoint goes to the
// even neighbour.  Midpoints times the scale are exact in fp64 (<= 31 bits).
int e4m3_scale_code_thresholds(double amax_b, double s_t) {
  int code = 0;
  for (int v = 0; v < kE4M3MaxCode; ++v) {
    const double mid = 0.5 * (e4m3_value(v) + e4m3_value(v + 1)) * 6.0 * s_t;
    const bool upper_is_even = ((v + 1) & 1) == 0;
    if (amax_b > mid || (amax_b == mid && upper_is_even)) code = v + 1;
  }
  return code;
}

int e2m1_index_thresholds(double ax, double s_b, double s_t) {
  int idx = 0;
  for (int i = 0; i < 7; ++i) {
    const double mid = 0.5 * (kE2M1[i] + kE2M1[i + 1]) * s_b * s_t;
    const bool upper_is_even = ((i + 1) & 1) == 0;
    if (ax > mid || (ax == mid && upper_is_even)) idx = i + 1;
  }
  return idx;
}

// Shared driver for both forms.  Returns 0, or -3 on a non-finite input.
int quantize_impl(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                  const float* amax_in, uint8_t* codes, uint8_t* scales, float* s_t_out,
                  bool threshold_form) {
  if (K <= 0 || K % 16 != 0 || rows < 0) return -2;
  // Q1: amax_t = max |x| over the whole tensor (max is exact: order free).
  double amax = 0.0;
  bool finite = true;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < K; ++c) {
      const float v = load_elem(x, dtype, r, ldx, c);
      if (!std::isfinite(v)) finite = false;
      amax = std::max(amax, (double)std::fabs(v));
    }
  if (!finite) return -3;
  if (amax_in) amax = (double)*amax_in;
  // Q2: s_t = fl32(amax_t / 2688).  The quotient is formed in fp64 and
  // rounded once more to fp32; with 53 >= 2*24 + 2 bits this double rounding
  // equals the correctly rounded fp32 quotient.
  const float s_t = (float)(amax / kTensorScaleDivisor);
  *s_t_out = s_t;
  const double st = (double)s_t;
  const int64_t nb = K / 16;
  parallel_for(rows, [&](int64_t r) {
    for (int64_t b = 0; b < nb; ++b) {
      double amax_b = 0.0;
      for (int j = 0; j < 16; ++j)
        amax_b = std::max(amax_b, (double)std::fabs(load_elem(x, dtype, r, ldx, b * 16 + j)));
      // s_t == 0: every scale is 0 and every magnitude is 0.
      int sc = 0;
      if (st > 0.0)
        sc = threshold_form ? e4m3_scale_code_thresholds(amax_b, st)
                            : e4m3_scale_code_search(amax_b, st);
      scales[r * nb + b] = (uint8_t)sc;
      const double s_b = e4m3_value(sc);
      for (int j = 0; j < 16; j += 2) {
        uint8_t nib[2];
        for (int h = 0; h < 2; ++h) {
          const float v = load_elem(x, dtype, r, ldx, b * 16 + j + h);
          int idx = 0;
          if (sc != 0)
            idx = threshold_form ? e2m1_index_thresholds(std::fabs((double)v), s_b, st)
                                 : e2m1_index_search(std::fabs((double)v), s_b, st);
          nib[h] = (uint8_t)((std::signbit(v) ? 8 : 0) | idx);
        }
        // Q5: even element in the low nibble.
        codes[r * (K / 2) + (b * 16 + j) / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
      }
    }
  });
  return 0;
}

// D.  Dequantized value of one element: sign * fl32(fl32(G * s_b) * s_t).
// G * s_b has <= 6 significant bits and is exact in fp32; the product with s_t
// is formed exactly in fp64 (<= 30 bits) and rounded once to fp32.
float dequant_elem(const uint8_t* codes, const uint8_t* scales, float s_t, int64_t K,
                   int64_t r, int64_t c) {
  const uint8_t byte = codes[r * (K / 2) + c / 2];
  const int nib = (c & 1) ? (byte >> 4) : (byte & 0xF);
  const double s_b = e4m3_value(scales[r * (K / 16) + c / 16]);
  const float mag = (float)(kE2M1[nib & 7] * s_b * (double)s_t);
  return (nib & 8) ? -mag : mag;
}

// Exact real value G * s_b * s_t of one element (fp64, exact: <= 30 bits).
double dequant_exact(const uint8_t* codes, const uint8_t* scales, float s_t, int64_t K,
                     int64_t r, int64_t c) {
  const uint8_t byte = codes[r * (K / 2) + c / 2];
  const int nib = (c & 1) ? (byte >> 4) : (byte & 0xF);
  const double v = kE2M1[nib & 7] * e4m3_value(scales[r * (K / 16) + c / 16]) * (double)s_t;
  return (nib & 8) ? -v : v;
}

// bf16 value of the fp32 residual r = fl32(x - v) of one element, as double.
double residual_bf16(const void* x, int dtype, int64_t ldx, const uint8_t* codes,
                     const uint8_t* scales, float s_t, int64_t K, int64_t r, int64_t c) {
  const float xv = load_elem(x, dtype, r, ldx, c);
  const float v = dequant_elem(codes, scales, s_t, K, r, c);
  const float res = xv - v;
  return (double)bf16_bits_to_float(float_to_bf16_rne(res));
}

// ------------------------------------------------ rollout-guided rounding --
//
// TRACE post, "L'idée centrale de TRACE": the rollout's quantization result
// guides the trainer's rounding, and the cache keeps only the mantissa and the
// scale factors.  "Fonctionnement, côté ingénierie": for each value, rounding
// to the grid point above or below is the one discrete choice that the trainer
// must make the same way as the rollout.  Two one-bit-per-element records are
// defined (the second is the up/down reading of the same passage):
//   mantissa  (mode 0): the mantissa bit of the rollout's E2M1 code (index & 1);
//   direction (mode 1): 1 when the rollout's magnitude G[i] s_b s_t lies
//                       strictly above |x| (rounded up), else 0.
// The record also carries the rollout's block scales and tensor scale, which
// the trainer reuses unchanged.

// One record bit for element x whose rollout code has magnitude index i.
// G[i] * s_b * s_t is exact in fp64 (<= 2 + 4 + 24 significant bits), so the
// comparison with |x| is exact.
int guidance_bit(float x, int i, double s_b, double s_t, int mode) {
  if (mode == 0) return i & 1;
  return kE2M1[i] * s_b * s_t > std::fabs((double)x) ? 1 : 0;
}

// Magnitude index chosen for a (possibly drifted) master value w under the
// cached block scale s_b, tensor scale s_t and record bit.  On the scaled grid
// G[i] s_b s_t the value |w| has a lower neighbour lo (largest i with
// G[i] s_b s_t <= |w|) and an upper neighbour hi (smallest i with
// G[i] s_b s_t >= |w|; none beyond 6 s_b s_t).
//   mantissa:  the two adjacent grid points a = min(lo, 6) and a + 1 have
//              different mantissa bits; take the one whose bit is the cached
//              bit.
//   direction: bit 1 takes hi (7 beyond the grid), bit 0 takes lo.
// A block whose scale product is 0 has magnitude 0.  All products are exact
// in fp64, so every comparison is exact.
int guided_index(double aw, double s_b, double s_t, int mode, int bit) {
  if (s_b * s_t == 0.0) return 0;
  int lo = 0;
  for (int i = 0; i < 8; ++i)
    if (kE2M1[i] * s_b * s_t <= aw) lo = i;
  int hi = -1;
  for (int i = 7; i >= 0; --i)
    if (kE2M1[i] * s_b * s_t >= aw) hi = i;
  if (mode == 0) {
    const int a = std::min(lo, 6);
    return (a & 1) == bit ? a : a + 1;
  }
  if (bit) return hi < 0 ? 7 : hi;
  return lo;
}

}  // namespace

extern "C" {

// ------------------------------------------------------------- tables ------

double orc_e2m1_value(int idx) { return kE2M1[idx & 7]; }
double orc_e4m3_value(int code) { return e4m3_value(code); }
float orc_tensor_scale(float amax) { return (float)((double)amax / kTensorScaleDivisor); }
uint16_t orc_float_to_bf16(float f) { return float_to_bf16_rne(f); }
uint16_t orc_double_to_bf16(double v) { return double_to_bf16_rne(v); }
void orc_float_to_bf16_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16_rne(x[i]);
}
int orc_threads(void) { return oracle_threads(); }

// ---------------------------------------------------------- quantizer ------

// NVFP4-quantize a row-major [rows, K] tensor (dtype 0 = f32, 1 = bf16, row
// stride ldx elements) with one tensor scale:
//   codes  [rows, K/2]  two E2M1 codes per byte, even element in the low nibble
//   scales [rows, K/16] E4M3 codes
//   *s_t   fp32 tensor scale
// amax_in (nullable) replaces the computed amax_t.  Returns 0, -2 (shape),
// -3 (non-finite input).
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                 const float* amax_in, uint8_t* codes, uint8_t* scales, float* s_t) {
  return quantize_impl(x, dtype, rows, K, ldx, amax_in, codes, scales, s_t, false);
}

// The same, decided by the threshold form (cross-check only).
int orc_quantize_threshold_form(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                                const float* amax_in, uint8_t* codes, uint8_t* scales,
                                float* s_t) {
  return quantize_impl(x, dtype, rows, K, ldx, amax_in, codes, scales, s_t, true);
}

// Guidance record of a quantized [rows, K] tensor (one s_t): bits
// [rows, K/8], element c in bit (c & 7) of byte c / 8.  x (the value that was
// quantized) is read only in direction mode and may be NULL in mantissa mode.
// Returns 0, -2 (shape), -1 (mode or missing x).
int orc_guidance_record(const void* x, int dtype, int64_t rows, int64_t K, const uint8_t* codes,
                        const uint8_t* scales, float s_t, int mode, uint8_t* bits) {
  if (K <= 0 || K % 16 != 0 || rows < 0) return -2;
  if ((mode != 0 && mode != 1) || (mode == 1 && !x)) return -1;
  parallel_for(rows, [&](int64_t r) {
    for (int64_t c8 = 0; c8 < K / 8; ++c8) {
      uint8_t byte = 0;
      for (int j = 0; j < 8; ++j) {
        const int64_t c = c8 * 8 + j;
        const uint8_t cb = codes[r * (K / 2) + c / 2];
        const int i = ((c & 1) ? (cb >> 4) : cb) & 7;
        const double s_b = e4m3_value(scales[r * (K / 16) + c / 16]);
        const float xv = mode == 1 ? load_elem(x, dtype, r, K, c) : 0.0f;
        byte |= (uint8_t)(guidance_bit(xv, i, s_b, (double)s_t, mode) << j);
      }
      bits[r * (K / 8) + c8] = byte;
    }
  });
  return 0;
}

// Codes of a (possibly drifted) master tensor w [rows, K] rebuilt from the
// rollout's guidance record (bits, scales, s_t): sign from signbit(w),
// magnitude from guided_index.  Returns 0, -2 (shape), -1 (mode),
// -3 (non-finite w).
int orc_guided_quantize(const void* w, int dtype, int64_t rows, int64_t K, const uint8_t* bits,
                        const uint8_t* scales, float s_t, int mode, uint8_t* codes) {
  if (K <= 0 || K % 16 != 0 || rows < 0) return -2;
  if (mode != 0 && mode != 1) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < K; ++c)
      if (!std::isfinite(load_elem(w, dtype, r, K, c))) return -3;
  parallel_for(rows, [&](int64_t r) {
    for (int64_t c = 0; c < K; c += 2) {
      uint8_t nib[2];
      for (int h = 0; h < 2; ++h) {
        const float v = load_elem(w, dtype, r, K, c + h);
        const int bit = (bits[r * (K / 8) + (c + h) / 8] >> ((c + h) & 7)) & 1;
        const double s_b = e4m3_value(scales[r * (K / 16) + (c + h) / 16]);
        const int i = guided_index(std::fabs((double)v), s_b, (double)s_t, mode, bit);
        nib[h] = (uint8_t)((std::signbit(v) ? 8 : 0) | i);
      }
      codes[r * (K / 2) + c / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
    }
  });
  return 0;
}

// Dequantize to fp32 [rows, K] (D).
void orc_dequantize_f32(const uint8_t* codes, const uint8_t* scales, float s_t, int64_t rows,
                        int64_t K, float* out) {
  parallel_for(rows, [&](int64_t r) {
    for (int64_t c = 0; c < K; ++c) out[r * K + c] = dequant_elem(codes, scales, s_t, K, r, c);
  });
}

// Dequantize to bf16 bits [rows, K]: the fp32 value rounded to nearest even.
void orc_dequantize_bf16(const uint8_t* codes, const uint8_t* scales, float s_t, int64_t rows,
                         int64_t K, uint16_t* out) {
  parallel_for(rows, [&](int64_t r) {
    for (int64_t c = 0; c < K; ++c)
      out[r * K + c] = float_to_bf16_rne(dequant_elem(codes, scales, s_t, K, r, c));
  });
}

// Residual score per channel (QUADS explainer §2.2-B: channels ranked by the
// magnitude of the quantization residual).  r[m,c] = fl32(x[m,c] - v[m,c]).
// The pages fix no summation order; this one is fixed so that the score is
// one exact fp32 value (every addition sequential, starting from +0):
//   Q[j,i] = sum of |r[m,c]| over rows m of sub-chunk i of chunk j (16 rows,
//            ascending m; a sub-chunk past the last row is +0),
//   P[j]   = sum over the 8 sub-chunks i = 0..7 of Q[j,i], ascending i,
//   score  = sum over the 128-row chunks j ascending of P[j].
void orc_residual_scores(const void* x, int dtype, int64_t ldx, const uint8_t* codes,
                         const uint8_t* scales, float s_t, int64_t rows, int64_t K,
                         float* scores) {
  const int64_t kChunk = 128, kSub = 16;
  parallel_for(K, [&](int64_t c) {
    float score = 0.0f;
    for (int64_t m0 = 0; m0 < rows; m0 += kChunk) {
      float part = 0.0f;
      for (int64_t s0 = m0; s0 < m0 + kChunk; s0 += kSub) {
        float sub = 0.0f;
        for (int64_t m = s0; m < std::min(rows, s0 + kSub); ++m) {
          const float xv = load_elem(x, dtype, m, ldx, c);
          const float v = dequant_elem(codes, scales, s_t, K, m, c);
          const float r = xv - v;
          sub += std::fabs(r);
        }
        part += sub;
      }
      score += part;
    }
    scores[c] = score;
  });
}

// The same score in the plainer order of a sequential fp32 sum inside each
// 128-row chunk (no 16-row level), chunks summed in ascending order.  The
// pages fix no order; this one is kept beside the order above so the tests
// can show that the choice of order does not change which channels are
// selected on the workloads' activations.
void orc_residual_scores_chunk128(const void* x, int dtype, int64_t ldx, const uint8_t* codes,
                                  const uint8_t* scales, float s_t, int64_t rows, int64_t K,
                                  float* scores) {
  const int64_t kChunk = 128;
  parallel_for(K, [&](int64_t c) {
    float score = 0.0f;
    for (int64_t m0 = 0; m0 < rows; m0 += kChunk) {
      float part = 0.0f;
      for (int64_t m = m0; m < std::min(rows, m0 + kChunk); ++m) {
        const float xv = load_elem(x, dtype, m, ldx, c);
        const float v = dequant_elem(codes, scales, s_t, K, m, c);
        const float r = xv - v;
        part += std::fabs(r);
      }
      score += part;
    }
    scores[c] = score;
  });
}

// The k channels with the largest score, ties to the lower channel index,
// written in rank order (QUADS explainer §2.2-B: binary mask of the top
// residual channels).
void orc_topk(const float* scores, int64_t K, int64_t k, int32_t* idx) {
  std::vector<int32_t> order(K);
  for (int64_t c = 0; c < K; ++c) order[c] = (int32_t)c;
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (scores[a] != scores[b]) return scores[a] > scores[b];
    return a < b;
  });
  for (int64_t j = 0; j < k; ++j) idx[j] = order[j];
}

// Residual of selected channels, rounded to bf16: out[m, j] = bf16(fl32(x -
// v))[m, idx[j]] for rows m of the tensor (the compensation operand).
void orc_residual_columns_bf16(const void* x, int dtype, int64_t ldx, const uint8_t* codes,
                               const uint8_t* scales, float s_t, int64_t rows, int64_t K,
                               const int32_t* idx, int64_t k, uint16_t* out) {
  parallel_for(rows, [&](int64_t m) {
    for (int64_t j = 0; j < k; ++j) {
      const float xv = load_elem(x, dtype, m, ldx, idx[j]);
      const float v = dequant_elem(codes, scales, s_t, K, m, idx[j]);
      out[m * k + j] = float_to_bf16_rne(xv - v);
    }
  });
}

// ------------------------------------------------------- MoE routing -------

// Per token, the topk largest of E logits in descending order, ties to the
// lower expert id; weights = softmax over the chosen logits (fp64, rounded to
// fp32).  (TRACE post, "Fonctionnement": the router makes a discrete expert
// choice; the normalisation over the chosen experts is a reading.)
void orc_route(const float* logits, int64_t T, int64_t E, int64_t topk, int32_t* ids,
               float* weights) {
  parallel_for(T, [&](int64_t t) {
    std::vector<int32_t> order(E);
    for (int64_t e = 0; e < E; ++e) order[e] = (int32_t)e;
    const float* l = logits + t * E;
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      if (l[a] != l[b]) return l[a] > l[b];
      return a < b;
    });
    const double lmax = l[order[0]];
    double den = 0.0;
    for (int64_t j = 0; j < topk; ++j) den += std::exp((double)l[order[j]] - lmax);
    for (int64_t j = 0; j < topk; ++j) {
      ids[t * topk + j] = order[j];
      weights[t * topk + j] = (float)(std::exp((double)l[order[j]] - lmax) / den);
    }
  });
}

// Token-expert pairs p = t*topk + j sorted stably by expert: sorted_pair[P],
// expert offsets [E+1] (exclusive scan of the per-expert counts) and the
// inverse map pos[p] (position of pair p in sorted order).  Returns -4 if an
// id is out of [0, E).
int orc_permute(const int32_t* ids, int64_t T, int64_t topk, int64_t E, int32_t* sorted_pair,
                int32_t* offsets, int32_t* pos) {
  const int64_t P = T * topk;
  std::vector<int64_t> count(E, 0);
  for (int64_t p = 0; p < P; ++p) {
    if (ids[p] < 0 || ids[p] >= E) return -4;
    count[ids[p]]++;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + (int32_t)count[e];
  std::vector<int64_t> fill(offsets, offsets + E);
  for (int64_t p = 0; p < P; ++p) {  // ascending p: stable
    const int64_t dst = fill[ids[p]]++;
    sorted_pair[dst] = (int32_t)p;
    pos[p] = (int32_t)dst;
  }
  return 0;
}

// ------------------------------------------------------------- GEMMs -------

// W4A4 expert GEMM with residual compensation, for a list of output rows
// (QUADS explainer §2.2-B; W4A4 for the bulk, a correction on the selected
// channels added to the quantized output):
//   Y[s, n] = sum_c  A^[t,c] * W^_e[n,c]  +  sum_{j<k} bf16(r[t, S_j]) * W^_e[n, S_j]
// with t = row_token[s], e = row_expert[s], A^ and W^ the exact real values
// G * s_b * s_t of the NVFP4 tensors, r the fp32 residual of the activation
// (x_hi is the pre-quantization activation [T, K]).  The compensation weight
// is the dequantized NVFP4 weight W^ (a reading: the rollout holds only the
// NVFP4 weights).  fp64 accumulation.  out is [nsel, ncol] for the output
// columns cols (nullable: all N columns).
void orc_moe_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, float a_st,
                       const void* x_hi, int x_dtype, int64_t K, const int32_t* comp_idx,
                       int64_t k, const uint8_t* w_codes, const uint8_t* w_scales,
                       const float* w_st, int64_t N, const int32_t* row_token,
                       const int32_t* row_expert, int64_t nsel, const int32_t* cols,
                       int64_t ncol, double* out) {
  parallel_for(nsel, [&](int64_t s) {
    const int64_t t = row_token[s];
    const int64_t e = row_expert[s];
    const uint8_t* wc = w_codes + e * N * (K / 2);
    const uint8_t* ws = w_scales + e * N * (K / 16);
    std::vector<double> a(K), rb(k);
    for (int64_t c = 0; c < K; ++c) a[c] = dequant_exact(a_codes, a_scales, a_st, K, t, c);
    for (int64_t j = 0; j < k; ++j)
      rb[j] = residual_bf16(x_hi, x_dtype, K, a_codes, a_scales, a_st, K, t, comp_idx[j]);
    for (int64_t q = 0; q < ncol; ++q) {
      const int64_t n = cols ? cols[q] : q;
      double acc = 0.0;
      for (int64_t c = 0; c < K; ++c) acc += a[c] * dequant_exact(wc, ws, w_st[e], K, n, c);
      for (int64_t j = 0; j < k; ++j) acc += rb[j] * dequant_exact(wc, ws, w_st[e], K, n, comp_idx[j]);
      out[s * ncol + q] = acc;
    }
  });
}

// SwiGLU on a fused gate/up output y [rows, 2I] (gate = first I columns):
// h = bf16(silu(g) * u), silu(z) = z / (1 + exp(-z)), evaluated in fp64 and
// rounded once from fp64 to bf16.
void orc_swiglu_bf16(const double* y, int64_t rows, int64_t I, uint16_t* h) {
  parallel_for(rows, [&](int64_t r) {
    for (int64_t i = 0; i < I; ++i) {
      const double g = y[r * 2 * I + i];
      const double u = y[r * 2 * I + I + i];
      const double v = g / (1.0 + std::exp(-g)) * u;
      h[r * I + i] = double_to_bf16_rne(v);
    }
  });
}

// Combine: out[t, n] = bf16( sum_j w[t,j] * Y[pos[t*topk+j], n] ), j ascending,
// fp64, rounded once from fp64 to bf16.  Y is fp32 [P, N] in sorted-pair
// order; pairs with pos < 0 (dropped by the permutation for an expert id
// outside [0, E)) are left out of the sum.
void orc_combine_bf16(const float* y, const int32_t* pos, const float* w, int64_t T,
                      int64_t topk, int64_t N, uint16_t* out) {
  parallel_for(T, [&](int64_t t) {
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t j = 0; j < topk; ++j) {
        const int64_t p = pos[t * topk + j];
        if (p < 0) continue;  // a pair the permutation dropped contributes nothing
        acc += (double)w[t * topk + j] * (double)y[p * N + n];
      }
      out[t * N + n] = double_to_bf16_rne(acc);
    }
  });
}

// Backward of the MoE layer's glue for the chained QAT backward (the
// straight-through GEMMs are the QAT functions below).
//
// SwiGLU backward.  h = silu(g) u with silu(g) = g s, s = 1 / (1 + exp(-g)),
// so dh/dg = u s (1 + g (1 - s)) and dh/du = g s.  y1 [rows, 2I] holds the
// gate pre-activation in columns [0, I) and the up one in [I, 2I) (dtype 0 =
// fp32, 1 = bf16); dh bf16 [rows, I]; dy1 [rows, 2I] fp64 = (dh dh/dg, dh dh/du).
void orc_swiglu_backward(const void* y1, int dtype, int64_t rows, int64_t I, const uint16_t* dh,
                         double* dy1) {
  parallel_for(rows, [&](int64_t r) {
    for (int64_t i = 0; i < I; ++i) {
      const double g = load_elem(y1, dtype, r, 2 * I, i);
      const double u = load_elem(y1, dtype, r, 2 * I, I + i);
      const double d = bf16_bits_to_float(dh[r * I + i]);
      const double sg = 1.0 / (1.0 + std::exp(-g));
      dy1[r * 2 * I + i] = d * u * sg * (1.0 + g * (1.0 - sg));
      dy1[r * 2 * I + I + i] = d * g * sg;
    }
  });
}

// Combine backward.  out[t] = sum_j w[t,j] y[pos[t,j]] gives
//   dy[pos[t,j], n] = bf16(fl32(w[t,j] dout[t,n]))   (the gradient the down
//                     projection's bf16 backward consumes; the fp32 product of
//                     a 24-bit and an 8-bit significand is exact in fp64, so
//                     rounding it to fp32 is fl32 of the real product)
//   dw[t,j]         = sum_n dout[t,n] y[pos[t,j], n]   (fp64; the routing
//                     weights' gradient).
// dout bf16 [T, N], y bf16 [P, N] (sorted-pair order), pos [T*topk].  Pairs
// with pos < 0 are skipped (dw = 0).  dw may be NULL.
void orc_combine_backward(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                          const float* w, int64_t T, int64_t topk, int64_t N, uint16_t* dy,
                          double* dw) {
  parallel_for(T, [&](int64_t t) {
    for (int64_t j = 0; j < topk; ++j) {
      const int64_t p = pos[t * topk + j];
      if (dw) dw[t * topk + j] = 0.0;
      if (p < 0) continue;
      const double wj = w[t * topk + j];
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double d = bf16_bits_to_float(dout[t * N + n]);
        dy[p * N + n] = float_to_bf16_rne((float)(wj * d));
        acc += d * (double)bf16_bits_to_float(y[p * N + n]);
      }
      if (dw) dw[t * topk + j] = acc;
    }
  });
}

// Asymmetric W4A16 QAT forward (QUADS explainer §2.2-A; TRACE post: the
// trainer takes its rounding from the rollout's recorded codes and scales):
//   Y[s, n] = sum_c a[a_row[s], c] * W^_e[n, c],   e = row_expert[s],
// a bf16 activations [*, K] (row stride lda).  out [nsel, ncol], fp64.
void orc_qat_fwd(const uint16_t* a, int64_t lda, const int32_t* a_row, const int32_t* row_expert,
                 int64_t nsel, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                 const float* w_st, int64_t N, const int32_t* cols, int64_t ncol, double* out) {
  parallel_for(nsel, [&](int64_t s) {
    const int64_t e = row_expert[s];
    const uint8_t* wc = w_codes + e * N * (K / 2);
    const uint8_t* ws = w_scales + e * N * (K / 16);
    for (int64_t q = 0; q < ncol; ++q) {
      const int64_t n = cols ? cols[q] : q;
      double acc = 0.0;
      for (int64_t c = 0; c < K; ++c)
        acc += (double)bf16_bits_to_float(a[a_row[s] * lda + c]) *
               dequant_exact(wc, ws, w_st[e], K, n, c);
      out[s * ncol + q] = acc;
    }
  });
}

// Straight-through input gradient: dX[s, c] = sum_n dY[dy_row[s], n] * W^_e[n, c]
// (identity STE through the fake quantizer).  dY bf16 [*, N].
void orc_qat_dgrad(const uint16_t* dy, int64_t ldy, const int32_t* dy_row,
                   const int32_t* row_expert, int64_t nsel, int64_t N, const uint8_t* w_codes,
                   const uint8_t* w_scales, const float* w_st, int64_t K, const int32_t* cols,
                   int64_t ncol, double* out) {
  parallel_for(nsel, [&](int64_t s) {
    const int64_t e = row_expert[s];
    const uint8_t* wc = w_codes + e * N * (K / 2);
    const uint8_t* ws = w_scales + e * N * (K / 16);
    for (int64_t q = 0; q < ncol; ++q) {
      const int64_t c = cols ? cols[q] : q;
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n)
        acc += (double)bf16_bits_to_float(dy[dy_row[s] * ldy + n]) *
               dequant_exact(wc, ws, w_st[e], K, n, c);
      out[s * ncol + q] = acc;
    }
  });
}

// Straight-through weight gradient of expert e:
//   dW_e[n, c] = sum over the expert's rows p in [p0, p1) of dY[p, n] * a[a_row[p], c]
// (dY rows in sorted-pair order, a gathered by a_row).  Output the requested
// (n, c) pairs: out[i] for (ns[i], cs[i]), fp64.
void orc_qat_wgrad(const uint16_t* dy, int64_t ldy, const uint16_t* a, int64_t lda,
                   const int32_t* a_row, int64_t p0, int64_t p1, const int32_t* ns,
                   const int32_t* cs, int64_t npts, double* out) {
  parallel_for(npts, [&](int64_t i) {
    double acc = 0.0;
    for (int64_t p = p0; p < p1; ++p)
      acc += (double)bf16_bits_to_float(dy[p * ldy + ns[i]]) *
             (double)bf16_bits_to_float(a[(int64_t)a_row[p] * lda + cs[i]]);
    out[i] = acc;
  });
}

}  // extern "C"

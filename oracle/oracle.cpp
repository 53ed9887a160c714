// oracle.cpp -- plain, slow fp64 CPU reference for the W4 (NVFP4) + dynamic LoRA linear.
//
// TEST INFRASTRUCTURE ONLY. This file is the yardstick the HIP path is measured against. Only the
// test suite, the smoke check and the benchmark's CPU-baseline leg may load it; the library under
// bit_linear_dynamic_amd/ never includes, links or calls it, and it shares no code with it.
//
// What it computes (FL2VA Turbo page, section "Implementation"):
//     output = NVFP4_base(x) + strength * (alpha / rank) * B(A(x))
// where the base path sees the activation multiplied by the checkpoint's per-input-channel
// pre_quant_scale and the bf16 LoRA branch sees the ORIGINAL activation (same section), and the
// LoRA delta is never folded into the 4-bit weights.
//
// The pages name the weight format only as "NVFP4" (FL2VA Turbo, first paragraph; MiniMax-H3
// Ultra Fast, "Active optimization stack" table). The element and scale encodings used here are the
// public definitions of that format: E2M1 elements (bias 1, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6),
// one E4M3 "FN" scale per 16 consecutive K-elements (bias 7, no infinities, NaN = S.1111.111,
// largest finite 448), and one fp32 per-tensor scale applied by multiplication on decode.
//
// Everything below is written for obviousness, not speed: scalar loops, fp64 accumulation in
// ascending k, nearest-value searches over the whole code table. OpenMP only splits independent
// output rows across threads; it does not change any output's arithmetic.

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// bf16 bit pattern -> exact double (bf16 is the top half of an IEEE binary32).
double bf16_to_double(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

}  // namespace

extern "C" {

// ------------------------------------------------------------------------------------------------
// Element and scale decoders (closed forms of the two 8-bit-or-less minifloats).
// ------------------------------------------------------------------------------------------------

// E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit. Exponent 0 is subnormal (0 or 0.5).
double orc_e2m1_value(int code) {
  const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  const double mag = (e == 0) ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

// E4M3 "FN": sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal
// (m/8 * 2^-6); all-ones exponent with all-ones mantissa is NaN; there are no infinities.
double orc_e4m3_value(int code) {
  const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return std::nan("");
  const double mag = (e == 0) ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

// ------------------------------------------------------------------------------------------------
// Encoders: round-to-nearest, ties to the code with an even (zero) mantissa LSB, saturating.
// The argument is the real number to encode; callers pass exact values or fp64 quotients that are
// provably on the same side of every rounding midpoint as the exact quotient.
// ------------------------------------------------------------------------------------------------

// Magnitude code 0..7 of the E2M1 value nearest |q|; |q| >= 6 saturates to 6 (code 7).
static int e2m1_nearest_magnitude(double a) {
  if (a >= 6.0) return 7;
  int lo = 0;
  for (int c = 0; c < 8; ++c)
    if (orc_e2m1_value(c) <= a) lo = c;
  if (lo == 7) return 7;
  const int hi = lo + 1;
  const double mid = 0.5 * (orc_e2m1_value(lo) + orc_e2m1_value(hi));  // exact: short dyadics
  if (a < mid) return lo;
  if (a > mid) return hi;
  return (lo & 1) ? hi : lo;  // tie: the code whose mantissa bit is 0
}

// E2M1 code of q. A result of magnitude zero is encoded as +0 (code 0) whatever the sign of q.
int orc_e2m1_encode(double q) {
  const int mag = e2m1_nearest_magnitude(std::fabs(q));
  if (mag == 0) return 0;
  return (q < 0.0) ? (0x8 | mag) : mag;
}

// E4M3 code of a non-negative v; v >= 448 saturates to 448 (code 0x7E), never to NaN.
int orc_e4m3_encode_nonneg(double v) {
  if (!(v > 0.0)) return 0;
  if (v >= 448.0) return 0x7E;
  int lo = 0;
  for (int c = 0; c <= 0x7E; ++c)
    if (orc_e4m3_value(c) <= v) lo = c;
  const int hi = lo + 1;  // lo < 0x7E because v < 448
  const double mid = 0.5 * (orc_e4m3_value(lo) + orc_e4m3_value(hi));
  if (v < mid) return lo;
  if (v > mid) return hi;
  return (lo & 1) ? hi : lo;
}

// ------------------------------------------------------------------------------------------------
// NVFP4 quantizer (dynamic activation quantization of the W4A4 variant, and the synthetic-weight
// fixture). MiniMax-H3 Ultra Fast, "Kernel path": activations are quantized to NVFP4 on every call.
// Reading of the format's scale rules (plain reading, stated here because the pages give none):
//   ts     = f32_rne(amax(|v|) / (6 * 448))       (1 if the tensor is all zero)
//   s_b    = E4M3_rne_satfinite(amax_b / (6 * ts))  per block of 16 along K
//   code   = E2M1_rne_sat(v / (E4M3(s_b) * ts))     (all codes 0 when s_b decodes to 0)
// Each quotient is the exact real quotient rounded once. fp64 realizes that: the numerators have
// at most 24 significant bits and the divisors at most 28, so a quotient that is not exactly a
// rounding midpoint lies much farther from one than fp64's division error, and one that is exactly
// a midpoint is computed exactly. For the fp32 tensor scale, rounding the correctly rounded fp64
// quotient to fp32 is itself a correct rounding (53 >= 2*24 + 2).
// Layout: codes [rows][K/2] with the even k in the low nibble; scales [rows][K/16].
// Returns 0, or -1 if K is not a multiple of 16 or an input is not finite.
// ------------------------------------------------------------------------------------------------
int orc_quantize_nvfp4(const float* v, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                       float* ts_out) {
  if (K % 16 != 0 || rows < 0) return -1;
  double amax = 0.0;
  for (int64_t i = 0; i < rows * K; ++i) {
    if (!std::isfinite(v[i])) return -1;
    amax = std::fmax(amax, std::fabs(static_cast<double>(v[i])));
  }
  const float ts = (amax == 0.0) ? 1.0f : static_cast<float>(amax / 2688.0);
  *ts_out = ts;
  const double six_ts = 6.0 * static_cast<double>(ts);  // exact
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < K / 16; ++b) {
      const float* blk = v + r * K + b * 16;
      double amax_b = 0.0;
      for (int i = 0; i < 16; ++i) amax_b = std::fmax(amax_b, std::fabs(static_cast<double>(blk[i])));
      const int sc = orc_e4m3_encode_nonneg(amax_b / six_ts);
      scales[r * (K / 16) + b] = static_cast<uint8_t>(sc);
      const double d = orc_e4m3_value(sc) * static_cast<double>(ts);  // exact (4 x 24 bits)
      for (int i = 0; i < 16; i += 2) {
        const int c0 = (d == 0.0) ? 0 : orc_e2m1_encode(static_cast<double>(blk[i]) / d);
        const int c1 = (d == 0.0) ? 0 : orc_e2m1_encode(static_cast<double>(blk[i + 1]) / d);
        codes[r * (K / 2) + b * 8 + i / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
      }
    }
  }
  return 0;
}

// Activation value the W4A4 quantizer sees: v = f32_rne(f32(x) * pqs[k]) (pqs NULL means 1).
// The product of a bf16 and an fp32 is exact in fp64, so one cast gives the single rounding.
void orc_prescale_f32(const uint16_t* x, const float* pqs, int64_t rows, int64_t K, float* v) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const double p = pqs ? static_cast<double>(pqs[k]) : 1.0;
      v[r * K + k] = static_cast<float>(bf16_to_double(x[r * K + k]) * p);
    }
}

// ------------------------------------------------------------------------------------------------
// Dequantization: out[r][k] = E2M1(code[r][k]) * E4M3(scale[r][k/16]) * ts, in fp64 (exact: at most
// 2 + 4 + 24 significant bits). ts = 1 gives the bare E2M1 x E4M3 product.
// ------------------------------------------------------------------------------------------------
void orc_dequant(const uint8_t* codes, const uint8_t* scales, double ts, int64_t rows, int64_t K,
                 double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t byte = codes[r * (K / 2) + k / 2];
      const int c = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      out[r * K + k] = orc_e2m1_value(c) * orc_e4m3_value(scales[r * (K / 16) + k / 16]) * ts;
    }
}

// ------------------------------------------------------------------------------------------------
// The linear itself, one output element at a time, fp64, ascending k.
//   base[m][n]  = sum_k act[m][k] * Wd[n][k]
//   where act = x (*) pqs                                (W4A16: FL2VA Turbo, "Implementation")
//      or act = E2M1(acode) * E4M3(ascale) * ts_a        (W4A4: dynamically quantized activation)
//   t[m][j]     = sum_k x[m][k] * A[j][k]                 (original, unscaled x)
//   delta[m][n] = sum_j t[m][j] * B[n][j]
//   y           = base + (strength * alpha / rank) * delta
// x: bf16 [M][K]; pqs: fp32 [K] or NULL; codes/scales: weight [N][K/2] / [N][K/16]; ts: fp32;
// A: bf16 [rank][K]; B: bf16 [N][rank]; y: fp64 [M][N]. rank == 0 or A == NULL means no adapter.
// act_codes/act_scales (may be NULL): the W4A4 activation [M][K/2] / [M][K/16] with scale ts_a.
// ------------------------------------------------------------------------------------------------
int orc_linear(const uint16_t* x, int64_t M, int64_t K, const float* pqs, const uint8_t* codes,
               const uint8_t* scales, float ts, int64_t N, const uint16_t* A, const uint16_t* B,
               int64_t rank, double alpha, double strength, const uint8_t* act_codes,
               const uint8_t* act_scales, float ts_a, double* y) {
  if (K % 16 != 0 || M < 0 || N < 0 || rank < 0) return -1;
  std::vector<double> Wd(static_cast<size_t>(N * K));
  orc_dequant(codes, scales, static_cast<double>(ts), N, K, Wd.data());
  std::vector<double> act(static_cast<size_t>(M * K));
  if (act_codes) {
    orc_dequant(act_codes, act_scales, static_cast<double>(ts_a), M, K, act.data());
  } else {
    for (int64_t m = 0; m < M; ++m)
      for (int64_t k = 0; k < K; ++k)
        act[m * K + k] = bf16_to_double(x[m * K + k]) * (pqs ? static_cast<double>(pqs[k]) : 1.0);
  }
  const bool lora = (A != nullptr && B != nullptr && rank > 0);
  const double c = lora ? strength * alpha / static_cast<double>(rank) : 0.0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    std::vector<double> t(static_cast<size_t>(lora ? rank : 0));
    for (int64_t j = 0; lora && j < rank; ++j) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += bf16_to_double(x[m * K + k]) * bf16_to_double(A[j * K + k]);
      t[j] = s;
    }
    for (int64_t n = 0; n < N; ++n) {
      double base = 0.0;
      for (int64_t k = 0; k < K; ++k) base += act[m * K + k] * Wd[n * K + k];
      double delta = 0.0;
      for (int64_t j = 0; lora && j < rank; ++j) delta += t[j] * bf16_to_double(B[n * rank + j]);
      y[m * N + n] = base + c * delta;
    }
  }
  return 0;
}

// ------------------------------------------------------------------------------------------------
// Fused gate/up epilogue (MiniMax-H3 Ultra Fast, "Kernel path" and the MLP row of "Active
// optimization stack"): the fused [gate; up] projection output y [M][2F] becomes
//   h[m][j] = SiLU(y[m][j]) * y[m][F + j],   SiLU(z) = z / (1 + exp(-z)),   in fp64.
// ------------------------------------------------------------------------------------------------
void orc_swiglu(const double* y, int64_t M, int64_t F, double* h) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t j = 0; j < F; ++j) {
      const double g = y[m * 2 * F + j], u = y[m * 2 * F + F + j];
      h[m * F + j] = g / (1.0 + std::exp(-g)) * u;
    }
}

// Q/K RMSNorm and partial split-half rotary embedding on a fused QKV output (MiniMax-H3 Ultra
// Fast, "Active optimization stack" (attention projections) and "Kernel path" item 2: a three-axis
// split-half rotary; which 96 of the 128 head dimensions rotate: MiniMax-H3 Turbo CMF card, "On
// parity"). y holds M rows of [q (qw) | k (qw) | v (rest)]; q and k are split into heads of 128
// consecutive columns. Per row and head, in this order:
//   1. RMSNorm over the head:  u_i = y_i / sqrt( (1/128) sum_j y_j^2 + eps ) * gamma[head*128 + i]
//      (gamma_q for q heads, gamma_k for k heads);
//   2. rotate the first rot dims. They form n_sec consecutive sections of widths sec[0], sec[1], ...
//      (summing to rot; one section of rot when sec is NULL), and each section is rotated in split
//      halves within itself: for section j at dims [o, o + w) with h = w / 2, the angle table
//      columns [o/2, o/2 + h) belong to it, and with c = cos[m][o/2 + i], s = sin[m][o/2 + i]:
//        out_{o+i}   = u_{o+i} * c - u_{o+i+h} * s
//        out_{o+i+h} = u_{o+i+h} * c + u_{o+i} * s          (i < h)
//      and out_i = u_i for rot <= i < 128.
// The two readings of "three-axis split-half" are one section of 96 (the halves pair dim i with
// i + 48, the axes living only in the table's columns) and three sections of 32 (each axis's dims
// pair within the axis). v columns are copied unchanged. cos/sin are [M][rot/2] (the caller's
// per-token angle table).
void orc_qk_norm_rope(const double* y, int64_t M, int64_t N, int64_t qw, int32_t rot, double eps,
                      const float* gamma_q, const float* gamma_k, const float* cos_t, const float* sin_t,
                      const int32_t* sec, int32_t n_sec, double* out) {
  const int64_t hd = 128;
  const int64_t tab = rot / 2;
  const int32_t one[1] = {rot};
  if (!sec) {
    sec = one;
    n_sec = 1;
  }
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t m = 0; m < M; ++m) {
    const double* yr = y + m * N;
    double* orow = out + m * N;
    for (int64_t n = 0; n < N; ++n) orow[n] = yr[n];
    for (int64_t c0 = 0; c0 < 2 * qw; c0 += hd) {
      const float* gamma = c0 < qw ? gamma_q + c0 : gamma_k + (c0 - qw);
      double ss = 0.0;
      for (int64_t i = 0; i < hd; ++i) ss += yr[c0 + i] * yr[c0 + i];
      const double inv = 1.0 / std::sqrt(ss / static_cast<double>(hd) + eps);
      double u[128];
      for (int64_t i = 0; i < hd; ++i) u[i] = yr[c0 + i] * inv * static_cast<double>(gamma[i]);
      for (int64_t i = 0; i < hd; ++i) orow[c0 + i] = u[i];
      int64_t o = 0;
      for (int32_t j = 0; j < n_sec; ++j) {
        const int64_t half = sec[j] / 2;
        for (int64_t i = 0; i < half; ++i) {
          const double c = cos_t[m * tab + o / 2 + i], s = sin_t[m * tab + o / 2 + i];
          orow[c0 + o + i] = u[o + i] * c - u[o + i + half] * s;
          orow[c0 + o + i + half] = u[o + i + half] * c + u[o + i] * s;
        }
        o += sec[j];
      }
    }
  }
}

// Merged route, for comparison with the dynamic path (the LoRA update merged into the weight before
// quantizing: MiniMax-H3 Turbo CMF card, "What the conversion did", backbone item, and "Which file";
// the dynamic path of FL2VA Turbo, "Implementation", never does this). The base weight acts on
// x (*) pqs, so a merged weight that reproduces base + c B (A x) carries the adapter term divided by
// pqs per input column:
//   m[n][k] = f32( Wd[n][k] + (c * sum_j B[n][j] * A[j][k]) / pqs[k] ),   c = strength * alpha / rank
// in fp64 with j ascending and one rounding to fp32 at the end; pqs NULL means ones. Then
// m (x (*) pqs) = Wd (x (*) pqs) + c B (A x) up to that rounding. Quantizing m with
// orc_quantize_nvfp4 gives the merged NVFP4 weight. codes/scales: [N][K/2] / [N][K/16]; A: bf16
// [rank][K]; B: bf16 [N][rank]; m: fp32 [N][K]. rank == 0 or A == NULL merges nothing.
int orc_merge_lora(const uint8_t* codes, const uint8_t* scales, float ts, int64_t N, int64_t K,
                   const uint16_t* A, const uint16_t* B, int64_t rank, double alpha, double strength,
                   const float* pqs, float* m) {
  if (K % 16 != 0 || N < 0 || rank < 0) return -1;
  std::vector<double> Wd(static_cast<size_t>(N * K));
  orc_dequant(codes, scales, static_cast<double>(ts), N, K, Wd.data());
  const bool lora = (A != nullptr && B != nullptr && rank > 0);
  const double c = lora ? strength * alpha / static_cast<double>(rank) : 0.0;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double s = 0.0;
      for (int64_t j = 0; lora && j < rank; ++j)
        s += bf16_to_double(B[n * rank + j]) * bf16_to_double(A[j * K + k]);
      const double p = pqs ? static_cast<double>(pqs[k]) : 1.0;
      m[n * K + k] = static_cast<float>(Wd[n * K + k] + c * s / p);
    }
  return 0;
}

// AdaLN modulation as a rank-24 curve (MiniMax-H3 Turbo CMF card, "What the conversion did";
// MiniMax-H3 Ultra Fast, "Why the pruned transformer matters"). Per block b the modulation vector is
//   adaln_b(t) = W_p,b u(t) + bias_b + c B_b (A_b silu(e(t)))  =  [W_p,b | B_b] v_b(t) + bias_b,
//   v_b(t) = [u(t) ; c A_b silu(e(t))],
// with u the pruned checkpoint's rb-value time coordinate (shared by every block), A_b [rl][E] and B_b
// the adapter's factors written against the full modulation matrix, e(t) the E-wide timestep
// embedding and c = strength * alpha / rank. u and e are sampled at S points of t in [0, 1]
// (t_i = i / (S - 1)); v_b is tabulated at those points and linearly interpolated between them.
//
// orc_adaln_table: table[b][i][q] = u[i][q] for q < rb, c * sum_k A_b[q - rb][k] * silu(emb[i][k])
//   otherwise (silu(z) = z / (1 + exp(-z)), fp64). u: fp32 [S][rb]; emb: fp32 [S][E]; A: bf16
//   [blocks][rl][E]; table: fp64 [blocks][S][rb + rl].
void orc_adaln_table(const float* u, const float* emb, const uint16_t* A, double c, int64_t blocks, int64_t S,
                     int64_t E, int64_t rb, int64_t rl, double* table) {
  const int64_t R = rb + rl;
  for (int64_t b = 0; b < blocks; ++b)
    for (int64_t i = 0; i < S; ++i) {
      double* row = table + (b * S + i) * R;
      for (int64_t q = 0; q < rb; ++q) row[q] = static_cast<double>(u[i * rb + q]);
      for (int64_t j = 0; j < rl; ++j) {
        double s = 0.0;
        for (int64_t k = 0; k < E; ++k) {
          const double z = static_cast<double>(emb[i * E + k]);
          s += bf16_to_double(A[(b * rl + j) * E + k]) * (z / (1.0 + std::exp(-z)));
        }
        row[rb + j] = c * s;
      }
    }
}

// orc_adaln_apply: for each requested t (clamped to [0, 1]): p = t (S - 1), i0 = min(floor(p), S - 2),
//   th = p - i0, v = (1 - th) table[b][i0] + th table[b][i0 + 1], and
//   out[tau][b][r] = bias[b][r] + sum_q M[b][r][q] v[q]   (fp64).
// M: bf16 [blocks][rows][R] = [W_p | B] row by row; bias: fp32 [blocks][rows] or NULL; table: fp64
// [blocks][S][R]; t: fp32 [T]; out: fp64 [T][blocks][rows]. Needs S >= 2.
void orc_adaln_apply(const uint16_t* M, const float* bias, const double* table, const float* t, int64_t T,
                     int64_t blocks, int64_t rows, int64_t S, int64_t R, double* out) {
  std::vector<double> v(static_cast<size_t>(R));
  for (int64_t tau = 0; tau < T; ++tau) {
    double tt = static_cast<double>(t[tau]);
    tt = tt < 0.0 ? 0.0 : (tt > 1.0 ? 1.0 : tt);
    const double p = tt * static_cast<double>(S - 1);
    int64_t i0 = static_cast<int64_t>(std::floor(p));
    if (i0 > S - 2) i0 = S - 2;
    const double th = p - static_cast<double>(i0);
    for (int64_t b = 0; b < blocks; ++b) {
      const double* t0 = table + (b * S + i0) * R;
      const double* t1 = t0 + R;
      for (int64_t q = 0; q < R; ++q) v[q] = (1.0 - th) * t0[q] + th * t1[q];
      for (int64_t r = 0; r < rows; ++r) {
        double acc = bias ? static_cast<double>(bias[b * rows + r]) : 0.0;
        for (int64_t q = 0; q < R; ++q) acc += bf16_to_double(M[(b * rows + r) * R + q]) * v[q];
        out[(tau * blocks + b) * rows + r] = acc;
      }
    }
  }
}

// fp32 -> bf16 bit pattern, round to nearest with ties to even (finite inputs): add 0x7FFF plus the
// lowest kept bit, then drop the low half-word.
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Mirror mode (a diagnostic beside the graded fp64 oracle): the linear with the rounding points the
// GPU path declares, everything else exact in fp64 --
//   xs  = bf16( f32(x * pqs) )                         the base operand
//   f   = f32( strength * alpha / (rank * ts) )
//   t'  = bf16( f * f32( sum_k x * A[j] ) )             the folded LoRA-down output
//   acc = sum_k xs * (E2M1 * E4M3) + sum_j t' * B        (fp64)
//   y   = bf16( f32(ts) * f32(acc) )
// so the GPU's y differs from it only by the order and precision of its fp32 accumulation. Same
// arguments as orc_linear (W4A16 only); y_bits: bf16 bit patterns [M][N].
int orc_linear_mirror(const uint16_t* x, int64_t M, int64_t K, const float* pqs, const uint8_t* codes,
                      const uint8_t* scales, float ts, int64_t N, const uint16_t* A, const uint16_t* B,
                      int64_t rank, double alpha, double strength, uint16_t* y_bits) {
  if (K % 16 != 0 || M < 0 || N < 0 || rank < 0) return -1;
  std::vector<double> Wq(static_cast<size_t>(N * K));
  orc_dequant(codes, scales, 1.0, N, K, Wq.data());
  const bool lora = (A != nullptr && B != nullptr && rank > 0);
  const float f = lora ? static_cast<float>(strength * alpha / (static_cast<double>(rank) * static_cast<double>(ts))) : 0.0f;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    std::vector<double> xs(static_cast<size_t>(K));
    for (int64_t k = 0; k < K; ++k) {
      const double xv = bf16_to_double(x[m * K + k]);
      xs[k] = pqs ? bf16_to_double(orc_f32_to_bf16(static_cast<float>(xv * static_cast<double>(pqs[k])))) : xv;
    }
    std::vector<double> tq(static_cast<size_t>(lora ? rank : 0));
    for (int64_t j = 0; lora && j < rank; ++j) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += bf16_to_double(x[m * K + k]) * bf16_to_double(A[j * K + k]);
      tq[j] = bf16_to_double(orc_f32_to_bf16(f * static_cast<float>(s)));
    }
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += xs[k] * Wq[n * K + k];
      for (int64_t j = 0; lora && j < rank; ++j) acc += tq[j] * bf16_to_double(B[n * rank + j]);
      y_bits[m * N + n] = orc_f32_to_bf16(ts * static_cast<float>(acc));
    }
  }
  return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"

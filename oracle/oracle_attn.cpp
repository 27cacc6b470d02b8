// CPU oracle for quantized flash attention -- TEST INFRASTRUCTURE ONLY.
//
// This file is the slow, plain, obviously-correct reference that the GPU
// library is checked against.  Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg may load it.  It shares no source with the GPU
// library: every number format (fp16, OCP e4m3), quantizer and attention loop
// below is written out here from its definition.
//
// Sources (cited by page title and section):
//  [P1] "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8"
//       (zolotukhin.ai, 2026-07-13) -- the method: int8 QK^T after subtracting
//       K's per-channel mean (section "K's outliers, and the subtraction softmax
//       does not notice"), fp32 online softmax with P <= 1 by construction and a
//       static P scale (section "The scale P needs is already sitting in a
//       register"), e4m3 P with static scale 448 (section "fp8 is not faster, it
//       is shaped correctly"), int8 KV cache for decode (section "What actually
//       changed for decode").
//  [P2] "QFlash: Bridging Quantization and Memory Efficiency in Vision
//       Transformer Attention" -- symmetric int8 quantization, eq. (1)-(2);
//       int8 x int8 -> int32 score matmul, eq. (3); row max on int32 scores,
//       eq. (4); the softmax constant s_Q*s_K*d^-1/2*log2(e) folded into an
//       exp2, Algorithm 1; per-tensor granularity, section 3.3 (C3).
//
// Readings of points the pages leave open are listed beside the function that
// takes them.  Parity of the full-output accuracy (cosine vs fp64) is pinned
// only qualitatively by the pages (perplexity table of [P1]); see the tests.
//
// Build: g++ -O2 -std=c++17 -fopenmp -fPIC -shared oracle_attn.cpp -o liboracle_attn.so
// (no -ffast-math: every fp32 step below must be an IEEE correctly rounded op).

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>
#include <algorithm>
#ifdef _OPENMP
#include <omp.h>
#endif

#if defined(__FAST_MATH__)
#error "the oracle must be built without -ffast-math"
#endif

namespace {

// ---------------------------------------------------------------- fp16 -----
// IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1F;
  const int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = std::ldexp((double)f, -24);                 // subnormal: f * 2^-24
  } else if (e == 31) {
    v = f ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
  } else {
    v = std::ldexp((double)(1024 + f), e - 25);     // (1 + f/1024) * 2^(e-15)
  }
  return sign ? -v : v;
}

float half_to_float(uint16_t h) { return (float)half_to_double(h); }  // exact

// Round a finite fp32 to binary16, round-to-nearest-even, overflow -> inf.
uint16_t float_to_half_rne(float x) {
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs((double)x);
  if (std::isnan(x)) return 0x7E00;
  if (a == 0.0) return sign;
  int e2;
  std::frexp(a, &e2);                // a = m * 2^e2, m in [0.5, 1)
  int E = e2 - 1;                    // a in [2^E, 2^(E+1))
  if (E < -14) E = -14;              // subnormal range shares the 2^-24 quantum
  double quantum = std::ldexp(1.0, E - 10);
  double q = a / quantum;            // exact (power-of-two scaling)
  double r = std::nearbyint(q);      // default rounding mode: ties to even
  double v = r * quantum;
  if (v >= 65520.0 || v > 65504.0) return sign | 0x7C00;
  // encode v
  if (v < std::ldexp(1.0, -14)) {
    return sign | (uint16_t)(v / std::ldexp(1.0, -24));
  }
  int ev;
  std::frexp(v, &ev);
  int Ev = ev - 1;
  uint16_t frac = (uint16_t)(v / std::ldexp(1.0, Ev - 10) - 1024.0);
  return sign | (uint16_t)((Ev + 15) << 10) | frac;
}

// ---------------------------------------------------------------- e4m3 -----
// OCP 8-bit floating point, E4M3 ("FN" flavour): exponent bias 7, 3 fraction
// bits, no infinities, 0x7F / 0xFF are NaN, largest finite value 448 = 1.75*2^8,
// smallest subnormal 2^-9.  [P1] section "fp8 is not faster, it is shaped
// correctly" fixes the static scale 448, i.e. this flavour's largest value.
double e4m3_decode(uint8_t b) {
  const int sign = (b >> 7) & 1;
  const int e = (b >> 3) & 0xF;
  const int f = b & 7;
  double v;
  if (e == 15 && f == 7) return std::numeric_limits<double>::quiet_NaN();
  if (e == 0) v = std::ldexp((double)f, -9);               // f/8 * 2^-6
  else v = std::ldexp((double)(8 + f), e - 10);            // (1+f/8) * 2^(e-7)
  return sign ? -v : v;
}

// Encode with round-to-nearest-even; finite values beyond 448 saturate to 448.
uint8_t e4m3_encode(float x) {
  if (std::isnan(x)) return 0x7F;
  uint8_t sign = std::signbit(x) ? 0x80 : 0;
  double a = std::fabs((double)x);
  if (a == 0.0) return sign;
  int e2;
  std::frexp(a, &e2);
  int E = e2 - 1;
  if (E < -6) E = -6;                 // subnormals: quantum 2^-9
  double quantum = std::ldexp(1.0, E - 3);
  double r = std::nearbyint(a / quantum);   // ties to even
  double v = r * quantum;
  if (v > 448.0) v = 448.0;           // saturate (RNE would give the absent 480)
  if (v == 0.0) return sign;
  if (v < std::ldexp(1.0, -6)) return sign | (uint8_t)(v / std::ldexp(1.0, -9));
  int ev;
  std::frexp(v, &ev);
  int Ev = ev - 1;
  uint8_t frac = (uint8_t)(v / std::ldexp(1.0, Ev - 3) - 8.0);
  return sign | (uint8_t)((Ev + 7) << 3) | frac;
}

// ---------------------------------------------------------------- int8 -----
// Symmetric int8 after [P2] eq. (1)-(2): scale s = amax / (2^(b-1) - 1) = amax/127,
// code = round(x / s).  Reading of the garbled rounding operator: round to
// nearest, ties to even (rint), clamped to [-127, 127]; a zero scale gives 0.
int8_t quant_i8(float x, float s) {
  if (s == 0.0f) return 0;
  float t = x / s;                    // IEEE fp32 division
  float r = std::rint(t);
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

float scale_from_amax(float amax) { return amax / 127.0f; }

enum { GRAN_TENSOR = 0, GRAN_BLOCK = 1, GRAN_TOKEN = 2, GRAN_CHANNEL = 3 };
// BLOCK granularity: one scale per block of BLOCK_N consecutive tokens of a (batch, head) --
// QFlash's per-block quantization with the blocks of its tiled loop (B_c keys, B_r queries).
constexpr int BLOCK_N = 64;
enum { PV_FP8 = 0, PV_INT8 = 1 };

// fp32(sm_scale * log2 e): the softmax constant is folded into an exp2 as in
// [P2] Algorithm 1 (s = s_Q * s_K * d^-1/2 * log2 e); computed in fp64 and
// rounded once.  sm_scale <= 0 selects 1/sqrt(d).
float softmax_kconst(float sm_scale, int d) {
  double sm = sm_scale > 0.0f ? (double)sm_scale : 1.0 / std::sqrt((double)d);
  return (float)(sm * 1.4426950408889634074);
}

// log2(448) rounded once to fp32: the static e4m3 scale expressed as an exponent
// offset, so that exp2(s - m + log2 448) = 448 * exp(s - m) <= 448.
const float LOG2_448 = (float)std::log2(448.0);
const float LOG2_127 = (float)std::log2(127.0);

}  // namespace

extern "C" {

// ------------------------------------------------------------ codecs -------
void orc_e4m3_encode(const float* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
}
void orc_e4m3_decode(const uint8_t* b, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_decode(b[i]);
}
void orc_half_to_double(const uint16_t* h, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = half_to_double(h[i]);
}
void orc_float_to_half(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_half_rne(x[i]);
}
void orc_quant_i8(const float* x, float s, int8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = quant_i8(x[i], s);
}
float orc_log2_448(void) { return LOG2_448; }
float orc_kconst(float sm_scale, int d) { return softmax_kconst(sm_scale, d); }

// ------------------------------------------------------- int32 QK^T --------
// acc[i][j] = sum_c a[i][c] * b[j][c] over int8 inputs ([P2] eq. (3)), computed
// in int64 and returned as int32 together with a flag saying whether any value
// left the int32 range.
int orc_int_dots(const int8_t* a, const int8_t* b, int32_t* acc, int m, int n, int d) {
  int overflow = 0;
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < n; ++j) {
      int64_t s = 0;
      for (int c = 0; c < d; ++c) s += (int64_t)a[(int64_t)i * d + c] * (int64_t)b[(int64_t)j * d + c];
      if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
      acc[(int64_t)i * n + j] = (int32_t)s;
    }
  return overflow;
}

// ------------------------------------------------------- V operand --------
// The PV operand of the prefill in its documented tile layout [B][Hkv][cap/64][d][64]: byte p
// of channel c in key tile T holds key 64T + perm(p), perm(p) = 32*((p%32)/16) + 8*((p%16)/4)
// + 4*(p/32) + p%4 (keys >= n_keys are 0).  [P1] "fp8 is not faster, it is shaped correctly"
// puts P and V on FP8 for the PV product; the cache keeps int8 V codes, so the operand is
// derived from them:
//   V CHANNEL, format PV_FP8:  e4m3(fp32(code))               (s_V[c] is applied after PV)
//   V CHANNEL, format PV_INT8: the code itself
//   V TOKEN (format PV_FP8 only): e4m3(fp32(code * f_n)), f_n = fp32(s_V[n] * c_V),
//     c_V = fp32(448 / fp32(127 * V_max)), V_max = max_n s_V[n] over the n_keys keys (written
//     to v_scale_max, the cache header), c_V = 0 when V_max = 0.  Reading: the per-token scale
//     is folded into the operand against one static bound per head, so |code * f_n| <= 448
//     (e4m3 saturates the last rounding) and P keeps its static scale; the output is
//     multiplied back by 1 / c_V.
static float token_v_factor(float vmax) { return vmax > 0.0f ? 448.0f / (127.0f * vmax) : 0.0f; }

// (vmax_in: the header V_max to build against, or NULL to compute it over the n_keys keys)
static void v_operand(int BH, int d, int cap, int n_keys, const int8_t* v_codes, const void* v_scales,
                      int v_gran, int v_op_format, uint8_t* v_op, float* v_scale_max,
                      const float* vmax_in = nullptr) {
  const int ntiles = cap / 64;
  for (int bg = 0; bg < BH; ++bg) {
    float cv = 0.0f;
    if (v_gran == GRAN_TOKEN) {
      float vmax = 0.0f;
      if (vmax_in) {
        vmax = vmax_in[bg];
      } else {
        for (int n = 0; n < n_keys; ++n)
          vmax = std::max(vmax, half_to_float(((const uint16_t*)v_scales)[(int64_t)bg * cap + n]));
      }
      if (v_scale_max) v_scale_max[bg] = vmax;
      cv = token_v_factor(vmax);
    }
    for (int T = 0; T < ntiles; ++T)
      for (int c = 0; c < d; ++c)
        for (int p = 0; p < 64; ++p) {
          const int perm = 32 * ((p % 32) / 16) + 8 * ((p % 16) / 4) + 4 * (p / 32) + p % 4;
          const int n = 64 * T + perm;
          uint8_t byte = 0;
          if (n < n_keys) {
            const int8_t code = v_codes[((int64_t)bg * cap + n) * d + c];
            if (v_gran == GRAN_TOKEN) {
              const float f = half_to_float(((const uint16_t*)v_scales)[(int64_t)bg * cap + n]) * cv;
              byte = e4m3_encode((float)code * f);
            } else {
              byte = v_op_format == PV_FP8 ? e4m3_encode((float)code) : (uint8_t)code;
            }
          }
          v_op[(((int64_t)bg * ntiles + T) * d + c) * 64 + p] = byte;
        }
  }
}

// ------------------------------------------------------ KV quantizer -------
// Quantize an fp16 K/V block [B][Hkv][N][d] into the int8 cache.
//
// K mean ([P1] "Why does subtracting K's channel mean not change the attention
// output?" and "K's outliers..."): one mean vector per (batch, kv-head) over all
// N keys (reading: the shift must be the same constant for every key of a
// query's row, which a per-head mean over every key guarantees).  The sum is
// taken exactly in int64 fixed point (every fp16 times 2^24 is an integer),
// then mu = fp32( double(S) / (N * 2^24) ).
//
// K codes: x = fp32(k) - mu (fp32 subtraction); scale over the granularity set
// (CHANNEL: fp32 per (b,g,c); TOKEN: per (b,g,n), stored as fp16; BLOCK: fp32 per
// (b,g, block of BLOCK_N keys) ([P2] section 3.3, per-block quantization); TENSOR: one
// fp32 for the whole tensor) s = fp32(amax/127), rounded to its storage type;
// code = quant_i8(x, s_stored).  V codes the same way without a mean (V never
// subtracts one).
//
// Layouts written (all row-major): k_codes/v_codes int8 [B][Hkv][cap][d];
// k_scales: CHANNEL fp32 [B][Hkv][d], TOKEN fp16 bits [B][Hkv][cap], BLOCK fp32
// [B][Hkv][cap / BLOCK_N] (amax over the block's keys below N and all channels), TENSOR fp32 [1];
// v_scales: CHANNEL fp32 [B][Hkv][d], TOKEN fp16 bits [B][Hkv][cap]; k_mean fp32 [B][Hkv][d].
//
// v_op (optional): the PV operand of the prefill (see v_operand above), for per-channel V
// (format PV_FP8 or PV_INT8) or per-token V (format PV_FP8; the header V_max goes to
// v_scale_max [B][Hkv]).
//
// k_sum (optional, int64 [B][Hkv][d]): receives S itself, the header from which
// orc_kv_append continues the running mean (computed whenever it is asked for,
// also without the subtraction).
void orc_kv_quantize(int B, int H, int N, int d, int cap,
                     const uint16_t* k, const uint16_t* v,
                     int subtract_mean, int k_gran, int v_gran,
                     int8_t* k_codes, int8_t* v_codes,
                     void* k_scales, void* v_scales, float* k_mean,
                     uint8_t* v_op, int v_op_format, int64_t* k_sum, float* v_scale_max) {
  const int64_t rowsz = d;
  std::vector<float> mu((size_t)B * H * d, 0.0f);
  // 1. mean
  for (int bg = 0; bg < B * H; ++bg) {
    for (int c = 0; c < d; ++c) {
      float m = 0.0f;
      int64_t S = 0;
      if ((subtract_mean || k_sum) && N > 0) {
        for (int n = 0; n < N; ++n) {
          double kv = half_to_double(k[((int64_t)bg * N + n) * rowsz + c]);
          S += (int64_t)std::llround(kv * 16777216.0);   // exact integer
        }
        if (subtract_mean) m = (float)((double)S / ((double)N * 16777216.0));
      }
      if (k_sum) k_sum[(size_t)bg * d + c] = S;
      mu[(size_t)bg * d + c] = m;
      k_mean[(size_t)bg * d + c] = m;
    }
  }
  auto kx = [&](int bg, int n, int c) -> float {
    return half_to_float(k[((int64_t)bg * N + n) * rowsz + c]) - mu[(size_t)bg * d + c];
  };
  auto vx = [&](int bg, int n, int c) -> float {
    return half_to_float(v[((int64_t)bg * N + n) * rowsz + c]);
  };
  // 2. K scales and codes
  float ktensor_s = 0.0f;
  if (k_gran == GRAN_TENSOR) {
    float amax = 0.0f;
    for (int bg = 0; bg < B * H; ++bg)
      for (int n = 0; n < N; ++n)
        for (int c = 0; c < d; ++c) amax = std::max(amax, std::fabs(kx(bg, n, c)));
    ktensor_s = scale_from_amax(amax);
    ((float*)k_scales)[0] = ktensor_s;
  }
  for (int bg = 0; bg < B * H; ++bg) {
    if (k_gran == GRAN_CHANNEL) {
      for (int c = 0; c < d; ++c) {
        float amax = 0.0f;
        for (int n = 0; n < N; ++n) amax = std::max(amax, std::fabs(kx(bg, n, c)));
        float s = scale_from_amax(amax);
        ((float*)k_scales)[(size_t)bg * d + c] = s;
        for (int n = 0; n < N; ++n)
          k_codes[((int64_t)bg * cap + n) * rowsz + c] = quant_i8(kx(bg, n, c), s);
      }
    } else if (k_gran == GRAN_BLOCK) {
      // one fp32 scale per block of BLOCK_N keys: the amax over the block's keys (those below
      // N) and all channels; k_scales fp32 [B][H][cap / BLOCK_N]
      for (int n0 = 0; n0 < N; n0 += BLOCK_N) {
        const int n1 = std::min(N, n0 + BLOCK_N);
        float amax = 0.0f;
        for (int n = n0; n < n1; ++n)
          for (int c = 0; c < d; ++c) amax = std::max(amax, std::fabs(kx(bg, n, c)));
        const float s = scale_from_amax(amax);
        ((float*)k_scales)[(int64_t)bg * (cap / BLOCK_N) + n0 / BLOCK_N] = s;
        for (int n = n0; n < n1; ++n)
          for (int c = 0; c < d; ++c) k_codes[((int64_t)bg * cap + n) * rowsz + c] = quant_i8(kx(bg, n, c), s);
      }
    } else if (k_gran == GRAN_TOKEN) {
      for (int n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int c = 0; c < d; ++c) amax = std::max(amax, std::fabs(kx(bg, n, c)));
        uint16_t sh = float_to_half_rne(scale_from_amax(amax));
        ((uint16_t*)k_scales)[(int64_t)bg * cap + n] = sh;
        float s = half_to_float(sh);
        for (int c = 0; c < d; ++c)
          k_codes[((int64_t)bg * cap + n) * rowsz + c] = quant_i8(kx(bg, n, c), s);
      }
    } else {
      for (int n = 0; n < N; ++n)
        for (int c = 0; c < d; ++c)
          k_codes[((int64_t)bg * cap + n) * rowsz + c] = quant_i8(kx(bg, n, c), ktensor_s);
    }
  }
  // 3. V scales and codes
  for (int bg = 0; bg < B * H; ++bg) {
    if (v_gran == GRAN_CHANNEL) {
      for (int c = 0; c < d; ++c) {
        float amax = 0.0f;
        for (int n = 0; n < N; ++n) amax = std::max(amax, std::fabs(vx(bg, n, c)));
        float s = scale_from_amax(amax);
        ((float*)v_scales)[(size_t)bg * d + c] = s;
        for (int n = 0; n < N; ++n)
          v_codes[((int64_t)bg * cap + n) * rowsz + c] = quant_i8(vx(bg, n, c), s);
      }
    } else {
      for (int n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int c = 0; c < d; ++c) amax = std::max(amax, std::fabs(vx(bg, n, c)));
        uint16_t sh = float_to_half_rne(scale_from_amax(amax));
        ((uint16_t*)v_scales)[(int64_t)bg * cap + n] = sh;
        float s = half_to_float(sh);
        for (int c = 0; c < d; ++c)
          v_codes[((int64_t)bg * cap + n) * rowsz + c] = quant_i8(vx(bg, n, c), s);
      }
    }
  }
  // 4. PV operand (and, for per-token V, the header V_max)
  if (v_op) v_operand(B * H, d, cap, N, v_codes, v_scales, v_gran, v_op_format, v_op, v_scale_max);
}

// The PV operand of a cache's first n_keys keys, from its int8 V codes and scales (after
// appends, whose rows the operand does not yet hold); see v_operand.
void orc_v_operand(int B, int H, int d, int cap, int n_keys, const int8_t* v_codes, const void* v_scales,
                   int v_gran, int v_op_format, uint8_t* v_op, float* v_scale_max) {
  v_operand(B * H, d, cap, n_keys, v_codes, v_scales, v_gran, v_op_format, v_op, v_scale_max);
}

// -------------------------------------------------------- KV append --------
// Append T new tokens to an int8 cache whose first n_before rows are filled,
// keeping the running per-channel K mean that [P1] describes for decode (section
// "K's outliers, and the subtraction softmax does not notice": K arrives one
// token at a time, a running channel mean lives in the cache header, the mean
// lags by one token, so the shift is no longer exactly zero).
//
// Readings:
//  - the token at position n (n = n_before + t) is shifted by the mean of the n
//    tokens before it, mu_n = fp32( double(S_n) / (n * 2^24) ), where S_n is the
//    exact int64 sum of fp16 * 2^24 over those tokens, and mu_0 = 0 (the first
//    token of an empty cache is not shifted);
//  - K and V scales are per token (fp16, as GRAN_TOKEN of orc_kv_quantize): a
//    shift that moves with n leaves no fixed per-channel range to scale;
//  - the header k_sum [B][Hkv][d] (int64) holds S_{n_before} on entry and
//    S_{n_before+T} on exit; k_mean [B][Hkv][d] receives the mean after the append.
// Layouts: k, v fp16 [B][Hkv][T][d]; k_codes/v_codes int8 [B][Hkv][cap][d] (rows
// n_before .. n_before+T-1 written); k_scales/v_scales fp16 bits [B][Hkv][cap].
void orc_kv_append(int B, int H, int T, int d, int cap, int n_before,
                   const uint16_t* k, const uint16_t* v, int64_t* k_sum,
                   int8_t* k_codes, int8_t* v_codes, uint16_t* k_scales, uint16_t* v_scales,
                   float* k_mean) {
  std::vector<float> x(d);
  for (int bg = 0; bg < B * H; ++bg) {
    int64_t* S = k_sum + (size_t)bg * d;
    for (int t = 0; t < T; ++t) {
      const int n = n_before + t;
      const uint16_t* kr = k + ((int64_t)bg * T + t) * d;
      const uint16_t* vr = v + ((int64_t)bg * T + t) * d;
      float kamax = 0.0f, vamax = 0.0f;
      for (int c = 0; c < d; ++c) {
        const float mu = n > 0 ? (float)((double)S[c] / ((double)n * 16777216.0)) : 0.0f;
        x[c] = half_to_float(kr[c]) - mu;
        kamax = std::max(kamax, std::fabs(x[c]));
        vamax = std::max(vamax, std::fabs(half_to_float(vr[c])));
      }
      const uint16_t ksh = float_to_half_rne(scale_from_amax(kamax));
      const uint16_t vsh = float_to_half_rne(scale_from_amax(vamax));
      k_scales[(int64_t)bg * cap + n] = ksh;
      v_scales[(int64_t)bg * cap + n] = vsh;
      const float ks = half_to_float(ksh), vs = half_to_float(vsh);
      for (int c = 0; c < d; ++c) {
        k_codes[((int64_t)bg * cap + n) * d + c] = quant_i8(x[c], ks);
        v_codes[((int64_t)bg * cap + n) * d + c] = quant_i8(half_to_float(vr[c]), vs);
      }
      for (int c = 0; c < d; ++c) S[c] += (int64_t)std::llround(half_to_double(kr[c]) * 16777216.0);
    }
    const int n_after = n_before + T;
    for (int c = 0; c < d; ++c)
      k_mean[(size_t)bg * d + c] = n_after > 0 ? (float)((double)S[c] / ((double)n_after * 16777216.0)) : 0.0f;
  }
}

// -------------------------------------------------------- Q quantizer ------
// Q rows [B][Hq][L][d] fp16 -> int8 codes and fp32 scales.  When K carries
// per-channel scales they are folded into Q first (q' = fp32(q) * s_K[g][c]),
// which makes the dequantization constant of a score row uniform across its
// keys, the condition [P2] section 3.3 (C3) names for comparing integer scores.
// q_gran TOKEN: one scale per row (fp32(amax/127)); BLOCK: one scale per block of
// BLOCK_N query positions of a (batch, head) ([P2] section 3.3: per-block quantization,
// the blocks the tiled loop takes); TENSOR: one scale over all rows of the call.  Outputs: codes [B][Hq][L][d], scales [B][Hq][L].
void orc_quantize_q(int B, int Hq, int Hkv, int L, int d, const uint16_t* q,
                    const float* k_scales_channel /* NULL unless K is CHANNEL */,
                    int q_gran, int8_t* codes, float* scales) {
  const int G = Hq / Hkv;
  std::vector<float> qq((size_t)B * Hq * L * d);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h)
      for (int i = 0; i < L; ++i)
        for (int c = 0; c < d; ++c) {
          size_t idx = (((size_t)b * Hq + h) * L + i) * d + c;
          float x = half_to_float(q[idx]);
          if (k_scales_channel) x = x * k_scales_channel[((size_t)b * Hkv + h / G) * d + c];
          qq[idx] = x;
        }
  float tensor_s = 0.0f;
  if (q_gran == GRAN_TENSOR) {
    float amax = 0.0f;
    for (float x : qq) amax = std::max(amax, std::fabs(x));
    tensor_s = scale_from_amax(amax);
  }
  const size_t rows = (size_t)B * Hq * L;
  for (size_t r = 0; r < rows; ++r) {
    float s = tensor_s;
    if (q_gran == GRAN_TOKEN) {
      float amax = 0.0f;
      for (int c = 0; c < d; ++c) amax = std::max(amax, std::fabs(qq[r * d + c]));
      s = scale_from_amax(amax);
    } else if (q_gran == GRAN_BLOCK) {
      // the block of BLOCK_N query positions of this (batch, head) that holds row r
      const size_t bh = r / L, i0 = (r % L) / BLOCK_N * BLOCK_N, i1 = std::min((size_t)L, i0 + BLOCK_N);
      float amax = 0.0f;
      for (size_t i = i0; i < i1; ++i)
        for (int c = 0; c < d; ++c) amax = std::max(amax, std::fabs(qq[(bh * L + i) * d + c]));
      s = scale_from_amax(amax);
    }
    scales[r] = s;
    for (int c = 0; c < d; ++c) codes[r * d + c] = quant_i8(qq[r * d + c], s);
  }
}

// ------------------------------------------------- prefill emulation -------
// Emulates the quantized prefill for the listed rows (or all rows when
// rows == NULL).  Keys are cut into tiles of block_c keys ([P2] Algorithm 1's loop
// over key blocks); tile t belongs to stream t % n_streams, and each stream runs
// its own online softmax over its tiles in ascending order.  Reading: the pages fix
// neither the order nor the grouping of the key blocks, so the split into
// interleaved streams (merged at the end by the log-sum-exp rule, below) is part of
// the numerical contract; P codes depend on the stream's running max.
//
// Per row (b, h, i), kv-head g = h / (Hq/Hkv), visible keys j < kv_len and,
// when causal, j <= q_offset + i:
//   acc_j  = sum_c qcode_c * kcode_{g,j,c}                  exact int32  [P2] eq. (3)
//   c_j    = fp32(s_Q * kconst)            (K CHANNEL: s_K folded into Q)
//          = fp32(fp32(s_Q * kconst) * s_K) (K TENSOR)
//          = fp32(fp32(s_Q * kconst) * s_K[j]) (K TOKEN: one fp16 scale per key;
//                                               K BLOCK: the fp32 scale of j's key block)
//   per tile: m_new = max(m_old, max_j fp32(c_j * acc_j))     running max  [P1] "The scale P needs..."
//             mL    = fp32(m_new - log2 448)   (log2 127 in INT8 mode)
//             x_j   = fp32(c_j * acc_j - mL)   one rounding (a fused multiply-add)
//             p_j   = fp32(exp2(x_j)) = static_scale * exp(s_j - m_new), <= static scale
//             FP8:  P_j = e4m3(p_j)                          [P1] static scale 448
//             INT8: P_j = rint(p_j) (<= 127)                  [P1] static scale 127
//   per stream: O_s = sum over its tiles of 2^(m_tile - m_s) * sum_j dec(P_j) * Vop_j,
//               l_s = sum over its tiles of 2^(m_tile - m_s) * sum_j w_j        (fp64)
//               with w_j = dec(P_j) (norm_fp32 == 0) or w_j = p_j (norm_fp32 == 1)
//   merge:      M = max_s m_s, O = sum_s 2^(m_s - M) O_s, l = sum_s 2^(m_s - M) l_s
//   out_c = O_c * g_c / l with g_c = s_V,c (V CHANNEL) or 1 / c_V (V TOKEN, whose operand
//   carries f_n = s_V[n] * c_V -- see v_operand);  lse (optional) = M + log2(l) - log2(static scale), the row's
//   base-2 log-sum-exp in the units of c * acc (log2 of the sum of 2^(c * acc_j) the weights
//   approximate); flushed_mass (optional, a diagnostic) = the share of the row's softmax
//   mass over the quantized scores, sum_j 2^(c * acc_j) in fp64, held by keys whose P code
//   is zero (the mass [P1]'s first figure counts below the int8 threshold).
// Readings: by default the denominator l sums the quantized weights dec(P_j), so mass
// whose code rounds to zero drops out of both numerator and denominator, the
// renormalization that [P1] section "Then the easy matmul turns out to be the hard one"
// describes for int8 P; norm_fp32 = 1 gives the other reading, l = sum of the unquantized
// fp32 p_j.  The static scale is applied as the exponent offset log2(448) that the max
// subtraction already carries.  V's PV operand is that of v_operand (e4m3 of the code, or of
// code * f_n for per-token V).
// exp2 is the correctly rounded fp64 exp2 rounded to fp32.
// MX scores (q_vals non-null; Q and K below 8 bits on the matrix core's fp6 / fp4 operand
// types, see orc_mx_quantize): acc_j is replaced by s_j = fp32(sum_c qv_c * kv_{g,j,c}), the
// dot of the dequantized MX values (q_vals [rows][d], k_vals [B*Hkv][cap][d]) in fp64 rounded
// once, and c_j = kconst; everything after the scores is the same.  debug_sf receives s_j.
// Returns the number of P codes produced (for diagnostics).
int64_t orc_prefill_emulate(int B, int Hq, int Hkv, int d, int q_len, int kv_len, int cap,
                            int q_offset, int causal, float sm_scale, int block_c, int n_streams,
                            const int8_t* qcodes, const float* qscales,
                            const int8_t* k_codes, const void* k_scales, int k_gran,
                            const int8_t* v_codes, const void* v_scales, int v_gran,
                            const float* v_scale_max,
                            int pv_mode, const int64_t* rows, int64_t nrows,
                            double* out, int32_t* debug_s, uint8_t* p_codes,
                            int64_t* flushed_count, int norm_fp32, double* lse,
                            double* flushed_mass, const double* q_vals, const double* k_vals,
                            float* debug_sf) {
  const int G = Hq / Hkv;
  const float kc = softmax_kconst(sm_scale, d);
  const int64_t total_rows = rows ? nrows : (int64_t)B * Hq * q_len;
  // value of the V operand for each int8 code (index code + 128), per-channel V
  double vdec[256];
  for (int code = -128; code < 128; ++code)
    vdec[code + 128] = pv_mode == PV_FP8 ? e4m3_decode(e4m3_encode((float)code)) : (double)code;
  // per-token V: the operand values e4m3(code * f_n) of every visible key, built once
  std::vector<double> vtok;
  if (v_gran == GRAN_TOKEN) {
    const int ntiles = cap / 64;
    std::vector<uint8_t> op((size_t)B * Hkv * ntiles * d * 64);
    v_operand(B * Hkv, d, cap, kv_len, v_codes, v_scales, GRAN_TOKEN, PV_FP8, op.data(), nullptr, v_scale_max);
    vtok.resize((size_t)B * Hkv * kv_len * d);
    for (int bg = 0; bg < B * Hkv; ++bg)
      for (int T = 0; T < ntiles; ++T)
        for (int c = 0; c < d; ++c)
          for (int p = 0; p < 64; ++p) {
            const int n = 64 * T + 32 * ((p % 32) / 16) + 8 * ((p % 16) / 4) + 4 * (p / 32) + p % 4;
            if (n < kv_len)
              vtok[((size_t)bg * kv_len + n) * d + c] = e4m3_decode(op[(((size_t)bg * ntiles + T) * d + c) * 64 + p]);
          }
  }
  int64_t produced = 0, flushed = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : produced, flushed)
  for (int64_t rr = 0; rr < total_rows; ++rr) {
    const int64_t r = rows ? rows[rr] : rr;
    const int i = (int)(r % q_len);
    const int h = (int)((r / q_len) % Hq);
    const int b = (int)(r / ((int64_t)q_len * Hq));
    const int g = h / G;
    const int64_t bg = (int64_t)b * Hkv + g;
    const int8_t* qc = q_vals ? nullptr : qcodes + r * d;
    const float sq = q_vals ? 1.0f : qscales[r];
    float c = q_vals ? kc : sq * kc;   // (MX scores carry their block scales: c = kconst)
    if (!q_vals && k_gran == GRAN_TENSOR) c = c * ((const float*)k_scales)[0];
    // the dequantization constant of key j
    auto cj = [&](int j) -> float {
      if (q_vals) return c;
      if (k_gran == GRAN_TOKEN) return c * half_to_float(((const uint16_t*)k_scales)[bg * cap + j]);
      if (k_gran == GRAN_BLOCK) return c * ((const float*)k_scales)[bg * (cap / BLOCK_N) + j / BLOCK_N];
      return c;
    };
    const int last = causal ? std::min(kv_len, q_offset + i + 1) : kv_len;
    const float L = pv_mode == PV_FP8 ? LOG2_448 : LOG2_127;
    const int ntiles = (last + block_c - 1) / block_c;
    std::vector<double> Os((size_t)n_streams * d, 0.0), ls(n_streams, 0.0);
    // diagnostic: softmax mass of the quantized scores (fp64 weights 2^(c*acc - m)) in total
    // and on the keys whose P code is zero, per stream, rescaled like l
    std::vector<double> mass_t(n_streams, 0.0), mass_z(n_streams, 0.0);
    std::vector<float> ms(n_streams, -std::numeric_limits<float>::infinity());
    std::vector<float> acc(block_c);   // the tile's scores: exact int32 dots, or MX fp32 dots
    for (int st = 0; st < n_streams; ++st) {
      double* O = &Os[(size_t)st * d];
      double& l = ls[st];
      float& m = ms[st];
      for (int t = st; t < ntiles; t += n_streams) {
        const int t0 = t * block_c, t1 = std::min(last, t0 + block_c);
        float mt = -std::numeric_limits<float>::infinity();
        for (int j = t0; j < t1; ++j) {
          if (q_vals) {
            // MX scores: the dot of the dequantized values (dyadic rationals, summed in
            // fp64), rounded once to fp32
            const double* qv = q_vals + r * d;
            const double* kv = k_vals + (bg * cap + j) * d;
            double s = 0.0;
            for (int cc = 0; cc < d; ++cc) s += qv[cc] * kv[cc];
            acc[j - t0] = (float)s;
            if (debug_sf) debug_sf[r * (int64_t)kv_len + j] = (float)s;
          } else {
            const int8_t* kr = k_codes + (bg * cap + j) * d;
            int64_t s = 0;
            for (int cc = 0; cc < d; ++cc) s += (int64_t)qc[cc] * (int64_t)kr[cc];
            acc[j - t0] = (float)s;   // (exact: |s| < 2^24)
            if (debug_s) debug_s[r * (int64_t)kv_len + j] = (int32_t)s;
          }
          mt = std::max(mt, cj(j) * acc[j - t0]);
        }
        const float mnew = std::max(m, mt);
        // rescale what earlier tiles of this stream accumulated: factor 2^(m_old - m_new)
        const double alpha = std::isinf(m) ? 0.0 : std::exp2((double)m - (double)mnew);
        for (int cc = 0; cc < d; ++cc) O[cc] *= alpha;
        l *= alpha;
        mass_t[st] *= alpha;
        mass_z[st] *= alpha;
        m = mnew;
        const float mL = mnew - L;
        for (int j = t0; j < t1; ++j) {
          const float x = std::fma(cj(j), acc[j - t0], -mL);
          const float p = (float)std::exp2((double)x);
          double pd;
          if (pv_mode == PV_FP8) {
            uint8_t code = e4m3_encode(p);
            if (p_codes) p_codes[r * (int64_t)kv_len + j] = code;
            pd = e4m3_decode(code);
            if (code == 0) ++flushed;
          } else {
            float pc = std::rint(p);
            if (pc > 127.0f) pc = 127.0f;
            if (p_codes) p_codes[r * (int64_t)kv_len + j] = (uint8_t)pc;
            pd = pc;
            if (pc == 0.0f) ++flushed;
          }
          ++produced;
          l += norm_fp32 ? (double)p : pd;   // normalizer (see the readings above)
          const double w = std::exp2((double)cj(j) * (double)acc[j - t0] - (double)mnew);
          mass_t[st] += w;
          if (pd == 0.0) mass_z[st] += w;
          if (v_gran == GRAN_TOKEN) {
            const double* vt = &vtok[((size_t)bg * kv_len + j) * d];
            for (int cc = 0; cc < d; ++cc) O[cc] += pd * vt[cc];
          } else {
            const int8_t* vr = v_codes + (bg * cap + j) * d;
            for (int cc = 0; cc < d; ++cc) O[cc] += pd * vdec[vr[cc] + 128];
          }
        }
      }
    }
    // merge the streams: every stream's sums are brought to the common max M
    float M = -std::numeric_limits<float>::infinity();
    for (int st = 0; st < n_streams; ++st) M = std::max(M, ms[st]);
    std::vector<double> O(d, 0.0);
    double l = 0.0, mt = 0.0, mz = 0.0;
    for (int st = 0; st < n_streams; ++st) {
      if (std::isinf(ms[st])) continue;   // a stream that saw no key
      const double f = std::exp2((double)ms[st] - (double)M);
      for (int cc = 0; cc < d; ++cc) O[cc] += f * Os[(size_t)st * d + cc];
      l += f * ls[st];
      mt += f * mass_t[st];
      mz += f * mass_z[st];
    }
    if (flushed_mass) flushed_mass[r] = mt > 0.0 ? mz / mt : 0.0;
    double* o = out + r * d;
    const float cv = v_gran == GRAN_TOKEN ? token_v_factor(v_scale_max[bg]) : 0.0f;
    for (int cc = 0; cc < d; ++cc) {
      const double g = v_gran == GRAN_TOKEN ? (cv > 0.0f ? 1.0 / (double)cv : 0.0)
                                            : (double)((const float*)v_scales)[bg * d + cc];
      o[cc] = l > 0.0 ? O[cc] * g / l : 0.0;
    }
    if (lse) lse[r] = (double)M + std::log2(l) - (double)L;
  }
  if (flushed_count) *flushed_count = flushed;
  return produced;
}

// -------------------------------------------------- decode emulation -------
// One query token per head against the int8 cache ([P1] "What actually changed
// for decode": attention at batch one streams the int8 KV cache; no matrix
// core).  Reading: Q is quantized to int8 per head (scale fp32(amax/127), K
// CHANNEL scales folded in first), dots are exact int32, and
//   s_n = fp32(c_n * acc_n),  c_n = fp32(fp32(s_Q * kconst) * s_K,n) (K TOKEN; K BLOCK: the
//                                   scale of n's key block)
//                             c   = fp32(s_Q * kconst)                (K CHANNEL)
// after which softmax and PV are plain arithmetic on the dequantized V
// (s_V * code), evaluated here in fp64 as base-2 softmax over s_n.
// q [B][Hq][d] fp16; out [B][Hq][d] fp64; debug_qk int32 [B][Hq][kv_len].
void orc_decode_emulate(int B, int Hq, int Hkv, int d, int kv_len, int cap, float sm_scale,
                        const uint16_t* q, const int8_t* k_codes, const void* k_scales, int k_gran,
                        const int8_t* v_codes, const void* v_scales, int v_gran,
                        double* out, int32_t* debug_qk) {
  const int G = Hq / Hkv;
  const float kc = softmax_kconst(sm_scale, d);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < (int64_t)B * Hq; ++r) {
    const int h = (int)(r % Hq), b = (int)(r / Hq), g = h / G;
    const int64_t bg = (int64_t)b * Hkv + g;
    std::vector<float> qq(d);
    float amax = 0.0f;
    for (int c = 0; c < d; ++c) {
      float x = half_to_float(q[r * d + c]);
      if (k_gran == GRAN_CHANNEL) x = x * ((const float*)k_scales)[bg * d + c];
      qq[c] = x;
      amax = std::max(amax, std::fabs(x));
    }
    const float sq = scale_from_amax(amax);
    std::vector<int8_t> qc(d);
    for (int c = 0; c < d; ++c) qc[c] = quant_i8(qq[c], sq);
    const float ch = sq * kc;
    std::vector<float> s(kv_len);
    float mx = -std::numeric_limits<float>::infinity();
    for (int n = 0; n < kv_len; ++n) {
      const int8_t* kr = k_codes + (bg * cap + n) * d;
      int64_t a = 0;
      for (int c = 0; c < d; ++c) a += (int64_t)qc[c] * (int64_t)kr[c];
      if (debug_qk) debug_qk[r * (int64_t)kv_len + n] = (int32_t)a;
      float cn = ch;
      if (k_gran == GRAN_TOKEN) cn = ch * half_to_float(((const uint16_t*)k_scales)[bg * cap + n]);
      if (k_gran == GRAN_BLOCK) cn = ch * ((const float*)k_scales)[bg * (cap / BLOCK_N) + n / BLOCK_N];
      s[n] = cn * (float)a;
      mx = std::max(mx, s[n]);
    }
    std::vector<double> o(d, 0.0);
    double l = 0.0;
    for (int n = 0; n < kv_len; ++n) {
      double p = std::exp2((double)s[n] - (double)mx);
      l += p;
      const int8_t* vr = v_codes + (bg * cap + n) * d;
      double sv = v_gran == GRAN_TOKEN ? half_to_double(((const uint16_t*)v_scales)[bg * cap + n]) : 1.0;
      for (int c = 0; c < d; ++c) o[c] += p * sv * (double)vr[c];
    }
    for (int c = 0; c < d; ++c) {
      double sv = v_gran == GRAN_CHANNEL ? (double)((const float*)v_scales)[bg * d + c] : 1.0;
      out[r * d + c] = kv_len > 0 ? o[c] * sv / l : 0.0;
    }
  }
}

// ----------------------------------------------------- exact fp64 ----------
// Plain attention in fp64 from fp16 inputs: s_j = sm_scale * sum_c q_c k_jc,
// softmax by the two-pass definition (max, then exp-sum), out = sum_j w_j v_j.
// Masking as above (causal: key j visible to query i iff j <= q_offset + i).
// Optional kmu [B][Hkv][d] (fp64) is subtracted from K first -- used to check
// the shift invariance that makes the K-mean subtraction exact.
void orc_attn_exact(int B, int Hq, int Hkv, int d, int q_len, int kv_len,
                    int q_offset, int causal, double sm_scale,
                    const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const double* kmu, const int64_t* rows, int64_t nrows, double* out) {
  const int G = Hq / Hkv;
  const double sm = sm_scale > 0 ? sm_scale : 1.0 / std::sqrt((double)d);
  const int64_t total_rows = rows ? nrows : (int64_t)B * Hq * q_len;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t rr = 0; rr < total_rows; ++rr) {
    const int64_t r = rows ? rows[rr] : rr;
    const int i = (int)(r % q_len);
    const int h = (int)((r / q_len) % Hq);
    const int b = (int)(r / ((int64_t)q_len * Hq));
    const int64_t bg = (int64_t)b * Hkv + h / G;
    const int last = causal ? std::min(kv_len, q_offset + i + 1) : kv_len;
    std::vector<double> qd(d), s(std::max(last, 1));
    for (int c = 0; c < d; ++c) qd[c] = half_to_double(q[r * d + c]);
    double mx = -std::numeric_limits<double>::infinity();
    for (int j = 0; j < last; ++j) {
      double a = 0.0;
      for (int c = 0; c < d; ++c) {
        double kk = half_to_double(k[(bg * kv_len + j) * d + c]);
        if (kmu) kk -= kmu[bg * d + c];
        a += qd[c] * kk;
      }
      s[j] = a * sm;
      mx = std::max(mx, s[j]);
    }
    double l = 0.0;
    for (int j = 0; j < last; ++j) { s[j] = std::exp(s[j] - mx); l += s[j]; }
    double* o = out + r * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j < last; ++j) {
      const double w = s[j] / l;
      for (int c = 0; c < d; ++c) o[c] += w * half_to_double(v[(bg * kv_len + j) * d + c]);
    }
  }
}

// ------------------------------------------- exact fp64 over the int8 cache --
// Plain attention in fp64 over the dequantized int8 cache: the reference of the
// precision mode that splits the other operand of each product into exact 8-bit parts
// ([P4], the int8-KV prompt attention that keeps K and V as stored codes and splits
// q and p * v_scale into three exact 8-bit parts, 24 bits in all).  With the codes
// fixed, that mode approaches this definition:
//   K^_jc = k_code_jc * s_K,c (CHANNEL) or * s_K (TENSOR)   (the mean is not added back:
//           a constant shift of K moves every score of a row equally, which softmax ignores)
//   s_j = sm_scale * sum_c q_c K^_jc (q fp16 -> fp64), softmax by the two-pass definition,
//   out_c = sum_j w_j v_code_jc * s_V,c (V per channel).
// Masking as orc_attn_exact; q [B][Hq][q_len][d] fp16; codes [B][Hkv][cap][d].
void orc_attn_dequant(int B, int Hq, int Hkv, int d, int q_len, int kv_len, int cap,
                      int q_offset, int causal, double sm_scale, const uint16_t* q,
                      const int8_t* k_codes, const float* k_scales, int k_gran,
                      const int8_t* v_codes, const float* v_scales_channel,
                      const int64_t* rows, int64_t nrows, double* out) {
  const int G = Hq / Hkv;
  const double sm = sm_scale > 0 ? sm_scale : 1.0 / std::sqrt((double)d);
  const int64_t total_rows = rows ? nrows : (int64_t)B * Hq * q_len;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t rr = 0; rr < total_rows; ++rr) {
    const int64_t r = rows ? rows[rr] : rr;
    const int i = (int)(r % q_len);
    const int h = (int)((r / q_len) % Hq);
    const int b = (int)(r / ((int64_t)q_len * Hq));
    const int64_t bg = (int64_t)b * Hkv + h / G;
    const int last = causal ? std::min(kv_len, q_offset + i + 1) : kv_len;
    std::vector<double> qk(d), s(std::max(last, 1));
    for (int c = 0; c < d; ++c) {
      const double ks = k_gran == GRAN_CHANNEL ? (double)k_scales[bg * d + c] : (double)k_scales[0];
      qk[c] = half_to_double(q[r * d + c]) * ks;   // (q_c * s_K,c) * code = q_c * K^_jc
    }
    double mx = -std::numeric_limits<double>::infinity();
    for (int j = 0; j < last; ++j) {
      const int8_t* kr = k_codes + (bg * cap + j) * d;
      double a = 0.0;
      for (int c = 0; c < d; ++c) a += qk[c] * (double)kr[c];
      s[j] = a * sm;
      mx = std::max(mx, s[j]);
    }
    double l = 0.0;
    for (int j = 0; j < last; ++j) { s[j] = std::exp(s[j] - mx); l += s[j]; }
    double* o = out + r * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j < last; ++j) {
      const double w = s[j] / l;
      const int8_t* vr = v_codes + (bg * cap + j) * d;
      for (int c = 0; c < d; ++c) o[c] += w * (double)vr[c];
    }
    for (int c = 0; c < d; ++c) o[c] *= (double)v_scales_channel[bg * d + c];
  }
}

// -------------------------------------------------- sub-8-bit Q and K ------
// The question [P1] closes with ("whether Q and K survive four bits with per-thread
// scales is an accuracy question ... ask it of the grid before the hardware"), asked of
// the grids themselves: attention in fp64 with Q and K replaced by their dequantized
// values in a format, V and the softmax exact, against attention on the unquantized
// inputs.  K is shifted by its exact per-head channel mean first, as in the int8 path.
// Formats (a "block" is 32 consecutive channels of one row, the unit that one lane feeds
// to a 64-deep matrix-core step and that the OCP MX formats give one shared scale):
//   LB_INT8_ROW    int8 codes, one scale fp32(amax/127) per row (the int8 path's Q grid)
//   LB_INT8_BLOCK  int8 codes, one scale per block
//   LB_INT4_BLOCK  int4 codes in [-7, 7], scale fp32(amax/7) per block
//   LB_MXFP6       OCP MX fp6 E2M3 elements (max 7.5) with a shared E8M0 scale per block
//   LB_MXFP4       OCP MX fp4 E2M1 elements (max 6) with a shared E8M0 scale per block
// MX scale (OCP Microscaling Formats v1.0): X = 2^(floor(log2 amax) - emax_elem), emax_elem
// = 2 for both element types; elements are x / X rounded to the nearest value of the
// element grid, ties to the even code, and clamped to the largest (values of x / X in
// (max, 8) saturate, as the spec's scale choice implies); amax = 0 gives X = 1.
enum { LB_INT8_ROW = 0, LB_INT8_BLOCK = 1, LB_INT4_BLOCK = 2, LB_MXFP6 = 3, LB_MXFP4 = 4 };

// nonnegative magnitudes of the E2M1 and E2M3 grids in code order (code = exponent bits
// then mantissa bits; code & 1 is the mantissa's last bit)
static double e2m1_value(int code) {
  const int e = (code >> 1) & 3, m = code & 1;
  return e == 0 ? m * 0.5 : (1.0 + m * 0.5) * std::ldexp(1.0, e - 1);
}
static double e2m3_value(int code) {
  const int e = (code >> 3) & 3, m = code & 7;
  return e == 0 ? m * 0.125 : (1.0 + m * 0.125) * std::ldexp(1.0, e - 1);
}
// nearest grid value to |x| (ties to the even code), sign restored; ncodes magnitudes
static double to_grid(double x, double (*value)(int), int ncodes, int* code_out) {
  const double a = std::fabs(x);
  int best = 0;
  for (int c = 1; c < ncodes; ++c) {
    const double d = std::fabs(value(c) - a), db = std::fabs(value(best) - a);
    if (d < db || (d == db && (c & 1) == 0 && (best & 1) == 1)) best = c;
  }
  if (code_out) *code_out = best;
  return x < 0 ? -value(best) : value(best);
}

// dequantized value of row x[0..n) in format fmt (n a multiple of 32 for block formats)
static void lowbit_row(const float* x, int n, int fmt, double* out) {
  const int blk = fmt == LB_INT8_ROW ? n : 32;
  for (int b0 = 0; b0 < n; b0 += blk) {
    float amax = 0.0f;
    for (int c = b0; c < b0 + blk; ++c) amax = std::max(amax, std::fabs(x[c]));
    if (fmt == LB_INT8_ROW || fmt == LB_INT8_BLOCK || fmt == LB_INT4_BLOCK) {
      const float qmax = fmt == LB_INT4_BLOCK ? 7.0f : 127.0f;
      const float s = amax / qmax;
      for (int c = b0; c < b0 + blk; ++c) {
        float r = s == 0.0f ? 0.0f : std::rint(x[c] / s);
        r = std::min(std::max(r, -qmax), qmax);
        out[c] = (double)r * (double)s;
      }
    } else {
      const double X = amax == 0.0f ? 1.0 : std::ldexp(1.0, (int)std::floor(std::log2((double)amax)) - 2);
      for (int c = b0; c < b0 + blk; ++c)
        out[c] = X * (fmt == LB_MXFP4 ? to_grid(x[c] / X, e2m1_value, 8, nullptr)
                                      : to_grid(x[c] / X, e2m3_value, 32, nullptr));
    }
  }
}

// q [B][Hq][L][d], k, v [B][Hkv][N][d] fp16; out fp64 [B][Hq][L][d] for the listed rows (or
// all); causal as orc_attn_exact.  fmt_q and fmt_k are independent.
void orc_attn_lowbit(int B, int Hq, int Hkv, int d, int q_len, int kv_len, int q_offset, int causal,
                     double sm_scale, const uint16_t* q, const uint16_t* k, const uint16_t* v, int fmt_q,
                     int fmt_k, const int64_t* rows, int64_t nrows, double* out) {
  const int G = Hq / Hkv;
  const double sm = sm_scale > 0 ? sm_scale : 1.0 / std::sqrt((double)d);
  // dequantized K per head after the exact mean shift
  std::vector<double> kq((size_t)B * Hkv * kv_len * d);
#pragma omp parallel for schedule(dynamic, 1)
  for (int bg = 0; bg < B * Hkv; ++bg) {
    std::vector<float> x(d);
    std::vector<float> mu(d);
    for (int c = 0; c < d; ++c) {
      int64_t S = 0;
      for (int n = 0; n < kv_len; ++n)
        S += (int64_t)std::llround(half_to_double(k[((int64_t)bg * kv_len + n) * d + c]) * 16777216.0);
      mu[c] = kv_len > 0 ? (float)((double)S / ((double)kv_len * 16777216.0)) : 0.0f;
    }
    for (int n = 0; n < kv_len; ++n) {
      for (int c = 0; c < d; ++c) x[c] = half_to_float(k[((int64_t)bg * kv_len + n) * d + c]) - mu[c];
      lowbit_row(x.data(), d, fmt_k, &kq[((size_t)bg * kv_len + n) * d]);
    }
  }
  const int64_t total_rows = rows ? nrows : (int64_t)B * Hq * q_len;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t rr = 0; rr < total_rows; ++rr) {
    const int64_t r = rows ? rows[rr] : rr;
    const int i = (int)(r % q_len);
    const int h = (int)((r / q_len) % Hq);
    const int b = (int)(r / ((int64_t)q_len * Hq));
    const int64_t bg = (int64_t)b * Hkv + h / G;
    const int last = causal ? std::min(kv_len, q_offset + i + 1) : kv_len;
    std::vector<float> qf(d);
    std::vector<double> qd(d), s(std::max(last, 1));
    for (int c = 0; c < d; ++c) qf[c] = half_to_float(q[r * d + c]);
    lowbit_row(qf.data(), d, fmt_q, qd.data());
    double mx = -std::numeric_limits<double>::infinity();
    for (int j = 0; j < last; ++j) {
      const double* kr = &kq[((size_t)bg * kv_len + j) * d];
      double a = 0.0;
      for (int c = 0; c < d; ++c) a += qd[c] * kr[c];
      s[j] = a * sm;
      mx = std::max(mx, s[j]);
    }
    double l = 0.0;
    for (int j = 0; j < last; ++j) { s[j] = std::exp(s[j] - mx); l += s[j]; }
    double* o = out + r * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j < last; ++j)
      for (int c = 0; c < d; ++c) o[c] += s[j] / l * half_to_double(v[(bg * kv_len + j) * d + c]);
  }
}

// the grids themselves, for the pins: value of x rounded in fmt 3 (E2M3) or 4 (E2M1) with
// unit scale, and the dequantized row of a format
void orc_lowbit_element(const double* x, int64_t n, int fmt, double* out, int32_t* codes) {
  for (int64_t i = 0; i < n; ++i) {
    int cd = 0;
    out[i] = fmt == LB_MXFP4 ? to_grid(x[i], e2m1_value, 8, &cd) : to_grid(x[i], e2m3_value, 32, &cd);
    if (codes) codes[i] = cd;
  }
}
void orc_lowbit_row(const float* x, int n, int fmt, double* out) { lowbit_row(x, n, fmt, out); }

// MX encoding of rows x [rows][d] (d a multiple of 32) in fmt LB_MXFP6 or LB_MXFP4, as the
// matrix core's scaled fp6 / fp4 operands take it: per block of 32 channels the shared
// scale X = 2^e, e = floor(log2 amax) - 2 (OCP MX v1.0's choice, emax 2 for both element
// types; amax = 0 gives e = 0), stored as its E8M0 byte 127 + e; per element the code of
// x / X on the element grid (to_grid: nearest, ties to the even code, saturating), with the
// sign bit (bit 5 for E2M3, bit 3 for E2M1) set for negative x whose magnitude code is not
// zero (a zero element is +0).  codes [rows][d], scale_bytes [rows][d/32], values (the
// dequantized +-grid * X, fp64) [rows][d].  Returns -1 if a scale falls outside the E8M0
// range, else 0.
int orc_mx_quantize(const float* x, int64_t rows, int d, int fmt, uint8_t* codes, uint8_t* scale_bytes,
                    double* values) {
  const int sign_bit = fmt == LB_MXFP4 ? 8 : 32;
  int bad = 0;
  for (int64_t r = 0; r < rows; ++r)
    for (int b0 = 0; b0 < d; b0 += 32) {
      const float* xr = x + r * d;
      float amax = 0.0f;
      for (int c = b0; c < b0 + 32; ++c) amax = std::max(amax, std::fabs(xr[c]));
      const int e = amax == 0.0f ? 0 : (int)std::floor(std::log2((double)amax)) - 2;
      if (e + 127 < 0 || e + 127 > 254) bad = 1;
      scale_bytes[r * (d / 32) + b0 / 32] = (uint8_t)(e + 127);
      const double X = std::ldexp(1.0, e);
      for (int c = b0; c < b0 + 32; ++c) {
        int mag = 0;
        const double g = fmt == LB_MXFP4 ? to_grid(xr[c] / X, e2m1_value, 8, &mag)
                                         : to_grid(xr[c] / X, e2m3_value, 32, &mag);
        codes[r * d + c] = (uint8_t)((xr[c] < 0.0f && mag != 0 ? sign_bit : 0) | mag);
        values[r * d + c] = mag == 0 ? 0.0 : g * X;
      }
    }
  return bad ? -1 : 0;
}

// Threads the oracle's OpenMP loops use from now on (n >= 1).
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"

// Internal device/host helpers of libattn_q (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/attn_q.h"

namespace attnq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// -------------------------------------------------------------- numerics ---
// Symmetric int8 code of x for scale s: round-to-nearest-even of the IEEE fp32
// quotient, clamped to [-127, 127]; a zero scale gives 0.
__device__ __forceinline__ int quant_i8(float x, float s) {
  float r = __builtin_rintf(x / s);           // (a zero scale is selected away below)
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return s == 0.0f ? 0 : (int)r;
}

// The same code from rs = fp32(1 / s) (an IEEE division done once per scale): q = x * rs,
// then one correction with the exact residual, q' = fma(fma(-q, s, x), rs, q).  With rs the
// correctly rounded reciprocal and q within an ulp of x / s, q' is the correctly rounded
// quotient (Markstein's theorem; no overflow or underflow can occur for |x| <= 127.5 * s
// and s a normal number), so the code equals quant_i8's.
__device__ __forceinline__ int quant_i8_rcp(float x, float s, float rs) {
  const float q0 = x * rs;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), rs, q0);
  float r = __builtin_rintf(q);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return s == 0.0f ? 0 : (int)r;
}

// fp16 bits -> the exact integer h * 2^24 (every fp16 value is a multiple of 2^-24, and
// |h| * 2^24 < 2^40, so sums of up to 2^23 of them are exact in int64)
__device__ __forceinline__ long long f16_times_2p24(uint16_t h) {
  const int e = (h >> 10) & 31, f = h & 1023;
  const long long mag = e == 0 ? (long long)f : (long long)(1024 + f) << (e - 1);
  return (h & 0x8000) ? -mag : mag;
}

// Mean of n keys from their exact fixed-point sum: fp32(S / (n * 2^24)), the fp64
// conversion and division IEEE-rounded (the value both quantizers shift K by).
__device__ __forceinline__ float mean_from_sum(long long S, long long n) {
  return (float)((double)S / ((double)n * 16777216.0));
}

// One appended token's row, 8 channels per lane on LPR consecutive lanes (LPR = d / 8): the
// key is shifted by the mean of the n keys before it (S: their exact int64 sum of k * 2^24,
// advanced here by this key), per-token fp16 scales s = fp16(amax / 127), codes by
// quant_i8_rcp; kw / vw hold the lane's 8 K / V code bytes.
template <int LPR>
__device__ __forceinline__ void append_row(const uint16_t *kh, const uint16_t *vh, long long (&S)[8], int n,
                                           uint32_t (&kw)[2], uint32_t (&vw)[2], __half &ksh, __half &vsh) {
  float kx[8], vx[8], ka = 0.0f, va = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float mu = n > 0 ? mean_from_sum(S[e], n) : 0.0f;
    kx[e] = __half2float(__ushort_as_half(kh[e])) - mu;
    vx[e] = __half2float(__ushort_as_half(vh[e]));
    S[e] += f16_times_2p24(kh[e]);
    ka = fmaxf(ka, fabsf(kx[e]));
    va = fmaxf(va, fabsf(vx[e]));
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    ka = fmaxf(ka, __shfl_xor(ka, m));
    va = fmaxf(va, __shfl_xor(va, m));
  }
  ksh = __float2half_rn(ka / 127.0f);
  vsh = __float2half_rn(va / 127.0f);
  const float ks = __half2float(ksh), vs = __half2float(vsh);
  const float krs = 1.0f / ks, vrs = 1.0f / vs;
  kw[0] = kw[1] = vw[0] = vw[1] = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kw[e / 4] |= (uint32_t)(quant_i8_rcp(kx[e], ks, krs) & 0xFF) << (8 * (e % 4));
    vw[e / 4] |= (uint32_t)(quant_i8_rcp(vx[e], vs, vrs) & 0xFF) << (8 * (e % 4));
  }
}

// The same code with the zero-scale case folded into the reciprocal: rs = fp32(1 / s) for
// s != 0 and rs = 0 for s == 0 (then q = 0 for any finite x).  The clamp to [-127, 127] before
// rounding equals the clamp after it (the bounds are integers).  quant_i8_val returns the
// code as an fp32 integer value (+0 for zero); quant_i8_byte returns its two's-complement low byte, the
// low byte of fp32(v + 1.5 * 2^23), whose add rounds v to nearest-even (|v| <= 127 lies in
// the binade where one ulp of the sum is 1).
__device__ __forceinline__ float quant_i8_q(float x, float s, float rs) {
  const float q0 = x * rs;
  return __builtin_amdgcn_fmed3f(__builtin_fmaf(__builtin_fmaf(-q0, s, x), rs, q0), -127.0f, 127.0f);
}
__device__ __forceinline__ float quant_i8_val(float x, float s, float rs) {
  return __builtin_rintf(quant_i8_q(x, s, rs)) + 0.0f;   // (+ 0: a code of zero is +0, never -0)
}
__device__ __forceinline__ uint32_t quant_i8_byte(float x, float s, float rs) {
  return __float_as_uint(quant_i8_q(x, s, rs) + 12582912.0f) & 0xFFu;
}
// rs for quant_i8_q: 0 for a zero scale
__device__ __forceinline__ float rcp_or_zero(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

// Two fp32 -> two OCP e4m3 bytes (round-to-nearest-even) in the low (hi=false)
// or high 16 bits of `old` (v_cvt_pk_fp8_f32).
template <bool HI>
__device__ __forceinline__ int cvt_pk_e4m3(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held by lane l^32 (v_permlane32_swap: after swapping the
// upper half of the first operand with the lower half of the second, each lane sees its
// own value in one result and its partner's in the other).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int max_xor32(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order-preserving 32-bit key of an fp16 bit pattern (larger value -> larger key).
__device__ __forceinline__ uint32_t f16_order_key(uint16_t h) {
  return (h & 0x8000u) ? (uint32_t)(~h & 0xFFFFu) : (uint32_t)(h | 0x8000u);
}
__device__ __forceinline__ float f16_from_order_key(uint32_t key) {
  uint16_t h = (key & 0x8000u) ? (uint16_t)(key & 0x7FFFu) : (uint16_t)(~key & 0xFFFFu);
  return __half2float(__ushort_as_half(h));
}

// Per-token V operand of the fp8 PV product: codes scaled by f_n = fp32(s_V[n] * c_V) with
// c_V = fp32(448 / fp32(127 * V_max)) (V_max = the largest per-token scale of the head, the
// cache header), so every |code * f_n| <= 448 and P keeps its static scale; the output is
// multiplied back by fp32(1 / c_V).  A zero V_max (all V zero) gives c_V = 0 and gain 0.
__device__ __forceinline__ float token_v_factor(float vmax) {
  return vmax > 0.0f ? 448.0f / (127.0f * vmax) : 0.0f;
}
__device__ __forceinline__ float token_v_gain(float vmax) {
  const float cv = token_v_factor(vmax);
  return cv > 0.0f ? 1.0f / cv : 0.0f;
}

// fp32(sm_scale * log2 e) computed in fp64 and rounded once; sm_scale <= 0 -> 1/sqrt(d).
inline float host_kconst(float sm_scale, int d) {
  double sm = sm_scale > 0.0f ? (double)sm_scale : 1.0 / __builtin_sqrt((double)d);
  return (float)(sm * 1.4426950408889634074);
}

// Work item id -> XCD-grouped linear index.  Workgroups are dispatched round-robin
// over the 8 XCDs (bid % 8), so giving consecutive linear indices to one XCD keeps
// workgroups that share K/V tiles on the same L2.  grid must be a multiple of 8.
__device__ __forceinline__ int xcd_linear(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace attnq

// ------------------------------------------------------------- launchers ---
// Internal launch entry points (one per source file); arguments already validated.
struct KvqLaunch {
  int B, H, N, D, cap;
  const uint16_t *k, *v;
  int subtract_mean, k_gran, v_gran;
  int8_t *k_codes, *v_codes;
  void *k_scales, *v_scales;
  float *k_mean;
  int64_t *k_sum;
  uint8_t *v_op;
  int v_op_format;
  float *v_scale_max;
  void *ws;
};
hipError_t launch_kv_quantize(const KvqLaunch &a, hipStream_t s);
size_t kvq_workspace_bytes(int B, int H, int D);

struct VopLaunch {
  int B, H, D, cap, n_keys;
  const int8_t *v_codes;
  const void *v_scales;
  int v_gran, fmt;
  uint8_t *v_op;
  float *v_scale_max;
};
hipError_t launch_v_operand(const VopLaunch &a, hipStream_t s);

struct KvAppendLaunch {
  int B, H, D, cap, n_before, T;
  const uint16_t *k, *v;
  int64_t *k_sum;
  int8_t *k_codes, *v_codes;
  uint16_t *k_scales, *v_scales;
  float *k_mean;
  void *ws;
};
hipError_t launch_kv_append(const KvAppendLaunch &a, hipStream_t s);
size_t kv_append_workspace_bytes(int B, int H, int D, int T);

struct ShortLaunch {
  int B, H, N, D;
  float kconst;
  const uint16_t *q, *k, *v;
  void *out;
  int out_f32;
  int32_t *debug_s;
};
hipError_t launch_short_fused(const ShortLaunch &a, hipStream_t s);

struct PrefillLaunch {
  int B, Hq, Hkv, D, q_len, kv_len, q_offset, causal, cap;
  float kconst;
  const uint16_t *q;
  int q_gran;
  const int8_t *k_codes;
  const void *k_scales;           // CHANNEL fp32 [B][Hkv][d], TENSOR fp32 [1], TOKEN fp16 [B][Hkv][cap],
                                  // BLOCK fp32 [B][Hkv][cap / 64]
  int k_gran;
  const uint8_t *v_op;
  const float *v_scales;
  int v_gran;
  const float *v_scale_max;
  int pv_mode;
  void *out;
  int out_f32;
  float *lse;
  int32_t *debug_s;
  uint8_t *debug_p;
  void *ws;
};
hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t s);
hipError_t launch_prefill_split24(const PrefillLaunch &a, hipStream_t s);
size_t prefill_workspace_bytes(int q_gran, int B, int Hq, int q_len);

struct KMxLaunch {
  int BH, N, D, cap, fmt;
  const uint16_t *k;
  const float *k_mean;
  uint8_t *k_mx, *k_sc;
};
hipError_t launch_k_mx(const KMxLaunch &a, hipStream_t s);

struct PrefillMxLaunch {
  int B, Hq, Hkv, D, q_len, kv_len, q_offset, causal, cap, q_fmt, k_fmt, out_f32;
  float kconst;
  const uint16_t *q;
  const uint8_t *k_mx, *k_sc, *v_op;
  const float *v_scales;
  void *out;
  float *debug_s;
};
hipError_t launch_prefill_mx(const PrefillMxLaunch &a, hipStream_t s);

// (pointers first: no padding, the smallest kernel-argument block -- its size measurably
// changes the launch cost of a 15-microsecond kernel)
struct DecodeLaunch {
  const uint16_t *q;
  const int8_t *k_codes;
  const void *k_scales;
  const int8_t *v_codes;
  const void *v_scales;
  void *out;
  int32_t *debug_qk;
  void *ws;
  const int32_t *kv_lens;   // optional: keys of each batch row (device); kv_len is their maximum
  int B, Hq, Hkv, D, kv_len, cap;
  int flags;                // kDecKTok | kDecVTok | kDecOutF32 | kDecKBlk
  float kconst;
};
constexpr int kDecKTok = 1, kDecVTok = 2, kDecOutF32 = 4, kDecKBlk = 8;
// fused one-token append: fp16 k, v [B][Hkv][D] of key kv_len - 1, the int64 K-sum header
// [B][Hkv][D], the optional fp32 mean output [B][Hkv][D], and the cache (writable) for the row
struct DecodeAppendLaunch {
  const uint16_t *k, *v;
  long long *k_sum;
  float *k_mean;
  int8_t *k_codes, *v_codes;
  __half *k_scales, *v_scales;
};
hipError_t launch_decode(const DecodeLaunch &a, const DecodeAppendLaunch *app, hipStream_t s);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D, int kv_len);
// the static scratch of attn_q_decode_noalloc: its size, and its address on the current device
size_t decode_scratch_bytes();
hipError_t decode_scratch_ptr(void **out);

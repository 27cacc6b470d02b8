// Q and K below 8 bits: MX operands on gfx950's scaled f8f6f4 matrix cores.
//
// "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8" closes on the question
// whether Q and K survive four bits.  gfx950 has no int4 matrix-core instruction; its
// v_mfma_scale_f32_32x32x64_f8f6f4 takes fp6 (E2M3) and fp4 (E2M1) operands with one E8M0
// scale per lane, and each lane feeds one block of 32 consecutive k-elements -- exactly the
// block of the OCP MX formats (Microscaling Formats v1.0).  Here Q and K are encoded in MX
// (K after the cache's per-channel mean shift), QK^T runs on that instruction with the
// block scales applied by the matrix core, and the softmax, P and PV steps are those of
// attn_q_prefill (e4m3 P with static scale 448, fp8 PV on the cache's V operand).
//
// Encoding of a block of 32 values x: X = 2^e, e = floor(log2 amax) - 2 (0 for a zero block),
// stored as the E8M0 byte 127 + e; each element is x / X (exact) rounded on the element grid
// to nearest, ties to even, saturating at the largest magnitude.  On the grid the spacing is
// 2^-mbits below 2 and doubles in [2, 4) and [4, 8), so the rounding is one rint of a / step
// (exact power-of-two scaling), and an even multiple of the step is an even code.
#include "common.h"

using namespace attnq;

namespace {

constexpr int KT = ATTN_Q_KEY_TILE;   // 64 keys per online-softmax step
constexpr int kStreams = ATTN_Q_KEY_STREAMS;   // key streams per row block (tile t to stream t % 2)
constexpr int kRowWaves = 4;                    // waves per stream, 32 query rows each
constexpr int kThreads = kStreams * kRowWaves * 64;
constexpr int kRowsPerWG = kRowWaves * 32;
static_assert(kStreams == 2, "the merge below combines two streams");
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448) rounded once to fp32

template <int F>
struct MxFmt;
template <>
struct MxFmt<ATTN_Q_MX_FP4> {   // E2M1
  static constexpr int bits = 4, mbits = 1;
  static constexpr float top = 6.0f;
};
template <>
struct MxFmt<ATTN_Q_MX_FP6> {   // E2M3
  static constexpr int bits = 6, mbits = 3;
  static constexpr float top = 7.5f;
};

// the block's shared exponent e = floor(log2 amax) - 2 (amax = 0: 0), within the E8M0 range
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (amax == 0.0f) return 0;
  int E;
  (void)frexpf(amax, &E);   // amax = f * 2^E, f in [0.5, 1)
  return max(E - 3, -127);
}

// code of x / 2^e: sign bit (negative x with a nonzero magnitude) | exponent field | mantissa
template <int F>
__device__ __forceinline__ uint32_t mx_code(float x, int e) {
  using M = MxFmt<F>;
  const float a = fabsf(ldexpf(x, -e));
  // the grid step is 2^(k - mbits) with k the binade of a (0, 1 or 2): a / step and
  // rint(.) * step are exact power-of-two scalings, written as ldexp (no division)
  const int k = a < 2.0f ? 0 : (a < 4.0f ? 1 : 2);
  const float r = fminf(ldexpf(rintf(ldexpf(a, M::mbits - k)), k - M::mbits), M::top);
  uint32_t mag;
  if (r < 1.0f) {
    mag = (uint32_t)(r * (float)(1 << M::mbits));                 // exponent field 0
  } else {
    const int E = (__float_as_int(r) >> 23) - 127;                 // 0, 1 or 2
    mag = ((uint32_t)(E + 1) << M::mbits) | (uint32_t)((ldexpf(r, -E) - 1.0f) * (float)(1 << M::mbits));
  }
  return ((x < 0.0f && mag != 0) ? (1u << (M::bits - 1)) : 0u) | mag;
}

// MX encoding of 32 values: packed codes (element c at bits [bits*c, bits*c + bits) of the
// little-endian words) and the E8M0 byte
template <int F>
__device__ __forceinline__ uint32_t mx_encode32(const float (&x)[32], uint32_t (&w)[MxFmt<F>::bits]) {
  constexpr int bits = MxFmt<F>::bits;
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(x[c]));
  const int e = mx_block_exp(amax);
#pragma unroll
  for (int i = 0; i < bits; ++i) w[i] = 0u;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const uint32_t code = mx_code<F>(x[c], e);
    const int bit = bits * c, wd = bit >> 5, sh = bit & 31;
    w[wd] |= code << sh;
    if (sh + bits > 32) w[wd + 1] |= code >> (32 - sh);
  }
  return (uint32_t)(e + 127);
}

__device__ __forceinline__ void halves32(const uint16_t *src, float (&x)[32]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const v4i r = *(const v4i *)(src + 8 * u);
    const uint16_t *hv = (const uint16_t *)&r;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[8 * u + e] = __half2float(__ushort_as_half(hv[e]));
  }
}

// ---------------------------------------------------------------- K encoding --
// one thread per (row, 32-channel block): x = fp32(k) - mu, encoded
template <int F, int D>
__global__ __launch_bounds__(256) void k_mx_kernel(const uint16_t *__restrict__ k, const float *__restrict__ k_mean,
                                                  int N, int cap, unsigned total, uint8_t *__restrict__ k_mx,
                                                  uint8_t *__restrict__ k_sc) {
  constexpr int NB = D / 32, bits = MxFmt<F>::bits, RB = D * bits / 8;
  const unsigned gid = blockIdx.x * 256u + threadIdx.x;
  if (gid >= total) return;
  const int blk = gid % NB;
  const unsigned row = gid / NB;   // bg * N + n
  const int n = row % N;
  const unsigned bg = row / N;
  float x[32];
  halves32(k + (size_t)row * D + blk * 32, x);
  const float *mu = k_mean + (size_t)bg * D + blk * 32;
#pragma unroll
  for (int c = 0; c < 32; ++c) x[c] = x[c] - mu[c];
  uint32_t w[bits];
  const uint32_t sb = mx_encode32<F>(x, w);
  uint8_t *dst = k_mx + ((size_t)bg * cap + n) * RB + blk * 4 * bits;
  if constexpr (bits == 4) {
    *(v4i *)dst = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  } else {   // 24 bytes at an 8-byte aligned offset
#pragma unroll
    for (int i = 0; i < 3; ++i) *(uint2 *)(dst + 8 * i) = make_uint2(w[2 * i], w[2 * i + 1]);
  }
  k_sc[((size_t)bg * cap + n) * NB + blk] = (uint8_t)sb;
}

// ----------------------------------------------------------------- prefill --
// A workgroup of 8 waves owns 128 consecutive query positions of one (batch, head): waves
// w and w + 4 hold the same 32 positions, one per lane pair (l, l ^ 32), and run the two key
// streams (even / odd tiles, as attn_q_prefill), merged at the end through LDS by the
// log-sum-exp rule.  S^T = K * Q^T on the scaled MFMA: lane l
// feeds key l % 32 of a 32-key block (A) and query l % 32 (B), channels 64*ch + 32*(l/32) ..
// +32 -- one MX block each, with its scale byte.  The accumulator holds, for query l % 32,
// keys 8*(q/4) + 4*(l/32) + q%4 of the block (element q), so the row max and the row sum
// need one exchange with lane l ^ 32, and the e4m3 P words are the B operand of the 64-deep
// fp8 PV product in the byte order of the cache's V operand.  Each stream takes its tiles
// in ascending order.  K and V operands are read straight from HBM / L2 into registers (the
// next tile's K while the current tile is processed).
template <int D, int KF, int QF>
struct MxOps {
  static constexpr int NC = D / 64;                       // 64-deep steps per score
  static constexpr int KW = MxFmt<KF>::bits;              // words per K operand
  static constexpr int QW = MxFmt<QF>::bits;
  static constexpr int RB = D * MxFmt<KF>::bits / 8;      // bytes per K row
};

template <int D, int KF>
__device__ __forceinline__ void load_k(const uint8_t *kbase, const uint8_t *sbase, int t, int n32, int hh,
                                       v8i (&kop)[2][D / 64], int (&ksc)[2][D / 64]) {
  constexpr int NC = D / 64, bits = MxFmt<KF>::bits, RB = D * bits / 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = t * KT + 32 * j + n32;
    const uint8_t *row = kbase + (size_t)n * RB;
    uint32_t sw;
    if constexpr (D == 128) sw = *(const uint32_t *)(sbase + (size_t)n * 4);
    else sw = *(const uint16_t *)(sbase + (size_t)n * 2);
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
      const int blk = 2 * ch + hh;
      const uint8_t *p = row + blk * 4 * bits;
      v8i o = v8i{};
      if constexpr (bits == 4) {
        const v4i r = *(const v4i *)p;
        o[0] = r[0]; o[1] = r[1]; o[2] = r[2]; o[3] = r[3];
      } else {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const uint2 r = *(const uint2 *)(p + 8 * i);
          o[2 * i] = (int)r.x; o[2 * i + 1] = (int)r.y;
        }
      }
      kop[j][ch] = o;
      ksc[j][ch] = (int)((sw >> (8 * blk)) & 0xFFu);
    }
  }
}

template <int D, int KF, int QF>
__global__ __launch_bounds__(kThreads) void prefill_mx_kernel(const PrefillMxLaunch a) {
  using Ops = MxOps<D, KF, QF>;
  constexpr int NC = Ops::NC, NM = D / 32;
  const int lane = threadIdx.x & 63, wv = (threadIdx.x >> 6) % kRowWaves, st = (threadIdx.x >> 6) / kRowWaves;
  const int n32 = lane & 31, hh = lane >> 5;
  // Workgroup order: each XCD (workgroups are dealt to the 8 XCDs round-robin) takes a run of
  // consecutive (head, position block) items, so the query heads of one kv-head group share
  // that XCD's L2; within a head the later (causal: heavier) position blocks go first.
  const int npos = (a.q_len + kRowsPerWG - 1) / kRowsPerWG;
  const int lin = gridDim.x % 8 == 0 ? xcd_linear(blockIdx.x, gridDim.x) : blockIdx.x;
  const int bh = lin / npos, pb = npos - 1 - lin % npos;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const size_t bg = (size_t)b * a.Hkv + h / (a.Hq / a.Hkv);
  const int i0 = min(pb * kRowsPerWG + wv * 32, a.q_len - 1);   // (a wave past the end
  const bool wave_ok = pb * kRowsPerWG + wv * 32 < a.q_len;    //  runs no tile)
  const int i = i0 + n32;
  const bool row_ok = wave_ok && i < a.q_len;
  const int last = row_ok ? (a.causal ? min(a.kv_len, a.q_offset + i + 1) : a.kv_len) : 1;
  const int wlast = a.causal ? min(a.kv_len, a.q_offset + min(i0 + 31, a.q_len - 1) + 1) : a.kv_len;
  const int ntiles = wave_ok ? (wlast + KT - 1) / KT : 0;
  // the smallest bound of the wave's valid rows (its first row's); rows past q_len see any
  // key (their results are not stored)
  const int last_min = a.causal ? min(a.kv_len, a.q_offset + i0 + 1) : a.kv_len;

  // Q: the lane's row, blocks 2*ch + hh, as the B operand
  v8i qop[NC];
  int qsc[NC];
  {
    const uint16_t *qrow = a.q + ((size_t)bh * a.q_len + (row_ok ? i : 0)) * D;
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
      float x[32];
      halves32(qrow + (2 * ch + hh) * 32, x);
      uint32_t w[Ops::QW];
      qsc[ch] = (int)mx_encode32<QF>(x, w);
      v8i o = v8i{};
#pragma unroll
      for (int u = 0; u < Ops::QW; ++u) o[u] = (int)w[u];
      qop[ch] = o;
    }
  }

  // e4m3 1.0 where output row block (l%16)/4 and key block l/16 have the same parity: one
  // 16x16x128 MFMA over the P registers then gives every lane its query's row sum
  const int one = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x38383838 : 0;
  const v8i ones = v8i{one, one, one, one, one, one, one, one};

  const uint8_t *kbase = a.k_mx + bg * a.cap * Ops::RB;
  const uint8_t *sbase = a.k_sc + bg * a.cap * (D / 32);
  const uint8_t *vbase = a.v_op + bg * (size_t)(a.cap / KT) * D * KT;
  const float c = a.kconst;
  float m = -INFINITY, l = 0.0f;
  v16f O[NM];
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) O[mt] = v16f{};
  v8i kop[2][NC], knx[2][NC];
  int ksc[2][NC], ksn[2][NC];
  auto tile = [&](int t) {
    if (t + kStreams < ntiles) load_k<D, KF>(kbase, sbase, t + kStreams, n32, hh, knx, ksn);
    v8i vop[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      const uint8_t *p = vbase + ((size_t)t * D + 32 * mt + n32) * KT + 32 * hh;
      const v4i lo = *(const v4i *)p, hi = *(const v4i *)(p + 16);
      vop[mt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    v16f S[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S[j] = v16f{};
#pragma unroll
      for (int ch = 0; ch < NC; ++ch)
        S[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[j][ch], qop[ch], S[j], KF, QF, 0, ksc[j][ch], 0,
                                                               qsc[ch]);
    }
    if (a.debug_s != nullptr) {   // (uniform: the scores of the visible pairs)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int key = t * KT + 32 * j + 8 * (q >> 2) + 4 * hh + (q & 3);
          if (key < last && row_ok) a.debug_s[((size_t)bh * a.q_len + i) * a.kv_len + key] = S[j][q];
        }
    }
    // visible keys (a tile below every valid row's bound needs no mask), the tile's row max
    // (the partner lane holds the other half of the keys)
    if ((t + 1) * KT > last_min) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int key = t * KT + 32 * j + 8 * (q >> 2) + 4 * hh + (q & 3);
          S[j][q] = key < last ? S[j][q] : -INFINITY;
        }
    }
    float smax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) smax = fmaxf(smax, S[j][q]);
    smax = max_xor32(smax);
    const float mnew = fmaxf(m, c * smax);
    const float alpha = mnew == m ? 1.0f : fast_exp2(m - mnew);
    const bool moved = __any(mnew != m);
    m = mnew;
    // (a row that has seen no visible key in this stream keeps m = -inf: its p are 0)
    const float negmL = m == -INFINITY ? -INFINITY : kLog2_448 - m;
    // p = exp2(fp32(c * s - mL)) (one rounding) to e4m3, packed as the PV B operand
    v8i P;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int j = w >> 2, r0 = (w & 3) * 4;
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = fast_exp2(__builtin_fmaf(c, S[j][r0 + u], negmL));
      const int lo = cvt_pk_e4m3<false>(p[0], p[1], 0);
      P[w] = cvt_pk_e4m3<true>(p[2], p[3], lo);
    }
    const float rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P, v4f{}, 0, 0, 0, 0, 0, 0)[0];
    l = l * alpha + rs;
    if (moved) {
      asm volatile("" ::: "memory");   // (keeps the branch: 64 multiplies skipped when no row moved)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) O[mt] *= alpha;
    }
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
      O[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mt], P, O[mt], 0, 0, 0, 0, 0, 0);
  };
  if (st < ntiles) load_k<D, KF>(kbase, sbase, st, n32, hh, kop, ksc);
  for (int t = st; t < ntiles; t += kStreams) {
    tile(t);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ch = 0; ch < NC; ++ch) { kop[j][ch] = knx[j][ch]; ksc[j][ch] = ksn[j][ch]; }
  }
  // merge the streams: M = max(m0, m1), O = sum_s 2^(m_s - M) O_s, l likewise (stream 1
  // hands its state over through LDS, lane-major so the accesses are conflict-free)
  __shared__ float s_x[kRowWaves][2 + D / 2][64];   // m, l, the 16 * D / 32 O values
  if (st == 1) {
    s_x[wv][0][lane] = m;
    s_x[wv][1][lane] = l;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
      for (int q = 0; q < 16; ++q) s_x[wv][2 + 16 * mt + q][lane] = O[mt][q];
  }
  __syncthreads();
  if (st == 1 || !row_ok) return;
  {
    const float m1 = s_x[wv][0][lane], l1 = s_x[wv][1][lane];
    const float M = fmaxf(m, m1);
    const float f0 = m == M ? 1.0f : fast_exp2(m - M), f1 = m1 == M ? 1.0f : fast_exp2(m1 - M);
    l = f0 * l + f1 * l1;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
      for (int q = 0; q < 16; ++q) O[mt][q] = f0 * O[mt][q] + f1 * s_x[wv][2 + 16 * mt + q][lane];
  }
  // out_c = O_c * s_V[c] / l; the lane holds channels 32*mt + 8*g + 4*(l/32) + 0..3
  const float rl = l > 0.0f ? 1.0f / l : 0.0f;
  const float *vs = a.v_scales + bg * D;
#pragma unroll
  for (int mt = 0; mt < NM; ++mt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ch0 = 32 * mt + 8 * gq + 4 * hh;
      const v4f s4 = *(const v4f *)(vs + ch0);
      float o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = O[mt][4 * gq + u] * s4[u] * rl;
      const size_t off = ((size_t)bh * a.q_len + i) * D + ch0;
      if (a.out_f32) {
        *(v4f *)((float *)a.out + off) = v4f{o[0], o[1], o[2], o[3]};
      } else {
        __half2 h01 = __floats2half2_rn(o[0], o[1]), h23 = __floats2half2_rn(o[2], o[3]);
        *(uint2 *)((__half *)a.out + off) = make_uint2(*(uint32_t *)&h01, *(uint32_t *)&h23);
      }
    }
}

template <int D, int KF>
hipError_t launch_k_d(const KMxLaunch &a, hipStream_t s) {
  const unsigned total = (unsigned)((size_t)a.BH * a.N * (D / 32));
  hipLaunchKernelGGL((k_mx_kernel<KF, D>), dim3((total + 255) / 256), dim3(256), 0, s, a.k, a.k_mean, a.N, a.cap,
                     total, a.k_mx, a.k_sc);
  return hipGetLastError();
}

template <int D, int KF, int QF>
hipError_t launch_p(const PrefillMxLaunch &a, hipStream_t s) {
  const unsigned nwg = (unsigned)((a.q_len + kRowsPerWG - 1) / kRowsPerWG) * (unsigned)(a.B * a.Hq);
  hipLaunchKernelGGL((prefill_mx_kernel<D, KF, QF>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_p_d(const PrefillMxLaunch &a, hipStream_t s) {
  if (a.k_fmt == ATTN_Q_MX_FP4)
    return a.q_fmt == ATTN_Q_MX_FP4 ? launch_p<D, ATTN_Q_MX_FP4, ATTN_Q_MX_FP4>(a, s)
                                    : launch_p<D, ATTN_Q_MX_FP4, ATTN_Q_MX_FP6>(a, s);
  return a.q_fmt == ATTN_Q_MX_FP4 ? launch_p<D, ATTN_Q_MX_FP6, ATTN_Q_MX_FP4>(a, s)
                                  : launch_p<D, ATTN_Q_MX_FP6, ATTN_Q_MX_FP6>(a, s);
}

}  // namespace

hipError_t launch_k_mx(const KMxLaunch &a, hipStream_t s) {
  if (a.D == 128) return a.fmt == ATTN_Q_MX_FP4 ? launch_k_d<128, ATTN_Q_MX_FP4>(a, s) : launch_k_d<128, ATTN_Q_MX_FP6>(a, s);
  return a.fmt == ATTN_Q_MX_FP4 ? launch_k_d<64, ATTN_Q_MX_FP4>(a, s) : launch_k_d<64, ATTN_Q_MX_FP6>(a, s);
}

hipError_t launch_prefill_mx(const PrefillMxLaunch &a, hipStream_t s) {
  if (a.q_len == 0) return hipSuccess;
  return a.D == 128 ? launch_p_d<128>(a, s) : launch_p_d<64>(a, s);
}

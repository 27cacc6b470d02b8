// attn_q_prefill, pv_mode ATTN_Q_PV_SPLIT24: the precision mode.  K and V stay the int8
// codes of the cache and both products run on the int8 matrix core; the other operand of
// each product is split into three exact 8-bit parts (24 bits), each part's int32 sum is
// exact and the parts are combined in fp32 -- the operand split of the "Strata" int8-KV
// prompt attention, whose error against fp64 is a few 1e-6.  The online softmax is the
// fp32 one of the other modes (running max, exp2 with log2(e) folded into the constant).
//
// Per row (query i of head h, kv-head g):
//   q' = fp32(q) * s_K[c] (K CHANNEL) or fp32(q); s_Q = fp32(amax(q') / 127);
//   X_c = clamp(rint(q'_c / s_Q * 2^16), +-127 * 2^16) = 2^16 h_c + 2^8 l_c + m_c with signed
//   bytes m_c, l_c in [-128, 127] (balanced digits) and h_c;
//   per key j: A_d = sum_c d_c k_jc (exact int32, d = h, l, m);
//   t_j = fp32(fp32(A_h + A_l * 2^-8) + A_m * 2^-16)  (~ sum_c X_c k_jc / 2^16);
//   s_j = c * t_j, c = fp32(s_Q * kconst) (K CHANNEL) or fp32(fp32(s_Q * kconst) * s_K);
//   online softmax per 64-key tile: m = max(m, max_j s_j), p_j = exp2(s_j - m) <= 1;
//   per (row, tile) scale p_max = max_j p_j = exp2(c * max_j t_j - m);
//   W_j = rint(p_j / p_max * 127 * 2^16) = 2^16 h_j + 2^8 l_j + m_j (balanced digits);
//   per channel: B_d = sum_j d_j v_jc (exact int32), O += (B_h + B_l 2^-8 + B_m 2^-16) p_max,
//   l += (sum_j W_j) 2^-16 p_max (both rescaled by 2^(m_old - m) when m moves; O and l carry
//   the same factor 127, which cancels; both are carried across tiles in fp64);
//   out_c = O_c * s_V[c] / l.
// gfx950 mapping: 4 waves x 32 query rows per workgroup (rows position-major across the G
// heads of a kv-head, as the fp8 kernel); 64-key K and V tiles double-buffered in LDS with
// the next tile's global loads in flight during the current tile's work; S^T = K Q^T and
// O^T = V^T P^T on v_mfma_i32_32x32x32_i8, three digit passes each.  The V operand is the
// int8 PV operand of kv_quantize_i8 (v_op_format ATTN_Q_PV_INT8).
#include <climits>

#include "common.h"

using namespace attnq;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerWG = 128;
constexpr int KT = 64;

template <int D>
struct SplitLds {
  static constexpr int KSTR = D + 16;          // K code row stride: 16-byte reads of consecutive
                                               // rows start on different banks
  static constexpr int VSTR = KT + 16;         // V operand row stride
  static constexpr int KB = KT * KSTR, VB = D * VSTR;
  static constexpr int BUF = KB + VB;
  static constexpr int KCH = KT * D / 16;      // 16-byte chunks per K tile
  static constexpr int VCH = D * KT / 16;      // ... per V tile
  static constexpr int KU = KCH / kThreads, VU = VCH / kThreads;
  static_assert(KCH % kThreads == 0 && VCH % kThreads == 0, "whole chunks per thread");
};

// x (an integer-valued fp32 with |x| < 2^24) -> balanced base-256 digits: x = 2^16 h + 2^8 l + m
__device__ __forceinline__ void digits3(int x, int &h, int &l, int &m) {
  m = (int)(int8_t)(x & 0xFF);
  const int x1 = (x - m) >> 8;
  l = (int)(int8_t)(x1 & 0xFF);
  h = (x1 - l) >> 8;
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_split24_kernel(PrefillLaunch a, int nblk, int total) {
  using L = SplitLds<D>;
  constexpr int NK = D / 32;
  __shared__ __align__(16) uint8_t s_buf[2][L::BUF];
  const int Lw = xcd_linear(blockIdx.x, gridDim.x);
  if (Lw >= total) return;
  const int G = a.Hq / a.Hkv;
  const bool causal = a.causal != 0;
  int blk = Lw % nblk;
  const int bg = Lw / nblk;
  if (causal) blk = nblk - 1 - blk;   // heaviest (latest) query blocks first
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int row = blk * kRowsPerWG + wave * 32 + n;
  const int i = row / G, h = g * G + row % G;
  const bool row_valid = i < a.q_len;
  const int iq = row_valid ? i : a.q_len - 1;
  const size_t qrow = ((size_t)b * a.Hq + (row_valid ? h : g * G)) * a.q_len + iq;
  const int8_t *kbase = a.k_codes + (size_t)bg * a.cap * D;
  const uint8_t *vbase = a.v_op + (size_t)bg * (a.cap / KT) * D * KT;

  const int i_wg_hi = min((blk * kRowsPerWG + kRowsPerWG - 1) / G, a.q_len - 1);
  const int kv_end = causal ? min(a.kv_len, a.q_offset + i_wg_hi + 1) : a.kv_len;
  const int ntiles = (kv_end + KT - 1) / KT;
  const int vis_last = min(causal ? a.q_offset + iq : a.kv_len - 1, a.kv_len - 1);   // the lane's row

  // ---- tile staging: 16-byte chunks, K rows of D bytes and V operand rows of 64 bytes
  v4i kreg[L::KU], vreg[L::VU];
  auto load_tile = [&](int tt) {
#pragma unroll
    for (int u = 0; u < L::KU; ++u) {
      const int q = t + u * kThreads;
      kreg[u] = *(const v4i *)(kbase + (size_t)tt * KT * D + q * 16);
    }
#pragma unroll
    for (int u = 0; u < L::VU; ++u) {
      const int q = t + u * kThreads;
      vreg[u] = *(const v4i *)(vbase + (size_t)tt * D * KT + q * 16);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < L::KU; ++u) {
      const int q = t + u * kThreads, r = q / (D / 16), ch = q % (D / 16);
      *(v4i *)(s_buf[buf] + r * L::KSTR + ch * 16) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < L::VU; ++u) {
      const int q = t + u * kThreads, r = q / (KT / 16), ch = q % (KT / 16);
      *(v4i *)(s_buf[buf] + L::KB + r * L::VSTR + ch * 16) = vreg[u];
    }
  };
  load_tile(0);

  // ---- Q: q' = q * s_K, per-row scale, 24-bit value split into three int8 digit operands
  float qf[NK][16];
  float amax = 0.0f;
  const uint16_t *qp = a.q + qrow * D;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const v4i r0 = *(const v4i *)(qp + kk * 32 + hh * 16);
    const v4i r1 = *(const v4i *)(qp + kk * 32 + hh * 16 + 8);
    const uint16_t *h0 = (const uint16_t *)&r0, *h1 = (const uint16_t *)&r1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = __half2float(__ushort_as_half(e < 8 ? h0[e] : h1[e - 8]));
      if (a.k_gran == ATTN_Q_GRAN_CHANNEL) x = x * ((const float *)a.k_scales)[(size_t)bg * D + kk * 32 + hh * 16 + e];
      qf[kk][e] = x;
      amax = fmaxf(amax, fabsf(x));
    }
  }
  amax = max_xor32(amax);
  const float sq = amax / 127.0f, rq = rcp_or_zero(sq);
  float c = sq * a.kconst;
  if (a.k_gran == ATTN_Q_GRAN_TENSOR) c = c * ((const float *)a.k_scales)[0];
  v4i qh[NK], ql[NK], qm[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t wh = 0, wl = 0, wm = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = __builtin_amdgcn_fmed3f(qf[kk][4 * w + e] * rq * 65536.0f, -8323072.0f, 8323072.0f);
        int dh, dl, dm;
        digits3((int)__builtin_rintf(y), dh, dl, dm);
        wh |= (uint32_t)(dh & 0xFF) << (8 * e);
        wl |= (uint32_t)(dl & 0xFF) << (8 * e);
        wm |= (uint32_t)(dm & 0xFF) << (8 * e);
      }
      qh[kk][w] = (int)wh;
      ql[kk][w] = (int)wl;
      qm[kk][w] = (int)wm;
    }

  // O and l carried across tiles in fp64: over thousands of tiles, fp32 rounding of the running
  // sums would dominate the error; each tile's contribution is formed in fp32 (one rounding)
  double O[NK][16];
#pragma unroll
  for (int mt = 0; mt < NK; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[mt][e] = 0.0;
  float m = -INFINITY;
  double l = 0.0;

  store_tile(0);
  __syncthreads();
  for (int tt = 0; tt < ntiles; ++tt) {
    const int buf = tt & 1;
    if (tt + 1 < ntiles) load_tile(tt + 1);
    const uint8_t *sk = s_buf[buf];
    const uint8_t *sv = s_buf[buf] + L::KB;
    // scores t_j for the lane's 32 keys: 64tt + 32j + 8(e>>2) + 4hh + (e&3)
    float ts[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t *kr = sk + (32 * j + n) * L::KSTR + 16 * hh;
      v4i kop[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) kop[kk] = *(const v4i *)(kr + 32 * kk);
      v16i Ah = v16i{}, Al = v16i{}, Am = v16i{};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) Ah = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[kk], qh[kk], Ah, 0, 0, 0);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) Al = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[kk], ql[kk], Al, 0, 0, 0);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) Am = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[kk], qm[kk], Am, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = tt * KT + 32 * j + 8 * (e >> 2) + 4 * hh + (e & 3);
        const float x = __builtin_fmaf((float)Am[e], 1.52587890625e-05f,
                                       __builtin_fmaf((float)Al[e], 0.00390625f, (float)Ah[e]));
        ts[j][e] = key <= vis_last ? x : -INFINITY;
      }
    }
    // online softmax (running max in log2 units)
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, ts[j][e]);
    mx = max_xor32(mx);
    const float mnew = fmaxf(m, mx == -INFINITY ? -INFINITY : c * mx);
    const float alpha = mnew == m ? 1.0f : fast_exp2(m - mnew);   // (0 on the first visible tile)
    m = mnew;
    // weights, scaled per (row, tile) to the tile's largest p (every tile keeps 24 bits):
    // W = rint(p / p_max * 127 * 2^16) split into digits, packed as the PV B operands
    const float pmax = mx == -INFINITY ? 0.0f : fast_exp2(__builtin_fmaf(c, mx, -m));
    const float wscale = pmax > 0.0f ? 8323072.0f / pmax : 0.0f;   // (a tile whose weights all
                                                                    //  underflow adds nothing)
    v8i Ph, Pl, Pm;
    int wsum = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int j = w >> 2, r0 = (w & 3) * 4;
      uint32_t wh = 0, wl = 0, wm = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = ts[j][r0 + e];
        const float p = x == -INFINITY ? 0.0f : fast_exp2(__builtin_fmaf(c, x, -m));
        const int W = (int)__builtin_rintf(p * wscale);
        wsum += W;
        int dh, dl, dm;
        digits3(W, dh, dl, dm);
        wh |= (uint32_t)(dh & 0xFF) << (8 * e);
        wl |= (uint32_t)(dl & 0xFF) << (8 * e);
        wm |= (uint32_t)(dm & 0xFF) << (8 * e);
      }
      Ph[w] = (int)wh;
      Pl[w] = (int)wl;
      Pm[w] = (int)wm;
    }
    wsum += __shfl_xor(wsum, 32);   // the row's other 32 keys
    l = __builtin_fma(l, (double)alpha, (double)wsum * 1.52587890625e-05 * (double)pmax);
#pragma unroll
    for (int mt = 0; mt < NK; ++mt) {
      const uint8_t *vr = sv + (32 * mt + n) * L::VSTR + 32 * hh;
      const v4i v0 = *(const v4i *)vr;
      const v4i v1 = *(const v4i *)(vr + 16);
      v16i Bh = v16i{}, Bl = v16i{}, Bm = v16i{};
      Bh = __builtin_amdgcn_mfma_i32_32x32x32_i8(v0, v4i{Ph[0], Ph[1], Ph[2], Ph[3]}, Bh, 0, 0, 0);
      Bh = __builtin_amdgcn_mfma_i32_32x32x32_i8(v1, v4i{Ph[4], Ph[5], Ph[6], Ph[7]}, Bh, 0, 0, 0);
      Bl = __builtin_amdgcn_mfma_i32_32x32x32_i8(v0, v4i{Pl[0], Pl[1], Pl[2], Pl[3]}, Bl, 0, 0, 0);
      Bl = __builtin_amdgcn_mfma_i32_32x32x32_i8(v1, v4i{Pl[4], Pl[5], Pl[6], Pl[7]}, Bl, 0, 0, 0);
      Bm = __builtin_amdgcn_mfma_i32_32x32x32_i8(v0, v4i{Pm[0], Pm[1], Pm[2], Pm[3]}, Bm, 0, 0, 0);
      Bm = __builtin_amdgcn_mfma_i32_32x32x32_i8(v1, v4i{Pm[4], Pm[5], Pm[6], Pm[7]}, Bm, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = __builtin_fmaf((float)Bm[e], 1.52587890625e-05f,
                                       __builtin_fmaf((float)Bl[e], 0.00390625f, (float)Bh[e]));
        O[mt][e] = __builtin_fma(O[mt][e], (double)alpha, (double)x * (double)pmax);
      }
    }
    if (tt + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O and l carry the same factor 127 (sums of W / 2^16 ~ 127 p)
  if (!row_valid) return;
  const double inv = 1.0 / l;
  const size_t orow = (((size_t)b * a.Hq + h) * a.q_len + i) * D;
  const float *vs = a.v_scales + (size_t)bg * D;
#pragma unroll
  for (int mt = 0; mt < NK; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int ch = mt * 32 + 8 * r4 + 4 * hh;
      float ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (float)(O[mt][4 * r4 + e] * (double)vs[ch + e] * inv);
      if (a.out_f32) {
        *(float4 *)((float *)a.out + orow + ch) = make_float4(ov[0], ov[1], ov[2], ov[3]);
      } else {
        __half2 lo = __floats2half2_rn(ov[0], ov[1]), hi = __floats2half2_rn(ov[2], ov[3]);
        *(uint2 *)((__half *)a.out + orow + ch) = make_uint2(*(uint32_t *)&lo, *(uint32_t *)&hi);
      }
    }
}

}  // namespace

hipError_t launch_prefill_split24(const PrefillLaunch &a, hipStream_t s) {
  if (a.q_len == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  const int nblk = (G * a.q_len + kRowsPerWG - 1) / kRowsPerWG;
  const int total = a.B * a.Hkv * nblk;
  const dim3 grid((total + 7) / 8 * 8);
  if (a.D == 128)
    hipLaunchKernelGGL(prefill_split24_kernel<128>, grid, dim3(kThreads), 0, s, a, nblk, total);
  else
    hipLaunchKernelGGL(prefill_split24_kernel<64>, grid, dim3(kThreads), 0, s, a, nblk, total);
  return hipGetLastError();
}

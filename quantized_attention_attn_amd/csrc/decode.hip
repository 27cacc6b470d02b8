// attn_q_decode: one query per head against the int8 KV cache.
//
// "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8", sections "Does
// quantizing attention help decode?" and "What actually changed for decode": at
// batch one attention is a matrix-vector product bound by how fast the KV cache
// streams from memory, so the matrix cores are not used; halving the cache's bytes
// is what speeds it up.
//
// gfx950 mapping.  One workgroup (8 waves) per (batch, kv-head, split of 512 keys); each
// wave owns 64 consecutive keys and works alone until the end:
//   * all K rows are requested first, then all V rows, so the scores and the softmax run
//     while V is still streaming in;
//   * exact int32 scores on v_mfma_i32_32x32x32_i8, K as the B operand as loaded (a lane
//     holds 16 channels of one key) and the int8 queries of all G heads in the A rows, the
//     wave's two 32-key blocks landing in disjoint accumulator rows, so lane l ends with
//     key l's dots for every head; s = fp32(c_n * acc);
//   * wave-local softmax: max and sums across lanes with DPP and the gfx950 permlane16/32
//     swaps; weights w = p (per-channel V) or p * s_V[n] (per-token V), to fp16 after an
//     exact power-of-two scaling;
//   * PV on v_mfma_f32_16x16x32_f16: the V codes become the exact fp16 values 1152 + code,
//     transposed through the wave's LDS region to one row of keys per channel (the +1152 is
//     removed once per head with the sum of the same fp16 weights); each lane's products
//     are exact and summed in fp32;
//   * the waves' partials meet in LDS; partial (m, l, o) per split go to the workspace and
//     a second small kernel merges them per (batch, kv-head, head).  (Merging inside the
//     first kernel would need a device-scope release/acquire per workgroup, which on a
//     multi-XCD part writes back and invalidates the whole L2 -- far costlier than a kernel
//     boundary.)
#include <atomic>

#include "common.h"

using namespace attnq;

namespace {

constexpr int kThreads = 512;
constexpr int kWavesD = kThreads / 64;
constexpr int KPS = 512;                // keys per split (workgroup)
constexpr int KPW = KPS / kWavesD;      // keys per wave (64)
constexpr int NPASS = KPW / 8;          // passes of 8 rows per wave

typedef _Float16 h8t __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecWs {
  float2 *ml;      // [BH][S][G]  (m, l)
  float *o;        // [BH][S][G][D]
};

__host__ __device__ inline DecWs dec_ws(void *ws, int BH, int G, int D, int S) {
  char *p = (char *)ws;
  DecWs w;
  w.ml = (float2 *)p;
  p += align256((size_t)BH * S * G * 8);
  w.o = (float *)p;
  return w;
}

// ---- cross-lane helpers (lane patterns checked on the device: quad_perm, half-row mirror,
//      row rotate by 8, and the 16- / 32-lane swaps)
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror8(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ float dpp_xor8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_add(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// max / sum over the 8 row groups of a wave (lanes l, l^8, l^16, l^32)
__device__ __forceinline__ float max_groups(float x) {
  x = fmaxf(x, dpp_xor8(x));
  x = swap16_max(x);
  return max_xor32(x);
}
__device__ __forceinline__ float add_groups(float x) {
  x += dpp_xor8(x);
  x = swap16_add(x);
  return add_xor32(x);
}

__device__ __forceinline__ int max_groups_i(int x) {
  x = max(x, __float_as_int(dpp_xor8(__int_as_float(x))));
  const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  return max_xor32(max((int)r[0], (int)r[1]));
}

template <int D, int G, bool APPEND>
__device__ __forceinline__ void decode_body(const DecodeLaunch &a, int S, const DecodeAppendLaunch &ap) {
  constexpr int CH = D / 8;            // V code bytes per lane and row
  constexpr int CW = CH / 4;           // ... in dwords
  constexpr int NK = D / 32;           // 32-channel steps of the QK matrix-core product
  static_assert(NPASS == 8 && G <= 8, "8 keys per row group; heads in accumulator elements 0..7");
  using Row = int __attribute__((ext_vector_type(CW)));
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = lane & 7, r = lane >> 3;          // chunk of the row, row group (PV)
  const int n32 = lane & 31, hh = lane >> 5;      // matrix-core column, k half (QK)
  const int nw = split * KPS + wave * KPW;        // first key of the wave
  const int nr = nw + r * NPASS;                  // first key of the lane's row group
  const int nk = nw + lane;                       // the key whose scores this lane holds

  __shared__ __attribute__((aligned(16))) int8_t s_q8[G][D];
  __shared__ __attribute__((aligned(16))) int s_nk[D / 4], s_nv[D / 4];   // (fused append: the new row)
  __shared__ float s_c[G];
  __shared__ float s_wm[kWavesD][G], s_wl[kWavesD][G], s_ww[kWavesD][G], s_ws[kWavesD][G];
  __shared__ float s_f[kWavesD][G], s_g[kWavesD][G];
  __shared__ __attribute__((aligned(16))) _Float16 s_wh[kWavesD][G][64];
  // per wave: V transposed to fp16 (D rows of 64 keys), then its partial o[h][ch]
  __shared__ __attribute__((aligned(16))) float s_vo[kWavesD][D * 32];

  // ---- loads: q and the lane's key scales first, then every K row, then every V row
  //      (rows past kv_len are clamped to the last row and masked below).  All of them are
  //      unconditional, from addresses that are valid whatever the granularity (the value
  //      is selected after the load): a load inside a branch makes the compiler wait for it
  //      where the branches join, which would hold back the K/V stream by a memory round trip.
  const bool ktok = (a.flags & kDecKTok) != 0, vtok = (a.flags & kDecVTok) != 0;
  const bool kblk = (a.flags & kDecKBlk) != 0;   // K BLOCK: one fp32 scale per 64 keys
  const bool kkey = ktok || kblk;                // a per-key K scale, nothing folded into q
  // keys of this batch row: kv_lens[b] (clamped to [1, kv_len]) or kv_len
  const int kvb = (!APPEND && a.kv_lens) ? min(max(a.kv_lens[b], 1), a.kv_len) : a.kv_len;
  if (split * KPS >= kvb) {
    // a split wholly past the row's keys (ragged batch): an empty partial (m = -inf, l = 0),
    // which the merge skips without reading its o
    if (t < G) dec_ws(a.ws, a.B * a.Hkv, G, D, S).ml[((size_t)bg * S + split) * G + t] = make_float2(-INFINITY, 0.0f);
    return;
  }
  float qx[D / 64], kch[D / 64];
  {
    const uint16_t *qp = a.q + ((size_t)b * a.Hq + g * G + min(wave, G - 1)) * D;   // (waves >= G: unused)
    const float *kcp = (const float *)a.k_scales + (kkey ? 0 : (size_t)bg * D);      // (TOKEN, BLOCK: unused)
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      const int ch = lane * (D / 64) + e;
      qx[e] = __half2float(__ushort_as_half(qp[ch]));
      const float kc = kcp[kkey ? 0 : ch];
      kch[e] = kkey ? 1.0f : kc;
    }
  }
  const bool live = nk < kvb;
  const int nks = min(nk, kvb - 1);
  const __half ksh = ((const __half *)a.k_scales)[ktok ? (size_t)bg * a.cap + nks : 0];   // (CHANNEL: unused)
  const float kbs = ((const float *)a.k_scales)[kblk ? (size_t)bg * (a.cap / 64) + nks / 64 : 0];
  const __half vsh = ((const __half *)a.v_scales)[vtok ? (size_t)bg * a.cap + nks : 0];
  float ksc = ktok ? __half2float(ksh) : (kblk ? kbs : 1.0f);
  float vsc = vtok ? __half2float(vsh) : 1.0f;
  const int8_t *kb = a.k_codes + (size_t)bg * a.cap * D;
  const int8_t *vb = a.v_codes + (size_t)bg * a.cap * D;
  // K as the B operand of S = Q K^T on v_mfma_i32_32x32x32_i8: for the wave's key block blk
  // (32 keys), lane holds key 32*blk + n32, channels 32*kk + 16*hh .. +15
  v4i kop[2][NK];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      kop[blk][kk] = *(const v4i *)(kb + (size_t)min(nw + 32 * blk + n32, kvb - 1) * D + kk * 32 + hh * 16);
  Row vr[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) vr[p] = *(const Row *)(vb + (size_t)min(nr + p, kvb - 1) * D + c * CH);

  // ---- fused one-token append (attn_q_decode_append): the wave holding the new key
  //      n_new = kv_len - 1 computes its row exactly as attn_q_kv_append_i8 does (shift by the
  //      mean of the keys before it, per-token scales), writes it to the cache and the header,
  //      and hands its codes and scales to its own lanes that hold that key.  Its inputs are
  //      requested here, with the K/V stream; nothing else in the workgroup waits for it.
  const int n_new = a.kv_len - 1;
  const bool app = APPEND && split == n_new / KPS && wave == (n_new % KPS) / KPW;   // (uniform)
  const int alane = lane & (D / 8 - 1);   // (every group of D/8 lanes computes the row)
  const size_t h0 = (size_t)bg * D + alane * 8;
  v4i akr, avr;
  long long aS[8];
  if (app) {
    akr = *(const v4i *)(ap.k + h0);
    avr = *(const v4i *)(ap.v + h0);
#pragma unroll
    for (int e = 0; e < 8; ++e) aS[e] = ap.k_sum[h0 + e];
  }

  // ---- quantize q per head (wave w handles head w)
  if (wave < G) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      qx[e] = qx[e] * kch[e];
      amax = fmaxf(amax, fabsf(qx[e]));
    }
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float sq = amax / 127.0f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) s_q8[wave][lane * (D / 64) + e] = (int8_t)quant_i8(qx[e], sq);
    if (lane == 0) s_c[wave] = sq * a.kconst;
  }
  __syncthreads();
  if (app) {
    uint32_t kw[2], vw[2];
    __half nksh, nvsh;
    append_row<D / 8>((const uint16_t *)&akr, (const uint16_t *)&avr, aS, n_new, kw, vw, nksh, nvsh);
    if (lane < D / 8) {
      const size_t row = ((size_t)bg * a.cap + n_new) * D + lane * 8;
      *(uint2 *)(ap.k_codes + row) = make_uint2(kw[0], kw[1]);
      *(uint2 *)(ap.v_codes + row) = make_uint2(vw[0], vw[1]);
      if (lane == 0) {
        ap.k_scales[(size_t)bg * a.cap + n_new] = nksh;
        ap.v_scales[(size_t)bg * a.cap + n_new] = nvsh;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ap.k_sum[h0 + e] = aS[e];
        if (ap.k_mean) ap.k_mean[h0 + e] = mean_from_sum(aS[e], (long long)n_new + 1);
      }
    }
    // the codes reach the lanes that hold key n_new through the wave's own LDS words (the
    // hardware keeps one wave's LDS operations in order; a compiler memory barrier between)
    if (lane < D / 8) {
      s_nk[lane * 2] = (int)kw[0];
      s_nk[lane * 2 + 1] = (int)kw[1];
      s_nv[lane * 2] = (int)vw[0];
      s_nv[lane * 2 + 1] = (int)vw[1];
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
      if (nw + 32 * blk + n32 == n_new) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) kop[blk][kk] = *(const v4i *)&s_nk[(kk * 32 + hh * 16) / 4];
      }
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
      if (nr + p == n_new) vr[p] = *(const Row *)&s_nv[c * CH / 4];
    if (nk == n_new) {
      ksc = __half2float(nksh);
      vsc = __half2float(nvsh);
    }
  }

  // ---- exact int32 scores on the matrix core.  Row R of the A operand holds head
  //      hA = 4*(R/8) + R%4 for key block bA = (R/4)%2 (zero rows elsewhere), so the two
  //      blocks' products land in disjoint rows of one accumulator: lane l then holds the
  //      dots of key nw + l with every head h in element h.
  v16i sacc;
  {
    const int hA = 4 * (n32 >> 3) + (n32 & 3), bA = (n32 >> 2) & 1;
    const bool rowq = hA < G;
    v4i qa[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const v4i qv = *(const v4i *)&s_q8[rowq ? hA : 0][kk * 32 + hh * 16];
      qa[kk] = rowq ? qv : v4i{0, 0, 0, 0};
    }
    const v4i zero = v4i{0, 0, 0, 0};
    v16i s0 = v16i{}, s1 = v16i{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(bA == 0 ? qa[kk] : zero, kop[0][kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(bA == 1 ? qa[kk] : zero, kop[1][kk], s1, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) sacc[h] = s0[h] + s1[h];
  }
  float ch[G];
#pragma unroll
  for (int h = 0; h < G; ++h) ch[h] = s_c[h];

  // ---- this lane's key: scores, wave-local softmax statistics and weights
  float mw[G], lw[G], ww[G], wsc[G];
  _Float16 wq[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int acc = sacc[h];
    if (a.debug_qk && live) a.debug_qk[((size_t)b * a.Hq + g * G + h) * a.kv_len + nk] = acc;
    const float cn = kkey ? ch[h] * ksc : ch[h];
    const float sc = live ? cn * (float)acc : -INFINITY;
    float m = fmaxf(sc, __int_as_float(dpp_xor1(__float_as_int(sc))));
    m = fmaxf(m, __int_as_float(dpp_xor2(__float_as_int(m))));
    m = fmaxf(m, __int_as_float(dpp_mirror8(__float_as_int(m))));
    mw[h] = max_groups(m);
    // (a wave with no live key keeps weight 0 everywhere)
    const float pr = live ? fast_exp2(sc - mw[h]) : 0.0f;
    float l = pr + __int_as_float(dpp_xor1(__float_as_int(pr)));
    l += __int_as_float(dpp_xor2(__float_as_int(l)));
    l += __int_as_float(dpp_mirror8(__float_as_int(l)));
    lw[h] = add_groups(l);
    // PV weight w = p (per-channel V) or p * s_V[n] (per-token V), taken to fp16 after an
    // exact power-of-two scaling that puts the wave's largest weight in [1, 2) (p alone
    // already peaks at exactly 1); the fp16 weights are the ones summed below
    float w = pr, scale = 1.0f;
    if (vtok) {
      // (a lane past kv_len may hold any scale bits, Inf or NaN included, from a row the
      // header leaves unspecified or that the fused append has not yet written: its weight
      // is selected to zero, never computed from that scale)
      w = live ? pr * vsc : 0.0f;
      int e = __float_as_int(w) >> 23;   // (w >= 0: biased exponent)
      e = max(e, dpp_xor1(e));
      e = max(e, dpp_xor2(e));
      e = max_groups_i(max(e, dpp_mirror8(e)));
      scale = (e >= 1 && e <= 253) ? __int_as_float((254 - e) << 23) : 1.0f;
    }
    wsc[h] = scale;
    wq[h] = (_Float16)(w * scale);
    const float wr = (float)wq[h];
    float sw = wr + __int_as_float(dpp_xor1(__float_as_int(wr)));
    sw += __int_as_float(dpp_xor2(__float_as_int(sw)));
    sw += __int_as_float(dpp_mirror8(__float_as_int(sw)));
    ww[h] = add_groups(sw);
  }
  // ---- PV on v_mfma_f32_16x16x32_f16: O^T[ch][h] = sum_n VT[ch][n] * W[n][h], over the
  //      wave's 64 keys in two steps of 32.  V enters as fp16 (1152 + code) -- bytes
  //      (code ^ 0x80) under the exponent byte 0x64, exact -- and the weights as fp16; the
  //      products are exact in fp32 and the 1152 is removed once per head with the sum of the
  //      same fp16 weights.  Both operands pass through the wave's own LDS region (wave-local):
  //      the weights head-major (a lane takes 8 keys of one head), V transposed to one row of
  //      64 keys per channel (a lane takes 8 keys of one channel), the row's 16-byte slots
  //      permuted by the channel so that the reads of 16 channels hit distinct banks.
#pragma unroll
  for (int h = 0; h < G; ++h) s_wh[wave][h][lane] = wq[h];
  float *vt = &s_vo[wave][0];
  auto slot = [](int sl, int chn) { return sl ^ ((chn >> 1) & 7) ^ ((chn >> 4) & 7); };
#pragma unroll
  for (int w = 0; w < CW; ++w)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // keys 8r .. 8r+7 of channel c*CH + 4w + e as four fp16 pairs (keys 2j, 2j+1)
      const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + e) << 16) | (uint32_t)e;
      v4f pk;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[j] = __uint_as_float(__builtin_amdgcn_perm((uint32_t)vr[2 * j + 1][w], (uint32_t)vr[2 * j][w], sel) ^
                                0x64806480u);
      const int chn = c * CH + 4 * w + e;
      *(v4f *)&vt[chn * 32 + slot(r, chn) * 4] = pk;
    }
  // (a compiler memory barrier: the reads below see the other lanes' stores, which the
  // compiler cannot know of without it -- the hardware keeps one wave's LDS operations in order;
  // every access uses the stores' element type)
  asm volatile("" ::: "memory");
  const int m16 = lane & 15, q4 = lane >> 4;
  v4f oacc[D / 16];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) oacc[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    h8t wb;
    const _Float16 *wrow = &s_wh[wave][m16 < G ? m16 : 0][32 * ks + 8 * q4];
#pragma unroll
    for (int i = 0; i < 8; ++i) wb[i] = wrow[i];
    if (m16 >= G) wb = h8t{};
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      const int chn = 16 * mt + m16;
      const v4f av = *(const v4f *)&vt[chn * 32 + slot(4 * ks + q4, chn) * 4];
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8t, av), wb, oacc[mt], 0, 0, 0);
    }
  }
  // ---- lane (m16 < G) holds O^T[16*mt + 4*q4 + i][m16]: into the wave's region as o[h][ch]
  //      (its V rows are no longer read: LDS operations of the wave are in order)
  asm volatile("" ::: "memory");
  if (m16 < G) {
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) *(v4f *)&vt[m16 * D + 16 * mt + 4 * q4] = oacc[mt];
  }
  // (every lane holds the wave's max and sums)
  if (lane < G) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (lane == h) {
        s_wm[wave][h] = mw[h];
        s_wl[wave][h] = lw[h];
        s_ww[wave][h] = ww[h];
        s_ws[wave][h] = wsc[h];
      }
  }
  __syncthreads();

  // ---- merge the waves: M = max_w m_w, f_w = 2^(m_w - M); the weighted sums carry the
  //      wave's weight scaling, undone by g_w = f_w / scale_w (a power of two)
  if (t < kWavesD * G) {
    const int w = t / G, h = t % G;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kWavesD; ++x) M = fmaxf(M, s_wm[x][h]);
    const float f = s_wm[w][h] == -INFINITY ? 0.0f : fast_exp2(s_wm[w][h] - M);
    s_f[w][h] = f;
    s_g[w][h] = f / s_ws[w][h];
  }
  __syncthreads();
  DecWs ws = dec_ws(a.ws, a.B * a.Hkv, G, D, S);
  float *myo = ws.o + ((size_t)bg * S + split) * G * D;
  for (int idx = t; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    float acc = 0.0f, wsum = 0.0f;
#pragma unroll
    for (int x = 0; x < kWavesD; ++x) {
      acc = __builtin_fmaf(s_g[x][h], s_vo[x][idx], acc);
      wsum = __builtin_fmaf(s_g[x][h], s_ww[x][h], wsum);
    }
    myo[idx] = acc - 1152.0f * wsum;
  }
  if (t < G) {
    float M = -INFINITY, L = 0.0f;
#pragma unroll
    for (int x = 0; x < kWavesD; ++x) M = fmaxf(M, s_wm[x][t]);
#pragma unroll
    for (int x = 0; x < kWavesD; ++x) L = __builtin_fmaf(s_f[x][t], s_wl[x][t], L);
    ws.ml[((size_t)bg * S + split) * G + t] = make_float2(M, L);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeLaunch a, int S) {
  decode_body<D, G, false>(a, S, DecodeAppendLaunch{});
}
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_append_kernel(DecodeLaunch a, int S, DecodeAppendLaunch ap) {
  decode_body<D, G, true>(a, S, ap);
}

// Merge of the S split partials of one (batch, kv-head, head): M = max m_s, weights
// f_s = 2^(m_s - M), out = sum_s f_s o_s / sum_s f_s l_s (times the per-channel V scale).
// One workgroup of kMergeQ * D threads per (batch, kv-head, head): thread (q, c) takes the
// splits s = q (mod kMergeQ) of channel c with all its loads issued up front, keeps a
// running max over them, and the kMergeQ partial sums of a channel meet in LDS.
constexpr int kMergeQ = 4;
constexpr int kMergeU = 16;   // loads in flight per thread and round
template <int D, int G>
__global__ __launch_bounds__(kMergeQ * D) void decode_merge_kernel(DecodeLaunch a, int S) {
  const int bgh = blockIdx.x;
  const int h = bgh % G, bg = bgh / G;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int t = threadIdx.x, q = t / D, c = t % D;
  __shared__ float s_m[kMergeQ][D], s_a[kMergeQ][D], s_l[kMergeQ][D];
  DecWs w = dec_ws(a.ws, a.B * a.Hkv, G, D, S);
  const float2 *ml = w.ml + (size_t)bg * S * G + h;
  const float *po = w.o + ((size_t)bg * S * G + h) * D + c;
  float M = -INFINITY, acc = 0.0f, L = 0.0f;
  for (int s0 = q; s0 < S; s0 += kMergeQ * kMergeU) {
    float2 mv[kMergeU];
    float vv[kMergeU];
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
      const int sp = min(s0 + u * kMergeQ, S - 1);   // (duplicates beyond S get weight 0)
      mv[u] = ml[(size_t)sp * G];
      vv[u] = po[(size_t)sp * G * D];
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kMergeU; ++u)
      if (s0 + u * kMergeQ < S) Mc = fmaxf(Mc, mv[u].x);
    const float rs = M == -INFINITY ? 0.0f : fast_exp2(M - Mc);
    acc *= rs;
    L *= rs;
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
      // (an empty or duplicate partial is skipped: its o was never written)
      const bool in = s0 + u * kMergeQ < S && mv[u].x != -INFINITY;
      const float f = in ? fast_exp2(mv[u].x - Mc) : 0.0f;
      acc = in ? __builtin_fmaf(f, vv[u], acc) : acc;
      L = in ? __builtin_fmaf(f, mv[u].y, L) : L;
    }
    M = Mc;
  }
  s_m[q][c] = M;
  s_a[q][c] = acc;
  s_l[q][c] = L;
  __syncthreads();
  if (q != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int x = 0; x < kMergeQ; ++x) Mt = fmaxf(Mt, s_m[x][c]);
  float A = 0.0f, Lt = 0.0f;
#pragma unroll
  for (int x = 0; x < kMergeQ; ++x) {
    const float f = s_m[x][c] == -INFINITY ? 0.0f : fast_exp2(s_m[x][c] - Mt);
    A = __builtin_fmaf(f, s_a[x][c], A);
    Lt = __builtin_fmaf(f, s_l[x][c], Lt);
  }
  float res = Lt > 0.0f ? A / Lt : 0.0f;
  if (!(a.flags & kDecVTok)) res *= ((const float *)a.v_scales)[(size_t)bg * D + c];
  const size_t oi = ((size_t)b * a.Hq + g * G + h) * D + c;
  if (a.flags & kDecOutF32) ((float *)a.out)[oi] = res;
  else ((__half *)a.out)[oi] = __float2half_rn(res);
}

template <int D, int G>
hipError_t launch_g(const DecodeLaunch &a, const DecodeAppendLaunch *app, hipStream_t s, int S) {
  if (app)
    hipLaunchKernelGGL((decode_append_kernel<D, G>), dim3(S, a.B * a.Hkv), dim3(kThreads), 0, s, a, S, *app);
  else
    hipLaunchKernelGGL((decode_kernel<D, G>), dim3(S, a.B * a.Hkv), dim3(kThreads), 0, s, a, S);
  hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3(a.B * a.Hkv * G), dim3(kMergeQ * D), 0, s, a, S);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dd(const DecodeLaunch &a, const DecodeAppendLaunch *app, hipStream_t s, int S) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<D, 1>(a, app, s, S);
    case 2: return launch_g<D, 2>(a, app, s, S);
    case 4: return launch_g<D, 4>(a, app, s, S);
    default: return launch_g<D, 8>(a, app, s, S);
  }
}

}  // namespace

// ------------------------------------------------------- static scratch ---
// The per-split partials of attn_q_decode_noalloc live in this file-scope array instead of a
// caller workspace (for callers that cannot allocate: code under graph capture, serving loops
// that forbid allocation).  Each GPU the library runs on holds its own copy until the process
// ends.  Host code never uses the array's name as an address: its device address is looked
// up once per device with hipGetSymbolAddress and kept.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch_ptr(void **out) {
  constexpr int kMaxDev = 64;
  static std::atomic<void *> s_ptr[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  void *p = s_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // (the current device is this one: the address is that device's copy of the array)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    s_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D, int kv_len) {
  const int G = Hq / Hkv, BH = B * Hkv;
  const int S = (kv_len + KPS - 1) / KPS;
  return align256((size_t)BH * S * G * 8) + align256((size_t)BH * S * G * D * 4);
}

hipError_t launch_decode(const DecodeLaunch &a, const DecodeAppendLaunch *app, hipStream_t s) {
  const int S = (a.kv_len + KPS - 1) / KPS;
  return a.D == 128 ? launch_dd<128>(a, app, s, S) : launch_dd<64>(a, app, s, S);
}

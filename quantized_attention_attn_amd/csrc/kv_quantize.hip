// kv_quantize_i8: fp16 K/V -> int8 KV cache (+ the e4m3 / int8 PV operand of the prefill).
//
// K is made int8-safe by subtracting its per-channel mean ("int8 Flash Attention
// on RDNA4: QK Wants Integers, PV Wants FP8", section "K's outliers, and the
// subtraction softmax does not notice"); codes follow the symmetric amax/127
// quantizer of eq. (1)-(2) of "QFlash: Bridging Quantization and Memory
// Efficiency in Vision Transformer Attention".
//
// Two launches over HBM-bound data (three for per-tensor K):
//   1. stats  : one pass over K (and V) accumulating, per (b, g, channel), the
//               exact int64 fixed-point sum of K (fp16 * 2^24 is an integer, so
//               the sum is order independent), K's max and min (order keys of the
//               fp16 bits) and |V|'s max -- the K-mean reduction fused into the
//               K tile loads.  Accumulation is atomic into the workspace, which the
//               caller zero-fills once and every call leaves zero-filled again.
//   2. codes  : each workgroup first derives its (b, g)'s statistics from the
//               accumulators: mu = fp32(S / (N * 2^24)); per-channel scales; the
//               centred absmax of channel c is max(|fl(kmax-mu)|, |fl(kmin-mu)|)
//               because x -> fl(x - mu) is monotonic.  Then one pass writing int8 K/V
//               codes (per-token scales reduced across the lanes holding one row), and
//               the PV operand tile of 64 keys transposed through LDS into its
//               documented permuted layout.  The last workgroup of a (b, g) to finish
//               (an atomic count) resets its accumulators.
//   Per-tensor K needs every (b, g)'s absmax before any code, so there a finalize
//   launch between the two takes the statistics (and resets the accumulators).
#include <algorithm>

#include "common.h"

using namespace attnq;

namespace {

constexpr int kThreads = 512;      // statistics workgroup
constexpr int kStatRows = 512;     // keys per statistics workgroup
constexpr int kCodesTilesPerWG = 4;     // at most, per codes workgroup
constexpr int kCodesMinWGs = 512;       // ... while at least this many workgroups remain

struct WsLayout {
  long long *ksum;       // [BH][D]  accumulators (zero between calls)
  uint32_t *kmax, *kmin; // [BH][D]  fp16 order keys, stored as key+1 / ~key so 0 is neutral
  uint32_t *vamax;       // [BH][D]  fp32 bits of max |v|
  float *bg_amax;        // [BH]     centred K absmax per (b, g) (per-tensor scale)
  uint32_t *done;        // [BH]     codes workgroups of (b, g) past the statistics (zero between calls)
};

__host__ __device__ inline WsLayout ws_layout(void *ws, int BH, int D) {
  char *p = (char *)ws;
  WsLayout w;
  w.ksum = (long long *)p;
  p += (size_t)BH * D * 8;
  w.kmax = (uint32_t *)p;
  p += (size_t)BH * D * 4;
  w.kmin = (uint32_t *)p;
  p += (size_t)BH * D * 4;
  w.vamax = (uint32_t *)p;
  p += (size_t)BH * D * 4;
  w.bg_amax = (float *)p;
  p += (size_t)BH * 4;
  w.done = (uint32_t *)p;
  return w;
}

// grid (ceil(N / kStatRows), BH); each thread owns 8 channels of kStatRows / RPP rows.  The
// statistics needed (K sum, K extrema, V absmax) are template flags, so the code has no
// branches.  All of a thread's row loads are issued before any is used.  The thread's K sum
// is taken in fp64, which is exact here: every fp16 value is a multiple of 2^-24 below 2^16,
// so a sum of at most 16 of them needs at most 44 significant bits; times 2^24 it is the
// exact int64 fixed-point value the accumulators hold.  Extrema are fp32 max / min of the
// converted values (exact), turned into fp16 order keys once per channel.
template <int D, bool need_sum, bool need_kminmax, bool need_vamax>
__global__ __launch_bounds__(kThreads) void kvq_stats(const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v, int N,
                                                      void *ws, int BH) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPP = kThreads / LPR;        // rows per pass
  constexpr int NP = kStatRows / RPP;        // passes (rows per thread)
  static_assert(NP <= 16, "exact fp64 partial sums of at most 16 fp16 values");
  const int bg = blockIdx.y;
  const int t = threadIdx.x;
  const int part = t % LPR, rsub = t / LPR;
  const int n0 = blockIdx.x * kStatRows;
  const int n1 = min(N, n0 + kStatRows);
  const size_t base = (size_t)bg * N * D;
  // rows past n1 repeat the group's first row (idempotent for max/min; zeroed for the sum)
  v4i kr[NP], vr[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int n = n0 + u * RPP + rsub;
    const int nn = n < n1 ? n : n0;
    if (need_sum || need_kminmax) kr[u] = *(const v4i *)(k + base + (size_t)nn * D + part * 8);
  }
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int n = n0 + u * RPP + rsub;
    const int nn = n < n1 ? n : n0;
    if (need_vamax) vr[u] = *(const v4i *)(v + base + (size_t)nn * D + part * 8);
  }
  __builtin_amdgcn_sched_barrier(0);   // (every load issued before the first use)
  double sum[8];
  float kmx[8], kmn[8], vam[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { sum[e] = 0.0; kmx[e] = -INFINITY; kmn[e] = INFINITY; vam[e] = 0.0f; }
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const bool in = n0 + u * RPP + rsub < n1;
    if (need_sum || need_kminmax) {
      const uint16_t *h = (const uint16_t *)&kr[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __half2float(__ushort_as_half(h[e]));
        if (need_sum) sum[e] += (double)(in ? x : 0.0f);
        kmx[e] = fmaxf(kmx[e], x);
        kmn[e] = fminf(kmn[e], x);
      }
    }
    if (need_vamax) {
      const uint16_t *h = (const uint16_t *)&vr[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) vam[e] = fmaxf(vam[e], fabsf(__half2float(__ushort_as_half(h[e]))));
    }
  }
  // reduce over the RPP row groups through LDS
  __shared__ long long s_sum[RPP][D];
  __shared__ uint32_t s_a[RPP][D], s_b[RPP][D], s_c[RPP][D];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = part * 8 + e;
    s_sum[rsub][c] = (long long)(sum[e] * 16777216.0);
    s_a[rsub][c] = f16_order_key(__half_as_ushort(__float2half_rn(kmx[e])));
    s_b[rsub][c] = f16_order_key(__half_as_ushort(__float2half_rn(kmn[e])));
    s_c[rsub][c] = __float_as_uint(vam[e]);
  }
  __syncthreads();
  WsLayout w = ws_layout(ws, BH, D);
  for (int c = t; c < D; c += kThreads) {
    long long S = 0;
    uint32_t a = 0u, b = 0xFFFFFFFFu, vv = 0u;
    for (int r = 0; r < RPP; ++r) {
      S += s_sum[r][c];
      a = max(a, s_a[r][c]);
      b = min(b, s_b[r][c]);
      vv = max(vv, s_c[r][c]);
    }
    const size_t idx = (size_t)bg * D + c;
    if (need_sum) atomicAdd((unsigned long long *)&w.ksum[idx], (unsigned long long)S);
    if (need_kminmax) {
      atomicMax(&w.kmax[idx], a + 1u);    // (order keys are < 2^16: zero stays neutral)
      atomicMax(&w.kmin[idx], ~b);        // max of ~key = min of key; zero is neutral
    }
    if (need_vamax) atomicMax(&w.vamax[idx], vv);
  }
}

// Per-channel results of the statistics at index idx = bg * D + c: mu = fp32(S / (N * 2^24))
// (0 without the shift); the centred K absmax max(|fl(kmax - mu)|, |fl(kmin - mu)|) (x -> fl(x -
// mu) is monotone); |V|'s max.
struct ChanStats {
  float mu, kamax, vamax;
};
__device__ __forceinline__ ChanStats chan_stats(const WsLayout &w, size_t idx, int N, int subtract_mean) {
  ChanStats r;
  r.mu = subtract_mean ? mean_from_sum(w.ksum[idx], N) : 0.0f;
  const float hi = f16_from_order_key(w.kmax[idx] - 1u);
  const float lo = f16_from_order_key(~w.kmin[idx]);
  r.kamax = fmaxf(fabsf(hi - r.mu), fabsf(lo - r.mu));
  r.vamax = __uint_as_float(w.vamax[idx]);
  return r;
}

// grid BH, block D threads.  Consumes and resets the accumulators (per-tensor K only; the other
// granularities take the statistics inside the codes kernel).
__global__ void kvq_finalize(int N, int D, int subtract_mean, int k_gran, int v_gran,
                             float *__restrict__ k_mean, long long *__restrict__ k_sum,
                             float *__restrict__ k_scales, float *__restrict__ v_scales, void *ws,
                             int BH) {
  const int bg = blockIdx.x, c = threadIdx.x;
  __shared__ float s_amax[256];
  WsLayout w = ws_layout(ws, BH, D);
  const size_t idx = (size_t)bg * D + c;
  float amax = 0.0f;
  if (c < D) {
    const ChanStats st = chan_stats(w, idx, N, subtract_mean);
    k_mean[idx] = st.mu;
    if (k_sum) k_sum[idx] = w.ksum[idx];
    if (k_gran == ATTN_Q_GRAN_CHANNEL || k_gran == ATTN_Q_GRAN_TENSOR) {
      amax = st.kamax;
      if (k_gran == ATTN_Q_GRAN_CHANNEL) k_scales[idx] = amax / 127.0f;
    }
    if (v_gran == ATTN_Q_GRAN_CHANNEL) v_scales[idx] = st.vamax / 127.0f;
    w.ksum[idx] = 0;
    w.kmax[idx] = 0u;
    w.kmin[idx] = 0u;
    w.vamax[idx] = 0u;
  }
  if (k_gran == ATTN_Q_GRAN_TENSOR) {
    s_amax[c] = amax;
    __syncthreads();
    if (c == 0) {
      float m = 0.0f;
      for (int i = 0; i < D; ++i) m = fmaxf(m, s_amax[i]);
      w.bg_amax[bg] = m;
    }
  }
}

// inverse of the PV-operand permutation: key r of a 64-key tile -> byte position
__device__ __forceinline__ int vop_pos(int r) {
  const int j = r >> 5, a = (r >> 3) & 3, h = (r >> 2) & 1, b = r & 3;
  return 32 * h + 16 * j + 4 * a + b;
}

// grid (ceil(ntiles / tpw), BH): each workgroup quantizes tpw consecutive 64-key tiles (four
// while that leaves at least 512 workgroups, two per CU), the loads of the next tile in flight
// while the current one is converted and stored.  The granularities are template arguments.
// Block: 16 rows per pass (2*D threads), so each thread owns 4 consecutive rows of a tile.
template <int D>
constexpr int codes_threads() { return 2 * D; }

template <int D, int KG, int VG>
__global__ __launch_bounds__(codes_threads<D>()) void kvq_codes(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int N, int cap, int8_t *__restrict__ k_codes,
    int8_t *__restrict__ v_codes, void *k_scales, void *v_scales, float *__restrict__ k_mean, uint8_t *__restrict__ v_op, int v_op_format,
    void *ws, int BH, int ntiles, int tpw, int fused, int subtract_mean, long long *__restrict__ k_sum) {
  constexpr int LPR = D / 8;
  constexpr int NT = codes_threads<D>();
  constexpr int RPP = NT / LPR;
  // (the granularities are template arguments: their branches fold away inside the row loop)
  constexpr int k_gran = KG, v_gran = VG;
  const int bg = blockIdx.y;
  const int t = threadIdx.x;
  const int part = t % LPR, rsub = t / LPR;
  __shared__ uint8_t s_vop[D * 64];
  __shared__ float s_bam[NT / 64];   // (K BLOCK: the waves' maxima)

  float mu[8], ksc[8], vsc[8];
  WsLayout w = ws_layout(ws, BH, D);
  const size_t in_base = (size_t)bg * N * D;
  const size_t out_base = (size_t)bg * cap * D;
  // thread (part, rsub) owns the 64 / RPP consecutive rows rsub * RW .. of the tile, so
  // the PV operand bytes of a channel for those rows are one LDS word
  constexpr int RW = 64 / RPP;
  static_assert(RW == 4, "PV-operand words of 4 consecutive keys");
  // (the first tile is requested before anything else waits)
  const int t0 = blockIdx.x * tpw, t1 = min(t0 + tpw, ntiles);
  v4i kin[RW], vin[RW], knx[RW], vnx[RW];
  auto load_tile = [&](int tile, v4i (&kd)[RW], v4i (&vd)[RW]) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int n = min(tile * 64 + rsub * RW + i, N - 1);   // (rows >= N are zeroed below)
      kd[i] = *(const v4i *)(k + in_base + (size_t)n * D + part * 8);
      vd[i] = *(const v4i *)(v + in_base + (size_t)n * D + part * 8);
    }
  };
  load_tile(t0, kin, vin);
  float ktensor = 0.0f;
  if (k_gran == ATTN_Q_GRAN_TENSOR) {   // (uniform over the grid)
    __shared__ float s_red[NT / 64];
    float m = 0.0f;
    for (int i = t; i < BH; i += NT) m = fmaxf(m, w.bg_amax[i]);
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((t & 63) == 0) s_red[t >> 6] = m;
    __syncthreads();
    m = 0.0f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) m = fmaxf(m, s_red[i]);
    ktensor = m / 127.0f;
    if (bg == 0 && blockIdx.x == 0 && t == 0) ((float *)k_scales)[0] = ktensor;
  }
  if (fused) {
    // the statistics of (b, g) taken here from the accumulators (the workgroups of the first
    // tile column also store mu, the header sum and the channel scales); the last workgroup of
    // (b, g) to finish zeroes the accumulators for the next call (at the end)
    // (one thread per channel; the results reach the others through LDS)
    __shared__ float s_mu[D], s_ks[D], s_vs[D];
    if (t < D) {
      const size_t idx = (size_t)bg * D + t;
      const ChanStats st = chan_stats(w, idx, N, subtract_mean);
      s_mu[t] = st.mu;
      s_ks[t] = k_gran == ATTN_Q_GRAN_CHANNEL ? st.kamax / 127.0f : 0.0f;
      s_vs[t] = v_gran == ATTN_Q_GRAN_CHANNEL ? st.vamax / 127.0f : 0.0f;
      if (blockIdx.x == 0) {
        k_mean[idx] = st.mu;
        if (k_sum) k_sum[idx] = w.ksum[idx];
        if (k_gran == ATTN_Q_GRAN_CHANNEL) ((float *)k_scales)[idx] = s_ks[t];
        if (v_gran == ATTN_Q_GRAN_CHANNEL) ((float *)v_scales)[idx] = s_vs[t];
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mu[e] = s_mu[part * 8 + e];
      ksc[e] = s_ks[part * 8 + e];
      vsc[e] = s_vs[part * 8 + e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = part * 8 + e;
      mu[e] = k_mean[(size_t)bg * D + c];
      ksc[e] = k_gran == ATTN_Q_GRAN_CHANNEL ? ((const float *)k_scales)[(size_t)bg * D + c] : ktensor;
      vsc[e] = v_gran == ATTN_Q_GRAN_CHANNEL ? ((const float *)v_scales)[(size_t)bg * D + c] : 0.0f;
    }
  }
  // reciprocals of the scales (per channel / tensor here; per token once per row below)
  float krs0[8], vrs0[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    krs0[e] = k_gran == ATTN_Q_GRAN_TOKEN ? 0.0f : rcp_or_zero(ksc[e]);
    vrs0[e] = v_gran == ATTN_Q_GRAN_TOKEN ? 0.0f : rcp_or_zero(vsc[e]);
  }
  for (int tile = t0; tile < t1; ++tile) {
  if (tile + 1 < t1) load_tile(tile + 1, knx, vnx);
  uint32_t vword[RW / 4][8];
  float krs[8], vrs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { krs[e] = krs0[e]; vrs[e] = vrs0[e]; }
  if (k_gran == ATTN_Q_GRAN_BLOCK) {
    // one scale for the tile's keys (a 64-key block): the amax of x = fp32(k) - mu over its keys
    // below N and all channels -- the lanes' maxima, then the waves'
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const bool valid = tile * 64 + rsub * RW + i < N;
      const uint16_t *kh = (const uint16_t *)&kin[i];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        am = valid ? fmaxf(am, fabsf(__half2float(__ushort_as_half(kh[e])) - mu[e])) : am;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
    if ((t & 63) == 0) s_bam[t >> 6] = am;
    __syncthreads();
    am = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) am = fmaxf(am, s_bam[w]);
    __syncthreads();   // (s_bam is rewritten by the next tile)
    const float sb = am / 127.0f, rsb = rcp_or_zero(sb);
#pragma unroll
    for (int e = 0; e < 8; ++e) { ksc[e] = sb; krs[e] = rsb; }
    if (t == 0 && tile * 64 < N) ((float *)k_scales)[(size_t)bg * (cap / 64) + tile] = sb;
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int rr = rsub * RW + i;
    const int n = tile * 64 + rr;
    const bool valid = n < N;
    float kx[8], vx[8];
    const uint16_t *kh = (const uint16_t *)&kin[i];
    const uint16_t *vh = (const uint16_t *)&vin[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kx[e] = valid ? __half2float(__ushort_as_half(kh[e])) - mu[e] : 0.0f;
      vx[e] = valid ? __half2float(__ushort_as_half(vh[e])) : 0.0f;
    }
    // per-token scales: absmax over the LPR consecutive lanes holding this row
    if (k_gran == ATTN_Q_GRAN_TOKEN || v_gran == ATTN_Q_GRAN_TOKEN) {
      float ka = 0.0f, va = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { ka = fmaxf(ka, fabsf(kx[e])); va = fmaxf(va, fabsf(vx[e])); }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) {
        ka = fmaxf(ka, __shfl_xor(ka, m));
        va = fmaxf(va, __shfl_xor(va, m));
      }
      if (k_gran == ATTN_Q_GRAN_TOKEN) {
        const __half sh = __float2half_rn(ka / 127.0f);
        const float sc = __half2float(sh), rsc = rcp_or_zero(sc);
#pragma unroll
        for (int e = 0; e < 8; ++e) { ksc[e] = sc; krs[e] = rsc; }
        if (valid && part == 0) ((__half *)k_scales)[(size_t)bg * cap + n] = sh;
      }
      if (v_gran == ATTN_Q_GRAN_TOKEN) {
        const __half sh = __float2half_rn(va / 127.0f);
        const float sc = __half2float(sh), rsc = rcp_or_zero(sc);
#pragma unroll
        for (int e = 0; e < 8; ++e) { vsc[e] = sc; vrs[e] = rsc; }
        if (valid && part == 0) ((__half *)v_scales)[(size_t)bg * cap + n] = sh;
      }
    }
    // codes: the clamped quotient q (quant_i8_q), its byte as the low byte of fp32(q + 1.5 * 2^23)
    // (whose add rounds to nearest-even) and, for the e4m3 operand, its rounded value
    uint32_t kb[8], vb[8];
    float vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kb[e] = quant_i8_byte(kx[e], ksc[e], krs[e]);
      const float qv = quant_i8_q(vx[e], vsc[e], vrs[e]);
      vb[e] = __float_as_uint(qv + 12582912.0f) & 0xFFu;
      vv[e] = __builtin_rintf(qv) + 0.0f;   // (+0 for a zero code: e4m3 of -0 is a different byte)
    }
    if (valid) {
      uint32_t klo = 0, khi = 0, vlo = 0, vhi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        klo |= kb[e] << (8 * e);
        khi |= kb[e + 4] << (8 * e);
        vlo |= vb[e] << (8 * e);
        vhi |= vb[e + 4] << (8 * e);
      }
      *(uint2 *)(k_codes + out_base + (size_t)n * D + part * 8) = make_uint2(klo, khi);
      if (v_codes) *(uint2 *)(v_codes + out_base + (size_t)n * D + part * 8) = make_uint2(vlo, vhi);
    }
    if (v_op) {
      // byte i%4 of the channel's word for keys rr - i%4 .. rr - i%4 + 3 (0 for keys >= N)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t byte;
        if (v_op_format == ATTN_Q_PV_FP8)
          byte = (uint32_t)cvt_pk_e4m3<false>(vv[e], 0.0f, 0) & 0xFFu;
        else
          byte = vb[e];
        if (!valid) byte = 0;
        if ((i & 3) == 0) vword[i / 4][e] = byte;
        else vword[i / 4][e] |= byte << (8 * (i & 3));
      }
    }
  }
  if (v_op) {
#pragma unroll
    for (int q = 0; q < RW / 4; ++q) {
      const int pos = vop_pos(rsub * RW + 4 * q);   // 4 consecutive keys -> 4 consecutive bytes
#pragma unroll
      for (int e = 0; e < 8; ++e) *(uint32_t *)&s_vop[(part * 8 + e) * 64 + pos] = vword[q][e];
    }
  }
  if (v_op) {
    __syncthreads();
    uint8_t *dst = v_op + ((size_t)bg * (cap / 64) + tile) * D * 64;
    for (int i = t; i < D * 64 / 16; i += NT)
      ((v4i *)dst)[i] = ((const v4i *)s_vop)[i];
    __syncthreads();   // (the next tile writes the LDS tile again)
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) { kin[i] = knx[i]; vin[i] = vnx[i]; }
  }
  if (fused) {
    // every thread's accumulator reads returned long ago (their values fed the codes); the
    // workgroup that counts (b, g) complete resets the accumulators
    __shared__ int s_last;
    __syncthreads();
    if (t == 0) s_last = atomicAdd(&w.done[bg], 1u) == gridDim.x - 1;
    __syncthreads();
    if (s_last) {
      for (int c = t; c < D; c += NT) {
        const size_t idx = (size_t)bg * D + c;
        w.ksum[idx] = 0;
        w.kmax[idx] = 0u;
        w.kmin[idx] = 0u;
        w.vamax[idx] = 0u;
      }
      if (t == 0) w.done[bg] = 0u;
    }
  }
}

}  // namespace

size_t kvq_workspace_bytes(int B, int H, int D) {
  return (size_t)B * H * D * 20 + (size_t)B * H * 8 + 256;
}

namespace {
template <int D, bool SUM, bool MM>
void launch_stats_v(dim3 g, hipStream_t s, const KvqLaunch &a, bool va, int BH) {
  if (va) hipLaunchKernelGGL((kvq_stats<D, SUM, MM, true>), g, dim3(kThreads), 0, s, a.k, a.v, a.N, a.ws, BH);
  else hipLaunchKernelGGL((kvq_stats<D, SUM, MM, false>), g, dim3(kThreads), 0, s, a.k, a.v, a.N, a.ws, BH);
}
template <int D>
void launch_stats(dim3 g, hipStream_t s, const KvqLaunch &a, bool sum, bool mm, bool va, int BH) {
  if (sum && mm) launch_stats_v<D, true, true>(g, s, a, va, BH);
  else if (sum) launch_stats_v<D, true, false>(g, s, a, va, BH);
  else if (mm) launch_stats_v<D, false, true>(g, s, a, va, BH);
  else launch_stats_v<D, false, false>(g, s, a, va, BH);
}
}  // namespace

namespace {
template <int D, int KG, int VG>
void launch_codes_g(const KvqLaunch &a, hipStream_t s, dim3 g, uint8_t *vop_here, int ntiles, int tpw, int fused) {
  hipLaunchKernelGGL((kvq_codes<D, KG, VG>), g, dim3(codes_threads<D>()), 0, s, a.k, a.v, a.N, a.cap, a.k_codes,
                     a.v_codes, a.k_scales, a.v_scales, a.k_mean, vop_here, a.v_op_format, a.ws, a.B * a.H, ntiles,
                     tpw, fused, (int)a.subtract_mean, (long long *)a.k_sum);
}
template <int D, int KG>
void launch_codes_k(const KvqLaunch &a, hipStream_t s, dim3 g, uint8_t *vop_here, int ntiles, int tpw, int fused) {
  if (a.v_gran == ATTN_Q_GRAN_TOKEN) launch_codes_g<D, KG, ATTN_Q_GRAN_TOKEN>(a, s, g, vop_here, ntiles, tpw, fused);
  else launch_codes_g<D, KG, ATTN_Q_GRAN_CHANNEL>(a, s, g, vop_here, ntiles, tpw, fused);
}
template <int D>
void launch_codes(const KvqLaunch &a, hipStream_t s, dim3 g, uint8_t *vop_here, int ntiles, int tpw, int fused) {
  switch (a.k_gran) {
    case ATTN_Q_GRAN_TOKEN: launch_codes_k<D, ATTN_Q_GRAN_TOKEN>(a, s, g, vop_here, ntiles, tpw, fused); break;
    case ATTN_Q_GRAN_BLOCK: launch_codes_k<D, ATTN_Q_GRAN_BLOCK>(a, s, g, vop_here, ntiles, tpw, fused); break;
    case ATTN_Q_GRAN_TENSOR: launch_codes_k<D, ATTN_Q_GRAN_TENSOR>(a, s, g, vop_here, ntiles, tpw, fused); break;
    default: launch_codes_k<D, ATTN_Q_GRAN_CHANNEL>(a, s, g, vop_here, ntiles, tpw, fused); break;
  }
}
}  // namespace

hipError_t launch_kv_quantize(const KvqLaunch &a, hipStream_t s) {
  const int BH = a.B * a.H;
  const bool need_sum = a.subtract_mean != 0 || a.k_sum != nullptr;
  const bool need_kminmax = a.k_gran == ATTN_Q_GRAN_CHANNEL || a.k_gran == ATTN_Q_GRAN_TENSOR;
  const bool need_vamax = a.v_gran == ATTN_Q_GRAN_CHANNEL;
  if (need_sum || need_kminmax || need_vamax) {
    dim3 g((a.N + kStatRows - 1) / kStatRows, BH);
    if (a.D == 128) launch_stats<128>(g, s, a, need_sum, need_kminmax, need_vamax, BH);
    else launch_stats<64>(g, s, a, need_sum, need_kminmax, need_vamax, BH);
  }
  // per-tensor K needs every (b, g)'s absmax before any code: a launch of its own; the other
  // granularities take their statistics inside the codes kernel
  const int fused = a.k_gran != ATTN_Q_GRAN_TENSOR;
  if (!fused)
    hipLaunchKernelGGL(kvq_finalize, dim3(BH), dim3(a.D), 0, s, a.N, a.D, a.subtract_mean, a.k_gran,
                       a.v_gran, a.k_mean, (long long *)a.k_sum, (float *)a.k_scales, (float *)a.v_scales, a.ws, BH);
  // with a per-channel PV operand every tile up to the capacity is written here (keys >= N as
  // 0); a per-token operand needs the header V_max over all keys first, so it is built after
  // the codes by the operand kernels
  uint8_t *vop_here = a.v_gran == ATTN_Q_GRAN_CHANNEL ? a.v_op : nullptr;
  const int ntiles = vop_here ? a.cap / 64 : (a.N + 63) / 64;
  // tiles per workgroup: enough workgroups to fill the chip, each with a few tiles to pipeline
  const int tpw = std::max(1, std::min(kCodesTilesPerWG, ntiles * BH / kCodesMinWGs));
  dim3 g((ntiles + tpw - 1) / tpw, BH);
  if (a.D == 128) launch_codes<128>(a, s, g, vop_here, ntiles, tpw, fused);
  else launch_codes<64>(a, s, g, vop_here, ntiles, tpw, fused);
  if (a.v_op && !vop_here) {
    VopLaunch vl;
    vl.B = a.B; vl.H = a.H; vl.D = a.D; vl.cap = a.cap; vl.n_keys = a.N;
    vl.v_codes = a.v_codes; vl.v_scales = a.v_scales; vl.v_gran = a.v_gran; vl.fmt = a.v_op_format;
    vl.v_op = a.v_op; vl.v_scale_max = a.v_scale_max;
    return launch_v_operand(vl, s);
  }
  return hipGetLastError();
}

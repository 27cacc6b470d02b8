// attn_q_decode: one query per head against the int8 KV cache.
//
// "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8", sections "Does
// quantizing attention help decode?" and "What actually changed for decode": at
// batch one attention is a matrix-vector product bound by how fast the KV cache
// streams from memory, so the matrix cores are not used; halving the cache's bytes
// is what speeds it up.
//
// gfx950 mapping.  One workgroup (8 waves) per (batch, kv-head, split of 512 keys):
//   * every thread issues all of its K and V loads up front (16 B per lane; 8
//     consecutive lanes cover one 128-byte code row, so each wave load instruction
//     reads 1 KB of contiguous cache) -- 128 KB in flight per workgroup;
//   * each K row serves all G query heads of the kv-head: exact int32 dots with
//     v_dot4_i32_i8 reduced over the lanes of the row; scores s = fp32(c_n * acc);
//   * softmax over the split in LDS (max, exp2, sum per head), then PV in fp32 on the
//     V codes (converted as unsigned bytes of code+128, the +128 removed once per head
//     at the end), folded across rows with lane shuffles and LDS;
//   * partial (m, l, o) per split go to the workspace and a second small kernel merges
//     them per (batch, kv-head) with its loads in flight at once.  (Merging inside the
//     first kernel would need a device-scope release/acquire per workgroup, which on a
//     multi-XCD part writes back and invalidates the whole L2 -- far costlier than a
//     kernel boundary.)
#include "common.h"

using namespace attnq;

namespace {

constexpr int kThreads = 512;
constexpr int kWavesD = kThreads / 64;
constexpr int KPS = 512;       // keys per split (workgroup)
constexpr int kMergeChunk = 128;  // partials staged in LDS per merge round
static_assert(KPS == kThreads, "one key scale per thread is staged in LDS");

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

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeLaunch a, int S) {
  constexpr int LPR = D / 16;            // lanes per code row (16 B each)
  constexpr int RPP = kThreads / LPR;    // rows per pass
  constexpr int NPASS = KPS / RPP;
  constexpr int RPW = 64 / LPR;          // rows per wave per pass
  constexpr int NGRP = kWavesD * (8 / LPR > 0 ? 8 / LPR : 1);  // row groups after 3 lane folds
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int part = t % LPR, rsub = t / LPR;
  const int n0 = split * KPS;

  __shared__ __attribute__((aligned(16))) int8_t s_q8[G][D];
  __shared__ float s_c[G];
  __shared__ float s_sc[G][KPS];
  __shared__ float s_m[G], s_l[G], s_wsum[G];
  __shared__ __attribute__((aligned(16))) float s_red[NGRP][G * D];
  __shared__ float s_ks[KPS], s_vs[KPS];

  // ---- loads: q and the split's per-key scales first (so waiting for them never waits
  //      for the code rows), then every K and V code row of the split
  float qx[D / 64], kch[D / 64];
  if (wave < G) {
    const uint16_t *qp = a.q + ((size_t)b * a.Hq + g * G + wave) * D;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      const int c = lane * (D / 64) + e;
      qx[e] = __half2float(__ushort_as_half(qp[c]));
      kch[e] = a.k_gran == ATTN_Q_GRAN_CHANNEL ? ((const float *)a.k_scales)[(size_t)bg * D + c] : 1.0f;
    }
  }
  float ksv = 1.0f, vsv = 1.0f;
  if (n0 + t < a.kv_len) {
    if (a.k_gran == ATTN_Q_GRAN_TOKEN) ksv = __half2float(((const __half *)a.k_scales)[(size_t)bg * a.cap + n0 + t]);
    if (a.v_gran == ATTN_Q_GRAN_TOKEN) vsv = __half2float(((const __half *)a.v_scales)[(size_t)bg * a.cap + n0 + t]);
  }
  const size_t cbase = (size_t)bg * a.cap * D;
  v4i kr[NPASS], vr[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int n = min(n0 + ps * RPP + rsub, a.kv_len - 1);  // rows past kv_len are masked later
    kr[ps] = *(const v4i *)(a.k_codes + cbase + (size_t)n * D + part * 16);
    vr[ps] = *(const v4i *)(a.v_codes + cbase + (size_t)n * D + part * 16);
  }

  // ---- quantize q per head (wave w handles head w)
  if (wave < G) {
    const int hq = wave;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      qx[e] = qx[e] * kch[e];
      amax = fmaxf(amax, fabsf(qx[e]));
    }
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float sq = amax / 127.0f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) s_q8[hq][lane * (D / 64) + e] = (int8_t)quant_i8(qx[e], sq);
    if (lane == 0) s_c[hq] = sq * a.kconst;
  }
  s_ks[t] = ksv;
  s_vs[t] = vsv;
  __syncthreads();

  // ---- scores
  int qw[G][4];
#pragma unroll
  for (int hq = 0; hq < G; ++hq)
#pragma unroll
    for (int w = 0; w < 4; ++w) qw[hq][w] = ((const int *)&s_q8[hq][part * 16])[w];
  float ch[G];
#pragma unroll
  for (int hq = 0; hq < G; ++hq) ch[hq] = s_c[hq];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int nl = ps * RPP + rsub, n = n0 + nl;
    const bool valid = n < a.kv_len;
    int acc[G];
#pragma unroll
    for (int hq = 0; hq < G; ++hq) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) s = __builtin_amdgcn_sdot4(kr[ps][w], qw[hq][w], s, false);
      acc[hq] = s;
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1)
#pragma unroll
      for (int hq = 0; hq < G; ++hq) acc[hq] += __shfl_xor(acc[hq], m);
    const float ksc = s_ks[nl];
#pragma unroll
    for (int hq = 0; hq < G; ++hq) {
      if ((hq % LPR) == part) {
        const float cn = a.k_gran == ATTN_Q_GRAN_TOKEN ? ch[hq] * ksc : ch[hq];
        s_sc[hq][nl] = valid ? cn * (float)acc[hq] : -INFINITY;
        if (a.debug_qk && valid) a.debug_qk[((size_t)b * a.Hq + g * G + hq) * a.kv_len + n] = acc[hq];
      }
    }
  }
  __syncthreads();

  // ---- softmax over the split, per head: weights w = p (CHANNEL V) or p * s_V[n]
  for (int hq = wave; hq < G; hq += kWavesD) {
    float mx = -INFINITY;
    for (int j = lane; j < KPS; j += 64) mx = fmaxf(mx, s_sc[hq][j]);
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    float sum = 0.0f, wsum = 0.0f;
    for (int j = lane; j < KPS; j += 64) {
      const float sv = s_sc[hq][j];
      const float p = sv == -INFINITY ? 0.0f : fast_exp2(sv - mx);
      sum += p;
      const float w = a.v_gran == ATTN_Q_GRAN_TOKEN ? p * s_vs[j] : p;
      wsum += w;
      s_sc[hq][j] = w;
    }
    for (int m = 32; m >= 1; m >>= 1) {
      sum += __shfl_xor(sum, m);
      wsum += __shfl_xor(wsum, m);
    }
    if (lane == 0) { s_m[hq] = mx; s_l[hq] = sum; s_wsum[hq] = wsum; }
  }
  __syncthreads();

  // ---- PV: o = sum_n w_n * (u_n - 128), u = code + 128 read as unsigned bytes
  float o[G][16];
#pragma unroll
  for (int hq = 0; hq < G; ++hq)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[hq][e] = 0.0f;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int nl = ps * RPP + rsub;
    float vf[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t word = (uint32_t)vr[ps][w] ^ 0x80808080u;
      vf[4 * w + 0] = (float)((word >> 0) & 0xFFu);
      vf[4 * w + 1] = (float)((word >> 8) & 0xFFu);
      vf[4 * w + 2] = (float)((word >> 16) & 0xFFu);
      vf[4 * w + 3] = (float)((word >> 24) & 0xFFu);
    }
#pragma unroll
    for (int hq = 0; hq < G; ++hq) {
      const float wgt = s_sc[hq][nl];
#pragma unroll
      for (int e = 0; e < 16; ++e) o[hq][e] = __builtin_fmaf(wgt, vf[e], o[hq][e]);
    }
  }
  // fold the rows held by lanes l, l^32, l^16, l^8 (same channel slice)
#pragma unroll
  for (int m = 32; m >= 8; m >>= 1)
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[hq][e] += __shfl_xor(o[hq][e], m);
  if (lane < 8) {
    const int grp = wave * (8 / LPR) + lane / LPR;
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
      for (int e = 0; e < 16; e += 4)
        *(float4 *)&s_red[grp][hq * D + part * 16 + e] =
            make_float4(o[hq][e], o[hq][e + 1], o[hq][e + 2], o[hq][e + 3]);
  }
  __syncthreads();

  DecWs w = dec_ws(a.ws, a.B * a.Hkv, G, D, S);
  float *myo = w.o + ((size_t)bg * S + split) * G * D;
  for (int idx = t; idx < G * D; idx += kThreads) {
    const int hq = idx / D;
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < NGRP; ++r) s += s_red[r][idx];
    myo[idx] = s - 128.0f * s_wsum[hq];
  }
  if (t < G) w.ml[((size_t)bg * S + split) * G + t] = make_float2(s_m[t], s_l[t]);

}

// Merge of the S split partials of one (batch, kv-head): M = max m_s, weights 2^(m_s - M),
// out = sum_s w_s o_s / sum_s w_s l_s (times the per-channel V scale).  A second launch:
// the kernel boundary is what makes every partial visible, with no device-wide fences.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeLaunch a, int S) {
  const int bg = blockIdx.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ float2 s_ml[kMergeChunk * G];
  __shared__ float s_M[G], s_L[G];
  DecWs w = dec_ws(a.ws, a.B * a.Hkv, G, D, S);

  float oacc[(G * D + kThreads - 1) / kThreads];
#pragma unroll
  for (int k = 0; k < (G * D + kThreads - 1) / kThreads; ++k) oacc[k] = 0.0f;
  if (t < G) { s_M[t] = -INFINITY; s_L[t] = 0.0f; }
  // pass 1: global max per head
  for (int s0 = 0; s0 < S; s0 += kMergeChunk) {
    const int cnt = min(kMergeChunk, S - s0);
    __syncthreads();
    for (int i = t; i < cnt * G; i += kThreads) s_ml[i] = w.ml[((size_t)bg * S + s0) * G + i];
    __syncthreads();
    for (int hq = wave; hq < G; hq += kWavesD) {
      float mx = -INFINITY;
      for (int s = lane; s < cnt; s += 64) mx = fmaxf(mx, s_ml[s * G + hq].x);
      for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
      if (lane == 0) s_M[hq] = fmaxf(s_M[hq], mx);
    }
  }
  // pass 2: weights, denominators and weighted partial outputs (16 loads in flight)
  for (int s0 = 0; s0 < S; s0 += kMergeChunk) {
    const int cnt = min(kMergeChunk, S - s0);
    __syncthreads();
    for (int i = t; i < cnt * G; i += kThreads) {
      const float2 ml = w.ml[((size_t)bg * S + s0) * G + i];
      const float M = s_M[i % G];
      const float f = ml.x == -INFINITY ? 0.0f : fast_exp2(ml.x - M);
      s_ml[i] = make_float2(f, f * ml.y);
    }
    __syncthreads();
    for (int hq = wave; hq < G; hq += kWavesD) {
      float l = 0.0f;
      for (int s = lane; s < cnt; s += 64) l += s_ml[s * G + hq].y;
      for (int m = 32; m >= 1; m >>= 1) l += __shfl_xor(l, m);
      if (lane == 0) s_L[hq] += l;
    }
#pragma unroll
    for (int k = 0; k < (G * D + kThreads - 1) / kThreads; ++k) {
      const int idx = t + k * kThreads;
      if (idx < G * D) {
        const int hq = idx / D;
        const float *po = w.o + ((size_t)bg * S + s0) * G * D + idx;
        float acc = 0.0f;
        int s = 0;
        for (; s + 16 <= cnt; s += 16) {
          float vv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) vv[u] = po[(size_t)(s + u) * G * D];
#pragma unroll
          for (int u = 0; u < 16; ++u) acc = __builtin_fmaf(s_ml[(s + u) * G + hq].x, vv[u], acc);
        }
        for (; s < cnt; ++s) acc = __builtin_fmaf(s_ml[s * G + hq].x, po[(size_t)s * G * D], acc);
        oacc[k] += acc;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < (G * D + kThreads - 1) / kThreads; ++k) {
    const int idx = t + k * kThreads;
    if (idx < G * D) {
      const int hq = idx / D, c = idx % D;
      float r = s_L[hq] > 0.0f ? oacc[k] / s_L[hq] : 0.0f;
      if (a.v_gran == ATTN_Q_GRAN_CHANNEL) r *= ((const float *)a.v_scales)[(size_t)bg * D + c];
      const size_t oi = ((size_t)b * a.Hq + g * G + hq) * D + c;
      if (a.out_f32) ((float *)a.out)[oi] = r;
      else ((__half *)a.out)[oi] = __float2half_rn(r);
    }
  }
}

template <int D, int G>
hipError_t launch_g(const DecodeLaunch &a, hipStream_t s, int S) {
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(S, a.B * a.Hkv), dim3(kThreads), 0, s, a, S);
  hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3(a.B * a.Hkv), dim3(kThreads), 0, s, a, S);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dd(const DecodeLaunch &a, hipStream_t s, int S) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<D, 1>(a, s, S);
    case 2: return launch_g<D, 2>(a, s, S);
    case 4: return launch_g<D, 4>(a, s, S);
    default: return launch_g<D, 8>(a, s, S);
  }
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D, int kv_len) {
  const int G = Hq / Hkv, BH = B * Hkv;
  const int S = (kv_len + KPS - 1) / KPS;
  return align256((size_t)BH * S * G * 8) + align256((size_t)BH * S * G * D * 4);
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t s) {
  const int S = (a.kv_len + KPS - 1) / KPS;
  return a.D == 128 ? launch_dd<128>(a, s, S) : launch_dd<64>(a, s, S);
}

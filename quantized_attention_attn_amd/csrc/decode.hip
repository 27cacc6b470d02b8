// attn_q_decode: one query per head against the int8 KV cache.
//
// "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8", sections "Does
// quantizing attention help decode?" and "What actually changed for decode": at
// batch one attention is a matrix-vector product bound by how fast the KV cache
// streams from memory, so the matrix cores are not used; halving the cache's bytes
// is what speeds it up.
//
// gfx950 mapping.  One workgroup (4 waves) per (batch, kv-head, split of 256 keys):
//   * every thread issues all of its K and V loads up front (16 B per lane, 8
//     consecutive lanes cover one 128-byte code row, so each wave load instruction
//     reads 1 KB of contiguous cache) -- enough bytes in flight to cover HBM latency;
//   * each K row load serves all G query heads of the kv-head: exact int32 dots with
//     v_dot4_i32_i8 reduced over the 8 lanes of the row; scores s = fp32(c_n * acc);
//   * softmax over the split in LDS (max, exp2, sum per head), then PV in fp32 on the
//     dequantized V codes, reduced across rows through LDS;
//   * partial (m, l, o) per split go to the workspace; the last workgroup of each
//     group of 16 splits merges them, and the last of those merges the groups --
//     two short merges spread over workgroups instead of one long serial one, with
//     no extra kernel launch.  Counters return to zero for the next call.
#include "common.h"

using namespace attnq;

namespace {

constexpr int kThreads = 256;
constexpr int KPS = 256;       // keys per split (workgroup)
constexpr int kGroup = 16;     // splits merged by one first-level merger

struct DecWs {
  float *part1;     // [BH][S][G][D+2]   (m, l, o[D])
  float *part2;     // [BH][S2][G][D+2]
  int *cnt1;        // [BH][S2]
  int *cnt2;        // [BH]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline DecWs dec_ws(void *ws, int BH, int G, int D, int S) {
  const int S2 = (S + kGroup - 1) / kGroup;
  char *p = (char *)ws;
  DecWs w;
  w.cnt1 = (int *)p;
  p += align256((size_t)BH * S2 * 4);
  w.cnt2 = (int *)p;
  p += align256((size_t)BH * 4);
  w.part1 = (float *)p;
  p += align256((size_t)BH * S * G * (D + 2) * 4);
  w.part2 = (float *)p;
  return w;
}

// merge `cnt` partials (m, l, o) of stride G*(D+2) floats; thread handles outputs idx
template <int D, int G>
__device__ void merge_partials(const float *src, int cnt, float *dst, bool final_out,
                               const DecodeLaunch &a, int b, int g) {
  const int t = threadIdx.x;
  const int stride = G * (D + 2);
  for (int idx = t; idx < G * D; idx += kThreads) {
    const int hq = idx / D, c = idx % D;
    float M = -INFINITY;
    for (int s = 0; s < cnt; ++s) M = fmaxf(M, __builtin_nontemporal_load(src + (size_t)s * stride + hq * (D + 2)));
    float l = 0.0f, o = 0.0f;
    for (int s = 0; s < cnt; ++s) {
      const float *ps = src + (size_t)s * stride + hq * (D + 2);
      const float ms = __builtin_nontemporal_load(ps);
      const float f = ms == -INFINITY ? 0.0f : fast_exp2(ms - M);
      l += f * __builtin_nontemporal_load(ps + 1);
      o += f * __builtin_nontemporal_load(ps + 2 + c);
    }
    if (!final_out) {
      float *pd = dst + hq * (D + 2);
      if (c == 0) { pd[0] = M; pd[1] = l; }
      pd[2 + c] = o;
    } else {
      const int h = g * G + hq;
      float r = l > 0.0f ? o / l : 0.0f;
      if (a.v_gran == ATTN_Q_GRAN_CHANNEL) r *= ((const float *)a.v_scales)[((size_t)b * a.Hkv + g) * D + c];
      const size_t oi = ((size_t)b * a.Hq + h) * D + c;
      if (a.out_f32) ((float *)a.out)[oi] = r;
      else ((__half *)a.out)[oi] = __float2half_rn(r);
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeLaunch a, int S) {
  constexpr int LPR = D / 16;            // lanes per code row (16 B each)
  constexpr int RPP = kThreads / LPR;    // rows per pass
  constexpr int NPASS = KPS / RPP;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int part = t % LPR, rsub = t / LPR;
  const int n0 = split * KPS;

  __shared__ __attribute__((aligned(16))) int8_t s_q8[G][D];
  __shared__ float s_c[G];
  __shared__ float s_sc[G][KPS];
  __shared__ float s_m[G], s_l[G];
  constexpr int NGRP = (kThreads / 64) * (16 / LPR);  // row groups left after two lane folds
  __shared__ float s_red[NGRP][G * D];               // [row group][hq][channel]
  __shared__ int s_last;

  // ---- issue every K and V load of the split first
  const size_t cbase = (size_t)bg * a.cap * D;
  v4i kr[NPASS], vr[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int n = n0 + ps * RPP + rsub;
    if (n < a.kv_len) {
      kr[ps] = *(const v4i *)(a.k_codes + cbase + (size_t)n * D + part * 16);
      vr[ps] = *(const v4i *)(a.v_codes + cbase + (size_t)n * D + part * 16);
    } else {
      kr[ps] = v4i{};
      vr[ps] = v4i{};
    }
  }

  // ---- quantize q per head (wave w handles heads w, w+4, ...)
  for (int hq = wave; hq < G; hq += kThreads / 64) {
    const int h = g * G + hq;
    const uint16_t *qp = a.q + ((size_t)b * a.Hq + h) * D;
    float x[D / 64];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      const int c = lane * (D / 64) + e;
      float v = __half2float(__ushort_as_half(qp[c]));
      if (a.k_gran == ATTN_Q_GRAN_CHANNEL) v = v * ((const float *)a.k_scales)[(size_t)bg * D + c];
      x[e] = v;
      amax = fmaxf(amax, fabsf(v));
    }
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float sq = amax / 127.0f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) s_q8[hq][lane * (D / 64) + e] = (int8_t)quant_i8(x[e], sq);
    if (lane == 0) s_c[hq] = sq * a.kconst;
  }
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
    float ksc = 1.0f;
    if (a.k_gran == ATTN_Q_GRAN_TOKEN && valid)
      ksc = __half2float(((const __half *)a.k_scales)[(size_t)bg * a.cap + n]);
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

  // ---- softmax over the split, per head
  for (int hq = wave; hq < G; hq += kThreads / 64) {
    float mx = -INFINITY;
    for (int j = lane; j < KPS; j += 64) mx = fmaxf(mx, s_sc[hq][j]);
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    float sum = 0.0f;
    for (int j = lane; j < KPS; j += 64) {
      const float sv = s_sc[hq][j];
      const float p = sv == -INFINITY ? 0.0f : fast_exp2(sv - mx);
      sum += p;
      float w = p;
      if (a.v_gran == ATTN_Q_GRAN_TOKEN && n0 + j < a.kv_len)
        w = p * __half2float(((const __half *)a.v_scales)[(size_t)bg * a.cap + n0 + j]);
      s_sc[hq][j] = w;
    }
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
    if (lane == 0) { s_m[hq] = mx; s_l[hq] = sum; }
  }
  __syncthreads();

  // ---- PV on the dequantized codes (fp32)
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
      const int word = vr[ps][w];
#pragma unroll
      for (int e = 0; e < 4; ++e) vf[4 * w + e] = (float)(int8_t)((word >> (8 * e)) & 0xFF);
    }
#pragma unroll
    for (int hq = 0; hq < G; ++hq) {
      const float wgt = s_sc[hq][nl];
#pragma unroll
      for (int e = 0; e < 16; ++e) o[hq][e] = __builtin_fmaf(wgt, vf[e], o[hq][e]);
    }
  }
  // fold rows held by lanes l, l^32, l^16 (same channel slice: LPR divides 16)
#pragma unroll
  for (int m = 32; m >= 16; m >>= 1)
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[hq][e] += __shfl_xor(o[hq][e], m);
  if (lane < 16) {
    const int grp = wave * (16 / LPR) + lane / LPR;
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
      for (int e = 0; e < 16; e += 4)
        *(float4 *)&s_red[grp][hq * D + part * 16 + e] =
            make_float4(o[hq][e], o[hq][e + 1], o[hq][e + 2], o[hq][e + 3]);
  }
  __syncthreads();

  DecWs w = dec_ws(a.ws, a.B * a.Hkv, G, D, S);
  const int S2 = (S + kGroup - 1) / kGroup;
  float *my = w.part1 + ((size_t)bg * S + split) * G * (D + 2);
  for (int idx = t; idx < G * D; idx += kThreads) {
    const int hq = idx / D, c = idx % D;
    float s = 0.0f;
    for (int r = 0; r < NGRP; ++r) s += s_red[r][hq * D + c];
    my[hq * (D + 2) + 2 + c] = s;
    if (c == 0) { my[hq * (D + 2)] = s_m[hq]; my[hq * (D + 2) + 1] = s_l[hq]; }
  }

  // ---- level-1 merge by the last workgroup of each group of kGroup splits
  const int grp = split / kGroup;
  const int gsize = min(kGroup, S - grp * kGroup);
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const int old = atomicAdd(&w.cnt1[bg * S2 + grp], 1);
    s_last = old == gsize - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  float *g2 = w.part2 + ((size_t)bg * S2 + grp) * G * (D + 2);
  merge_partials<D, G>(w.part1 + ((size_t)bg * S + grp * kGroup) * G * (D + 2), gsize, g2, false, a, b, g);
  if (t == 0) w.cnt1[bg * S2 + grp] = 0;

  // ---- level-2 merge by the last first-level merger
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const int old = atomicAdd(&w.cnt2[bg], 1);
    s_last = old == S2 - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  merge_partials<D, G>(w.part2 + (size_t)bg * S2 * G * (D + 2), S2, nullptr, true, a, b, g);
  if (t == 0) w.cnt2[bg] = 0;
}

template <int D, int G>
hipError_t launch_g(const DecodeLaunch &a, hipStream_t s, int S) {
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(S, a.B * a.Hkv), dim3(kThreads), 0, s, a, S);
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
  const int S2 = (S + kGroup - 1) / kGroup;
  return align256((size_t)BH * S2 * 4) + align256((size_t)BH * 4) +
         align256((size_t)BH * S * G * (D + 2) * 4) + align256((size_t)BH * S2 * G * (D + 2) * 4);
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t s) {
  const int S = (a.kv_len + KPS - 1) / KPS;
  return a.D == 128 ? launch_dd<128>(a, s, S) : launch_dd<64>(a, s, S);
}

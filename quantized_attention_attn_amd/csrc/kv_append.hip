// attn_q_kv_append_i8: append fp16 K/V rows to the int8 cache, shifting K by the running
// per-channel mean kept in the cache header ("int8 Flash Attention on RDNA4: QK Wants
// Integers, PV Wants FP8", section "K's outliers, and the subtraction softmax does not
// notice": during decode K arrives one token at a time and the header mean lags by one).
//
// Token n is shifted by the mean of the n keys before it, so each token needs the exact
// sum S_n of those keys.  The fixed-point sum (fp16 * 2^24 in int64) is associative, so
// S_n is a parallel prefix scan whose value does not depend on how the scan is split:
//   - one new token (the decode step) takes one single-wave launch: its prefix is the
//     header itself;
//   - up to 64 new tokens take one launch: a workgroup per (batch, kv-head) scans its
//     tokens through LDS, writes codes and per-token scales, then the new header;
//   - longer appends take three: 64-token chunk sums, an exclusive scan over the chunks
//     (which also writes the new header), then the codes with each chunk's prefix.
// The work is a few bytes per element; one pass over the new rows, no matrix cores.
#include "common.h"

using namespace attnq;

namespace {

constexpr int kChunk = 64;                        // tokens per workgroup
constexpr int kGroups = 64;                       // row groups per workgroup
constexpr int kRowsPerThread = kChunk / kGroups;  // one row per thread: the per-row chain
                                                  // (8 fp64 divisions) is the latency

template <int D> constexpr int lanes_per_row() { return D / 8; }   // 8 channels per lane
template <int D> constexpr int app_threads() { return kGroups * lanes_per_row<D>(); }

// (1) chunk sums: csum[bg][j][c] = sum over chunk j's tokens of k * 2^24.   grid BH * nch
template <int D>
__global__ __launch_bounds__(app_threads<D>()) void kva_chunk_sums(const uint16_t *__restrict__ k, int T,
                                                                  int nch, long long *__restrict__ csum) {
  constexpr int LPR = lanes_per_row<D>();
  const int bg = blockIdx.x / nch, j = blockIdx.x % nch;
  const int t = threadIdx.x, part = t % LPR, grp = t / LPR;
  long long sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0;
  const size_t in_base = (size_t)bg * T * D;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = j * kChunk + grp * kRowsPerThread + i;
    if (r < T) {
      const v4i x = *(const v4i *)(k + in_base + (size_t)r * D + part * 8);
      const uint16_t *h = (const uint16_t *)&x;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += f16_times_2p24(h[e]);
    }
  }
  __shared__ long long s_tot[kGroups][D];
#pragma unroll
  for (int e = 0; e < 8; ++e) s_tot[grp][part * 8 + e] = sum[e];
  __syncthreads();
  for (int c = t; c < D; c += app_threads<D>()) {
    long long S = 0;
    for (int g = 0; g < kGroups; ++g) S += s_tot[g][c];
    csum[((size_t)bg * nch + j) * D + c] = S;
  }
}

// (2) exclusive scan over the chunks, in place, starting from the header; the header then
// receives the total and k_mean its mean.   grid BH, block D (one thread per channel)
__global__ void kva_scan(int nch, int D, long long n_total, long long *__restrict__ csum,
                         long long *__restrict__ k_sum, float *__restrict__ k_mean) {
  const int bg = blockIdx.x, c = threadIdx.x;
  const size_t h = (size_t)bg * D + c;
  long long run = k_sum[h];
  long long *p = csum + (size_t)bg * nch * D + c;
  for (int j0 = 0; j0 < nch; j0 += 8) {
    long long x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = j0 + u < nch ? p[(size_t)(j0 + u) * D] : 0ll;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < nch) {
        p[(size_t)(j0 + u) * D] = run;
        run += x[u];
      }
  }
  k_sum[h] = run;
  if (k_mean) k_mean[h] = mean_from_sum(run, n_total);
}

// (3) codes of one chunk.  kSingle: the only chunk of its (b, g); the starting prefix is the
// header, and the thread that reads a channel's header also writes its new value.
// Otherwise the starting prefix is the chunk's entry of the scanned chunk sums.
// grid BH * nch; thread (part, grp) owns channels part*8 .. +7 of row grp of the chunk.
// Only valid rows (r < T, a prefix) do the shift, the quantization and the stores; the LPR
// lanes of a row share its validity, so the lane shuffles never mix valid and idle lanes.
template <int D, bool kSingle>
__global__ __launch_bounds__(app_threads<D>()) void kva_codes(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int T, int nch, int n_before, int cap,
    long long *__restrict__ k_sum, const long long *__restrict__ cprefix, float *__restrict__ k_mean,
    int8_t *__restrict__ k_codes, int8_t *__restrict__ v_codes, __half *__restrict__ k_scales,
    __half *__restrict__ v_scales) {
  constexpr int LPR = lanes_per_row<D>();
  const int bg = blockIdx.x / nch, j = blockIdx.x % nch;
  const int t = threadIdx.x, part = t % LPR, grp = t / LPR;
  __shared__ long long s_tot[kGroups][D];
  long long base = 0;
  if (t < D) base = kSingle ? k_sum[(size_t)bg * D + t] : cprefix[((size_t)bg * nch + j) * D + t];

  const size_t in_base = (size_t)bg * T * D;
  const size_t out_base = (size_t)bg * cap * D;
  v4i kin[kRowsPerThread], vin[kRowsPerThread];
  const int r0 = j * kChunk + grp * kRowsPerThread;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = min(r0 + i, T - 1);   // rows >= T are loaded from row T-1 and never used
    kin[i] = *(const v4i *)(k + in_base + (size_t)r * D + part * 8);
    vin[i] = *(const v4i *)(v + in_base + (size_t)r * D + part * 8);
  }
  long long S[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) S[e] = 0;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    if (r0 + i < T) {
      const uint16_t *h = (const uint16_t *)&kin[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) S[e] += f16_times_2p24(h[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_tot[grp][part * 8 + e] = S[e];
  __syncthreads();
  // exclusive scan over the row groups, one thread per channel, in place
  if (t < D) {
    long long run = base;
    for (int g0 = 0; g0 < kGroups; g0 += 16) {
      long long x[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = s_tot[g0 + u][t];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        s_tot[g0 + u][t] = run;
        run += x[u];
      }
    }
    if (kSingle) {
      const size_t h = (size_t)bg * D + t;
      k_sum[h] = run;
      if (k_mean) k_mean[h] = mean_from_sum(run, (long long)n_before + T);
    }
  }
  __syncthreads();
  // S = sum of the keys before this thread's first row
#pragma unroll
  for (int e = 0; e < 8; ++e) S[e] = s_tot[grp][part * 8 + e];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = r0 + i;
    if (r >= T) break;
    const long long n = (long long)n_before + r;
    const uint16_t *kh = (const uint16_t *)&kin[i];
    const uint16_t *vh = (const uint16_t *)&vin[i];
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
    // per-token scales: absmax over the LPR consecutive lanes that hold the row
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      ka = fmaxf(ka, __shfl_xor(ka, m));
      va = fmaxf(va, __shfl_xor(va, m));
    }
    const __half ksh = __float2half_rn(ka / 127.0f), vsh = __float2half_rn(va / 127.0f);
    const float ks = __half2float(ksh), vs = __half2float(vsh);
    const float krs = 1.0f / ks, vrs = 1.0f / vs;
    uint32_t kw[2] = {0u, 0u}, vw[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kw[e / 4] |= (uint32_t)(quant_i8_rcp(kx[e], ks, krs) & 0xFF) << (8 * (e % 4));
      vw[e / 4] |= (uint32_t)(quant_i8_rcp(vx[e], vs, vrs) & 0xFF) << (8 * (e % 4));
    }
    *(uint2 *)(k_codes + out_base + (size_t)n * D + part * 8) = make_uint2(kw[0], kw[1]);
    *(uint2 *)(v_codes + out_base + (size_t)n * D + part * 8) = make_uint2(vw[0], vw[1]);
    if (part == 0) {
      k_scales[(size_t)bg * cap + n] = ksh;
      v_scales[(size_t)bg * cap + n] = vsh;
    }
  }
}

// One new token (the decode step): its prefix is the header itself, so no scan is needed.
// LPR lanes per (b, g), 64 / LPR of them per wave; no LDS, no barrier.   grid ceil(BH * LPR / 64)
template <int D>
__global__ __launch_bounds__(64) void kva_one(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                              int BH, int n, int cap, long long *__restrict__ k_sum,
                                              float *__restrict__ k_mean, int8_t *__restrict__ k_codes,
                                              int8_t *__restrict__ v_codes, __half *__restrict__ k_scales,
                                              __half *__restrict__ v_scales) {
  constexpr int LPR = lanes_per_row<D>();
  const int gi = blockIdx.x * 64 + threadIdx.x;
  const int bg = gi / LPR, part = gi % LPR;
  if (bg >= BH) return;   // whole rows leave together, so the row shuffles below stay within live lanes
  const size_t h0 = (size_t)bg * D + part * 8;
  const v4i kr = *(const v4i *)(k + h0);   // k, v are [BH][1][D]
  const v4i vr = *(const v4i *)(v + h0);
  long long S[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) S[e] = k_sum[h0 + e];
  uint32_t kw[2], vw[2];
  __half ksh, vsh;
  append_row<LPR>((const uint16_t *)&kr, (const uint16_t *)&vr, S, n, kw, vw, ksh, vsh);
  const size_t row = ((size_t)bg * cap + n) * D + part * 8;
  *(uint2 *)(k_codes + row) = make_uint2(kw[0], kw[1]);
  *(uint2 *)(v_codes + row) = make_uint2(vw[0], vw[1]);
  if (part == 0) {
    k_scales[(size_t)bg * cap + n] = ksh;
    v_scales[(size_t)bg * cap + n] = vsh;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    k_sum[h0 + e] = S[e];
    if (k_mean) k_mean[h0 + e] = mean_from_sum(S[e], (long long)n + 1);
  }
}

template <int D>
hipError_t launch_d(const KvAppendLaunch &a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int nch = (a.T + kChunk - 1) / kChunk;
  __half *ksc = (__half *)a.k_scales, *vsc = (__half *)a.v_scales;
  long long *hdr = (long long *)a.k_sum;
  if (a.T == 1) {
    const int blocks = (BH * lanes_per_row<D>() + 63) / 64;
    hipLaunchKernelGGL(kva_one<D>, dim3(blocks), dim3(64), 0, s, a.k, a.v, BH, a.n_before, a.cap, hdr,
                       a.k_mean, a.k_codes, a.v_codes, ksc, vsc);
    return hipGetLastError();
  }
  if (nch == 1) {
    hipLaunchKernelGGL((kva_codes<D, true>), dim3(BH), dim3(app_threads<D>()), 0, s, a.k, a.v, a.T, 1,
                       a.n_before, a.cap, hdr, (const long long *)nullptr, a.k_mean, a.k_codes, a.v_codes,
                       ksc, vsc);
    return hipGetLastError();
  }
  long long *csum = (long long *)a.ws;
  hipLaunchKernelGGL(kva_chunk_sums<D>, dim3(BH * nch), dim3(app_threads<D>()), 0, s, a.k, a.T, nch, csum);
  hipLaunchKernelGGL(kva_scan, dim3(BH), dim3(D), 0, s, nch, D, (long long)a.n_before + a.T, csum, hdr,
                     a.k_mean);
  hipLaunchKernelGGL((kva_codes<D, false>), dim3(BH * nch), dim3(app_threads<D>()), 0, s, a.k, a.v, a.T,
                     nch, a.n_before, a.cap, (long long *)nullptr, (const long long *)csum, a.k_mean,
                     a.k_codes, a.v_codes, ksc, vsc);
  return hipGetLastError();
}

}  // namespace

size_t kv_append_workspace_bytes(int B, int H, int D, int T) {
  if (T <= kChunk) return 0;
  const size_t nch = ((size_t)T + kChunk - 1) / kChunk;
  return (size_t)B * H * nch * D * sizeof(long long);
}

hipError_t launch_kv_append(const KvAppendLaunch &a, hipStream_t s) {
  return a.D == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

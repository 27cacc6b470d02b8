// attn_q_short_fused: quantized attention for short sequences, one workgroup per head and
// one pass over HBM (fp16 Q, K, V in, O out).
//
// The method is the one of attn_q_prefill ("int8 Flash Attention on RDNA4: QK Wants
// Integers, PV Wants FP8": K's per-channel mean subtracted, int8 QK^T with exact int32
// sums, fp32 softmax, P as e4m3 with the static scale 448, PV on fp8), at the shapes of the
// vision workloads of "QFlash: Bridging Quantization and Memory Efficiency in Vision
// Transformer Attention" (Table 1: ViT/DeiT heads of 197 tokens, d = 64; Swin windows of
// 49 tokens, d = 32).  A head of at most 256 keys fits in one workgroup, so its
// quantization is done in the same kernel and the key loop of QFlash's Algorithm 1 is a
// single block: the row max is exact before any exponential, so nothing is rescaled.
//
// Phases (256 threads):
//   1. each thread loads 8 channels of some K and V rows (registers), accumulates the
//      exact sum of K (in fp64, exact for N <= 256), K's max and min and |V|'s max; the
//      partials meet in LDS;
//   2. per channel: mu = fp32(S / N), s_K = fp32(amax(k - mu) / 127)
//      (the centred amax from the extrema: x -> fl(x - mu) is monotone), s_V = fp32(amax / 127);
//   3. the K codes go to LDS row-major, the V codes as e4m3 in the matrix-core operand
//      order (the permuted key order of kv_quantize_i8's v_op), over the statistics area;
//   4. each wave takes blocks of 32 query rows: q' = q * s_K per channel, int8 per row in
//      registers, S^T = K Q^T on v_mfma_i32_32x32x32_i8 for every key, the row max,
//      p = exp2(c*acc - (m - log2 448)) -> e4m3, O^T = V^T P^T on the fp8 matrix core,
//      l from an operand of ones, out = O * s_V / l.
#include <climits>

#include "common.h"

using namespace attnq;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int KT = 64;                    // keys per PV matrix-core step
constexpr int kBiasBits = 0x4B400000;     // fp32 1.5 * 2^23: biased QK accumulators (as prefill)
constexpr float kBias = 12582912.0f;
constexpr float kLog2_448 = 8.807354922057604f;

// LDS map of one head: statistics (phases 1-2) and, over them, the operands (phases 3-4).
// Phase 1 deals the keys to threads in groups of 4 consecutive keys (the 4 keys whose V
// bytes are adjacent in the PV operand row, so V is written as words): thread (part, rg)
// owns channels part*8 .. +7 of groups rg, rg + RG, ...
template <int D, int NT>
struct Lds {
  static constexpr int LPR = D / 8;              // lanes per key, 8 channels each
  static constexpr int RG = kThreads / LPR;      // key groups in flight (32 or 64)
  static constexpr int NP = NT * KT;             // padded keys
  static constexpr int NG = NP / 4;              // 4-key groups
  static constexpr int GPT = (NG + RG - 1) / RG; // groups per thread
  static constexpr int RED = kThreads / D;       // threads per channel in the reduction
  static constexpr int RGU = RG < NG ? RG : NG;  // key groups that hold keys (partials kept)
  static constexpr int KSTR = D + 16;            // K code row stride (bytes): 16-byte reads of
                                                 // consecutive rows start on different banks
  static constexpr int VSTR = KT + 16;           // V operand row stride (bytes)
  static constexpr int STAT_BYTES = RGU * D * (8 + 4 + 4 + 4);
  static constexpr int K_BYTES = NP * KSTR;
  static constexpr int V_BYTES = NT * D * VSTR;
  static constexpr int OPS_BYTES = K_BYTES + V_BYTES;
  static constexpr int BYTES = STAT_BYTES > OPS_BYTES ? STAT_BYTES : OPS_BYTES;
  static_assert(RGU % RED == 0, "whole reduction slices");
};

// key r of a 64-key tile -> its byte position in the PV operand row (inverse of the
// permutation perm(p) = 32*((p%32)/16) + 8*((p%16)/4) + 4*(p/32) + p%4)
__device__ __forceinline__ int vop_pos(int r) {
  const int j = r >> 5, a = (r >> 3) & 3, h = (r >> 2) & 1, b = r & 3;
  return 32 * h + 16 * j + 4 * a + b;
}

template <int D, int NT, bool DEBUG>
__global__ __launch_bounds__(kThreads) void short_fused_kernel(const uint16_t *__restrict__ q,
                                                               const uint16_t *__restrict__ k,
                                                               const uint16_t *__restrict__ v, int N,
                                                               float kconst, void *__restrict__ out,
                                                               int out_f32, int32_t *__restrict__ ds) {
  // every product is rounded as written: m = fp32(c * acc_max) must stay a rounded value
  // before log2(448) - m, which contraction into one fma would skip
#pragma clang fp contract(off)
  using L = Lds<D, NT>;
  constexpr int LPR = L::LPR, RG = L::RG, RGU = L::RGU, GPT = L::GPT, NK = D / 32;
  __shared__ __align__(16) uint8_t s_raw[L::BYTES];
  __shared__ double s_psum[L::RED][D];
  __shared__ float s_pmx[L::RED][D], s_pmn[L::RED][D], s_pva[L::RED][D];
  __shared__ float s_mu[D], s_sk[D], s_rk[D], s_sv[D], s_rv[D];
  double(*s_sum)[D] = (double(*)[D])s_raw;
  float(*s_kmx)[D] = (float(*)[D])(s_raw + RGU * D * 8);
  float(*s_kmn)[D] = (float(*)[D])(s_raw + RGU * D * 12);
  float(*s_vam)[D] = (float(*)[D])(s_raw + RGU * D * 16);
  uint8_t *s_k = s_raw;
  uint8_t *s_v = s_raw + L::K_BYTES;

  const int bh = blockIdx.x;
  const int t = threadIdx.x, part = t % LPR, rg = t / LPR;
  const int wv = t >> 6, lane = t & 63, col = lane & 31, hh = lane >> 5;
  const size_t base = (size_t)bh * N * D;
  const int nrb = (N + 31) / 32;

  // ---- 1. K / V rows into registers (4 consecutive keys per group), statistics
  v4i kin[GPT][4], vin[GPT][4];
  // K's channel sums in fp64: every fp16 is a multiple of 2^-24 below 2^16, so any sum of at
  // most 256 of them (N <= 256) is a multiple of 2^-24 below 2^24 and every partial sum is
  // exact; fp32(S / N) is then the mean of the exact int64 fixed-point sum used elsewhere
  double sum[8];
  float kmx[8], kmn[8], vam[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sum[e] = 0.0;
    kmx[e] = -INFINITY;
    kmn[e] = INFINITY;
    vam[e] = 0.0f;
  }
#pragma unroll
  for (int g = 0; g < GPT; ++g)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 4 * (rg + g * RG) + u;
      kin[g][u] = v4i{0, 0, 0, 0};
      vin[g][u] = v4i{0, 0, 0, 0};
      if (r < N) {
        kin[g][u] = *(const v4i *)(k + base + (size_t)r * D + part * 8);
        vin[g][u] = *(const v4i *)(v + base + (size_t)r * D + part * 8);
      }
    }
  // this wave's first block of 32 query rows, requested after K and V so that the statistics
  // wait only for K and V (the second block is requested when the attention starts)
  v4i qraw[2][NK][2];
  auto load_q = [&](int s2) {
    const int ii = min((wv + s2 * kWaves) * 32 + col, N - 1);   // rows past N repeat row N-1
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const uint16_t *qp = q + base + (size_t)ii * D + 32 * kk + 16 * hh;
      qraw[s2][kk][0] = v4i{0, 0, 0, 0};
      qraw[s2][kk][1] = v4i{0, 0, 0, 0};
      if (wv + s2 * kWaves < nrb) {
        qraw[s2][kk][0] = *(const v4i *)qp;
        qraw[s2][kk][1] = *(const v4i *)(qp + 8);
      }
    }
  };
  load_q(0);
#pragma unroll
  for (int g = 0; g < GPT; ++g)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (4 * (rg + g * RG) + u < N) {
        const uint16_t *kh = (const uint16_t *)&kin[g][u];
        const uint16_t *vh = (const uint16_t *)&vin[g][u];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kf = __half2float(__ushort_as_half(kh[e]));
          sum[e] += (double)kf;
          kmx[e] = fmaxf(kmx[e], kf);
          kmn[e] = fminf(kmn[e], kf);
          vam[e] = fmaxf(vam[e], fabsf(__half2float(__ushort_as_half(vh[e]))));
        }
      }
    }
  // (groups rg >= RGU start past the padded keys: they hold no key and keep no partials)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = part * 8 + e;
    if (rg >= RGU) break;
    s_sum[rg][c] = sum[e];
    s_kmx[rg][c] = kmx[e];
    s_kmn[rg][c] = kmn[e];
    s_vam[rg][c] = vam[e];
  }
  __syncthreads();

  // ---- 2. means and scales: RED threads per channel reduce slices of the partials, then
  // one thread per channel
  {
    const int c = t % D, sl = t / D;
    constexpr int PER = RGU / L::RED;
    double S = 0.0;
    float hi = -INFINITY, lo = INFINITY, va = 0.0f;
#pragma unroll
    for (int r = sl * PER; r < (sl + 1) * PER; ++r) {
      S += s_sum[r][c];
      hi = fmaxf(hi, s_kmx[r][c]);
      lo = fminf(lo, s_kmn[r][c]);
      va = fmaxf(va, s_vam[r][c]);
    }
    s_psum[sl][c] = S;
    s_pmx[sl][c] = hi;
    s_pmn[sl][c] = lo;
    s_pva[sl][c] = va;
  }
  __syncthreads();
  if (t < D) {
    double S = 0.0;
    float hi = -INFINITY, lo = INFINITY, va = 0.0f;
#pragma unroll
    for (int r = 0; r < L::RED; ++r) {
      S += s_psum[r][t];
      hi = fmaxf(hi, s_pmx[r][t]);
      lo = fminf(lo, s_pmn[r][t]);
      va = fmaxf(va, s_pva[r][t]);
    }
    const float mu = (float)(S / (double)N);
    const float sk = fmaxf(fabsf(hi - mu), fabsf(lo - mu)) / 127.0f;
    const float sv = va / 127.0f;
    s_mu[t] = mu;
    s_sk[t] = sk;
    s_rk[t] = rcp_or_zero(sk);
    s_sv[t] = sv;
    s_rv[t] = rcp_or_zero(sv);
  }
  __syncthreads();

  // ---- 3. operands: K codes row-major; V codes as e4m3 in the PV operand order, one
  // 32-bit word per channel and group of 4 keys (keys past N are zero)
  {
    float mu[8], sk[8], rk[8], sv[8], rv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = part * 8 + e;
      mu[e] = s_mu[c];
      sk[e] = s_sk[c];
      rk[e] = s_rk[c];
      sv[e] = s_sv[c];
      rv[e] = s_rv[c];
    }
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
      const int gi = rg + g * RG;
      if (gi < L::NG) {
        uint32_t vw[8];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {       // keys 4gi + 2h2, 4gi + 2h2 + 1 -> bytes 2h2, 2h2 + 1
          float vv[2][8];
#pragma unroll
          for (int u2 = 0; u2 < 2; ++u2) {
            const int u = 2 * h2 + u2, r = 4 * gi + u;
            // rows past N were loaded as zeros: their V codes are 0, and their K codes (any
            // bytes) only feed scores that are masked
            const uint16_t *kh = (const uint16_t *)&kin[g][u];
            const uint16_t *vh = (const uint16_t *)&vin[g][u];
            uint32_t kw[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float kx = __half2float(__ushort_as_half(kh[e])) - mu[e];
              kw[e / 4] |= quant_i8_byte(kx, sk[e], rk[e]) << (8 * (e % 4));
              vv[u2][e] = quant_i8_val(__half2float(__ushort_as_half(vh[e])), sv[e], rv[e]);
            }
            *(uint2 *)(s_k + r * L::KSTR + part * 8) = make_uint2(kw[0], kw[1]);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vw[e] = h2 == 0 ? (uint32_t)cvt_pk_e4m3<false>(vv[0][e], vv[1][e], 0)
                            : (uint32_t)cvt_pk_e4m3<true>(vv[0][e], vv[1][e], (int)vw[e]);
        }
        const int tile = (4 * gi) / KT, pos = vop_pos((4 * gi) % KT);   // 4 adjacent bytes
#pragma unroll
        for (int e = 0; e < 8; ++e) *(uint32_t *)(s_v + (tile * D + part * 8 + e) * L::VSTR + pos) = vw[e];
      }
    }
  }
  __syncthreads();

  // ---- 4. attention, 32 query rows per wave and step
  load_q(1);
  const v16i bias = v16i{kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits,
                         kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits, kBiasBits};
  const int one8 = 0x38383838;   // e4m3 1.0 in every byte
  const v8i ones = v8i{one8, one8, one8, one8, one8, one8, one8, one8};
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int rb = wv + s2 * kWaves;
    if (rb >= nrb) break;
    const int i = rb * 32 + col;
    // q' = fp32(q) * s_K per channel, per-row int8 (the row's lanes are col and col + 32)
    float qq[NK][16];
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int c0 = 32 * kk + 16 * hh;
      const uint16_t *ha = (const uint16_t *)&qraw[s2][kk][0];
      const uint16_t *hb = (const uint16_t *)&qraw[s2][kk][1];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = __half2float(__ushort_as_half(e < 8 ? ha[e] : hb[e - 8])) * s_sk[c0 + e];
        qq[kk][e] = x;
        amax = fmaxf(amax, fabsf(x));
      }
    }
    amax = fmaxf(amax, max_xor32(amax));
    const float sq = amax / 127.0f, rq = rcp_or_zero(sq);
    v4i qop[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) word |= quant_i8_byte(qq[kk][4 * w + e], sq, rq) << (8 * e);
        qop[kk][w] = (int)word;
      }
    const float c = sq * kconst;

    // S^T = K Q^T of key tile tt: lane holds query col and keys 64tt + 32j + 8(e>>2) + 4hh + (e&3);
    // the padded keys of the last tile read INT_MIN.  Computed twice (a pass for the row max,
    // a pass for P): the matrix-core work is small and only one tile's scores stay live.
    auto qk = [&](int tt, v16i (&S)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint8_t *kr = s_k + (tt * KT + 32 * j + col) * L::KSTR + 16 * hh;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          S[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(*(const v4i *)(kr + 32 * kk), qop[kk],
                                                       kk == 0 ? bias : S[j], 0, 0, 0);
      }
      if (tt == NT - 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (tt * KT + 32 * j + 8 * (e >> 2) + 4 * hh + (e & 3) >= N) S[j][e] = INT_MIN;
      }
    };
    int mx = INT_MIN;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      v16i S[2];
      qk(tt, S);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (DEBUG && ds && i < N && S[j][e] != INT_MIN)
            ds[((size_t)bh * N + i) * N + tt * KT + 32 * j + 8 * (e >> 2) + 4 * hh + (e & 3)] = S[j][e] - kBiasBits;
          mx = max(mx, S[j][e]);
        }
    }
    mx = max_xor32(mx);
    // (a compiler barrier: the second pass re-reads the K operands instead of keeping the
    // first pass's scores live)
    asm volatile("" ::: "memory");
    // (biased scores order like the scores; every row sees at least key 0)
    const float m = c * (__int_as_float(mx) - kBias);
    const float negmL = kLog2_448 - m;   // = -fp32(m - log2 448), exactly
    v16f O[NK];
#pragma unroll
    for (int mt = 0; mt < NK; ++mt) O[mt] = v16f{};
    v16f lsum = v16f{};
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      v16i S[2];
      qk(tt, S);
      v8i P;
      // (a 32-key half of the last tile that lies wholly past N keeps P = 0 without exp2)
      const bool hi_live = tt < NT - 1 || tt * KT + 32 < N;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int j = w >> 2, r0 = (w & 3) * 4;
        if (j == 1 && !hi_live) {
          P[w] = 0;
          continue;
        }
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sc = S[j][r0 + e];
          // fp32(c * acc - mL) with one rounding; (B + acc) - B = acc exactly
          const float pe = fast_exp2(__builtin_fmaf(c, __int_as_float(sc) - kBias, negmL));
          p[e] = (tt == NT - 1 && sc == INT_MIN) ? 0.0f : pe;   // (padded keys: last tile only)
        }
        const int word = cvt_pk_e4m3<false>(p[0], p[1], 0);
        P[w] = cvt_pk_e4m3<true>(p[2], p[3], word);
      }
#pragma unroll
      for (int mt = 0; mt < NK; ++mt) {
        const uint8_t *vr = s_v + (tt * D + 32 * mt + col) * L::VSTR + 32 * hh;
        const v4i lo = *(const v4i *)vr;
        const v4i hi = *(const v4i *)(vr + 16);
        const v8i vop = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        O[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, P, O[mt], 0, 0, 0, 0, 0, 0);
      }
      lsum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, P, lsum, 0, 0, 0, 0, 0, 0);
    }
    if (i < N) {
      const float rl = 1.0f / lsum[0];
      const size_t orow = (base + (size_t)i * D);
#pragma unroll
      for (int mt = 0; mt < NK; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = 32 * mt + 8 * g + 4 * hh;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = O[mt][4 * g + e] * s_sv[c0 + e] * rl;
          if (out_f32) {
            *(v4f *)((float *)out + orow + c0) = v4f{o[0], o[1], o[2], o[3]};
          } else {
            __half2 h01 = __floats2half2_rn(o[0], o[1]), h23 = __floats2half2_rn(o[2], o[3]);
            *(uint2 *)((__half *)out + orow + c0) =
                make_uint2(*(const uint32_t *)&h01, *(const uint32_t *)&h23);
          }
        }
    }
  }
}

template <int D>
hipError_t launch_d(const ShortLaunch &a, hipStream_t s) {
  const int nt = (a.N + KT - 1) / KT;
  const dim3 g(a.B * a.H), b(kThreads);
#define SHORT_CASE(NT_)                                                                               \
  case NT_:                                                                                           \
    if (a.debug_s)                                                                                    \
      hipLaunchKernelGGL((short_fused_kernel<D, NT_, true>), g, b, 0, s, a.q, a.k, a.v, a.N, a.kconst, \
                         a.out, a.out_f32, a.debug_s);                                                \
    else                                                                                              \
      hipLaunchKernelGGL((short_fused_kernel<D, NT_, false>), g, b, 0, s, a.q, a.k, a.v, a.N,          \
                         a.kconst, a.out, a.out_f32, a.debug_s);                                      \
    break;
  switch (nt) {
    SHORT_CASE(1)
    SHORT_CASE(2)
    SHORT_CASE(3)
    SHORT_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef SHORT_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_short_fused(const ShortLaunch &a, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, s) : launch_d<32>(a, s);
}

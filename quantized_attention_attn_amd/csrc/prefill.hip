// attn_q_prefill: fused int8-QK^T / fp32 online softmax / e4m3-P fp8-PV flash attention.
//
// Method: "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8" -- QK^T on
// int8 with int32 accumulation after K-mean subtraction; running row max m and
// exp(s - m) in fp32 so P <= 1 and its scale is a constant (section "The scale P
// needs is already sitting in a register"); P as e4m3 with static scale 448 and PV
// on fp8 (section "fp8 is not faster, it is shaped correctly").  The tiled loop over
// key blocks, the int32 row max and the exp2 with s_Q*s_K*d^-1/2*log2(e) folded in
// follow Algorithm 1 and eq. (3)-(4) of "QFlash: Bridging Quantization and Memory
// Efficiency in Vision Transformer Attention".
//
// gfx950 mapping.  A workgroup of 4 waves owns 128 query rows of one (batch, kv-head):
// rows are ordered position-major across the G query heads of the group, so the
// waves share every K/V tile and carry the same causal bound.  Each wave owns 32
// rows and computes S^T = K * Q^T with v_mfma_i32_32x32x32_i8: lane l holds query
// l%32 and 32 of the tile's 64 keys, so the row max and row sum are in-lane plus
// one exchange with lane l^32.  The running max is taken on the int32 accumulators
// (exact: the row's dequantization constant is uniform).  p = exp2(fma(c, acc,
// -(m - log2 448))) is converted to e4m3 in registers and fed, without leaving the
// registers, as the B operand of O^T = V^T * P^T on v_mfma_f32_32x32x64_f8f6f4; the V
// operand is pre-arranged by kv_quantize_i8 in exactly the order the lanes hold P.
#include "common.h"

using namespace attnq;

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;
constexpr int KT = ATTN_Q_KEY_TILE;  // 64

// log2(448), log2(127) rounded once to fp32
constexpr float kLog2_448 = 8.807354922057604f;
constexpr float kLog2_127 = 6.988684686772166f;

__global__ void prefill_ws_init(uint32_t *ws) { *ws = 0u; }

// amax over all q' (q scaled per channel by s_K when K is per-channel), for q_gran TENSOR
__global__ void q_amax_kernel(const uint16_t *__restrict__ q, size_t n, int D, int Hq, int Hkv,
                              int L, const float *__restrict__ k_scales, int k_channel,
                              uint32_t *ws) {
  float a = 0.0f;
  const int G = Hq / Hkv;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    float x = __half2float(__ushort_as_half(q[i]));
    if (k_channel) {
      const size_t row = i / D;
      const int c = (int)(i % D);
      const int h = (int)((row / L) % Hq), b = (int)(row / ((size_t)L * Hq));
      x = x * k_scales[((size_t)b * Hkv + h / G) * D + c];
    }
    a = fmaxf(a, fabsf(x));
  }
  for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m));
  if ((threadIdx.x & 63) == 0) atomicMax(ws, __float_as_uint(a));
}

template <int D, int PV, bool CAUSAL, bool DEBUG>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillLaunch a, int nblk, int total) {
  constexpr int NK = D / 32;  // 32-wide d chunks = QK MFMAs per S tile = PV m-tiles
  const int L = xcd_linear(blockIdx.x, gridDim.x);
  if (L >= total) return;
  const int G = a.Hq / a.Hkv;
  int blk = L % nblk;
  const int bg = L / nblk;
  if (CAUSAL) blk = nblk - 1 - blk;  // heaviest (latest) query blocks first
  const int b = bg / a.Hkv, g = bg % a.Hkv;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int wrow0 = blk * kRowsPerWG + wave * kRowsPerWave;
  const int row = wrow0 + n;
  const int i = row / G;
  const int h = g * G + row % G;
  const bool row_valid = i < a.q_len;
  const int iq = row_valid ? i : a.q_len - 1;
  const size_t qrow = ((size_t)b * a.Hq + (row_valid ? h : g * G)) * a.q_len + iq;

  // ---- Q prologue: q' = q * s_K (per-channel K), int8 per row, B operand of S^T
  float qf[NK][16];
  float amax = 0.0f;
  const uint16_t *qp = a.q + qrow * D;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    v4i r0 = *(const v4i *)(qp + kk * 32 + hh * 16);
    v4i r1 = *(const v4i *)(qp + kk * 32 + hh * 16 + 8);
    const uint16_t *h0 = (const uint16_t *)&r0, *h1 = (const uint16_t *)&r1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qf[kk][e] = __half2float(__ushort_as_half(h0[e]));
      qf[kk][e + 8] = __half2float(__ushort_as_half(h1[e]));
    }
    if (a.k_gran == ATTN_Q_GRAN_CHANNEL) {
      const float *ks = a.k_scales + (size_t)bg * D + kk * 32 + hh * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) qf[kk][e] = qf[kk][e] * ks[e];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(qf[kk][e]));
  }
  float sq;
  if (a.q_gran == ATTN_Q_GRAN_TENSOR) {
    sq = __uint_as_float(*(const uint32_t *)a.ws) / 127.0f;
  } else {
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    sq = amax / 127.0f;
  }
  float c = sq * a.kconst;
  if (a.k_gran == ATTN_Q_GRAN_TENSOR) c = c * a.k_scales[0];
  v4i qop[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) word |= (uint32_t)(quant_i8(qf[kk][4 * w + e], sq) & 0xFF) << (8 * e);
      qop[kk][w] = (int)word;
    }
  }

  // ---- key range of this wave
  const int i_lo = min(wrow0 / G, a.q_len - 1);
  const int i_hi = min((wrow0 + kRowsPerWave - 1) / G, a.q_len - 1);
  const int kv_end = CAUSAL ? min(a.kv_len, a.q_offset + i_hi + 1) : a.kv_len;
  const int ntiles = (kv_end + KT - 1) / KT;
  const int vis_last = CAUSAL ? a.q_offset + iq : a.kv_len - 1;  // last visible key of the lane

  const float Lsc = PV == ATTN_Q_PV_FP8 ? kLog2_448 : kLog2_127;
  float m = -INFINITY, l = 0.0f;
  v16f O[NK];
#pragma unroll
  for (int mt = 0; mt < NK; ++mt) O[mt] = v16f{};

  const int8_t *kbase = a.k_codes + (size_t)bg * a.cap * D;
  const uint8_t *vbase = a.v_op + (size_t)bg * (a.cap / KT) * D * KT;

  for (int t = 0; t < ntiles; ++t) {
    const int key0 = t * KT;
    // -- S^T tile = K Q^T, two 32-key halves
    v16i S[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v16i acc = v16i{};
      const int8_t *kp = kbase + (size_t)(key0 + 32 * j + n) * D + hh * 16;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        v4i kv = *(const v4i *)(kp + kk * 32);
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qop[kk], acc, 0, 0, 0);
      }
      S[j] = acc;
    }
    // -- masking (only tiles that reach past a bound)
    const bool need_mask = (key0 + KT > a.kv_len) || (CAUSAL && key0 + KT - 1 > a.q_offset + i_lo);
    if (need_mask) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > vis_last || key >= a.kv_len) S[j][r] = INT_MIN;
        }
    }
    if (DEBUG) {
      int32_t *ds = a.debug_s + (((size_t)b * a.Hq + h) * a.q_len + i) * a.kv_len;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (row_valid && key <= vis_last && key < a.kv_len) ds[key] = S[j][r];
        }
    }
    // -- running max on the int32 accumulators
    int mx = INT_MIN;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = max(mx, S[j][r]);
    mx = max(mx, __shfl_xor(mx, 32));
    const float mt_ = mx == INT_MIN ? -INFINITY : c * (float)mx;
    const float mnew = fmaxf(m, mt_);
    if (__any(mnew != m)) {
      const float alpha = fast_exp2(m - mnew);  // m = -inf on the first tile -> 0
      l *= alpha;
#pragma unroll
      for (int mt = 0; mt < NK; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[mt][r] *= alpha;
      m = mnew;
    }
    const float negmL = -(m - Lsc);
    // -- p = exp2(c*acc - mL), row sum, P to 8 bits in registers
    float p[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = S[j][r] == INT_MIN ? -INFINITY : __builtin_fmaf(c, (float)S[j][r], negmL);
        p[j][r] = fast_exp2(x);
        l += p[j][r];
      }
    if (PV == ATTN_Q_PV_FP8) {
      v8i P8;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int j = w >> 2, r0 = (w & 3) * 4;
        int word = cvt_pk_e4m3<false>(p[j][r0], p[j][r0 + 1], 0);
        word = cvt_pk_e4m3<true>(p[j][r0 + 2], p[j][r0 + 3], word);
        P8[w] = word;
      }
      const uint8_t *vp = vbase + (size_t)t * D * KT + (size_t)n * KT + hh * 32;
#pragma unroll
      for (int mt = 0; mt < NK; ++mt) {
        v8i va = *(const v8i *)(vp + (size_t)mt * 32 * KT);
        O[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, P8, O[mt], 0, 0, 0, 0, 0, 0);
      }
    } else {
      v4i P8[2];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int j = w >> 2, r0 = (w & 3) * 4;
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pc = (int)fminf(__builtin_rintf(p[j][r0 + e]), 127.0f);
          word |= (uint32_t)pc << (8 * e);
        }
        P8[j][w & 3] = (int)word;
      }
      const uint8_t *vp = vbase + (size_t)t * D * KT + (size_t)n * KT + hh * 32;
#pragma unroll
      for (int mt = 0; mt < NK; ++mt) {
        v16i pv = v16i{};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          v4i va = *(const v4i *)(vp + (size_t)mt * 32 * KT + j * 16);
          pv = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, P8[j], pv, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) O[mt][r] += (float)pv[r];
      }
    }
  }

  // ---- epilogue: o = O * s_V / l
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  if (!row_valid) return;
  const size_t orow = (((size_t)b * a.Hq + h) * a.q_len + i) * D;
  const float *vs = a.v_scales + (size_t)bg * D;
#pragma unroll
  for (int mt = 0; mt < NK; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int ch = mt * 32 + 8 * r4 + 4 * hh;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = O[mt][4 * r4 + e] * (vs[ch + e] * inv);
      if (a.out_f32) {
        *(float4 *)((float *)a.out + orow + ch) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        __half2 lo = __floats2half2_rn(o[0], o[1]), hi = __floats2half2_rn(o[2], o[3]);
        uint2 pk = make_uint2(*(uint32_t *)&lo, *(uint32_t *)&hi);
        *(uint2 *)((__half *)a.out + orow + ch) = pk;
      }
    }
}

template <int D, int PV, bool CAUSAL>
hipError_t launch_t(const PrefillLaunch &a, hipStream_t s, dim3 grid, int nblk, int total) {
  if (a.debug_s)
    hipLaunchKernelGGL((prefill_kernel<D, PV, CAUSAL, true>), grid, dim3(kThreads), 0, s, a, nblk, total);
  else
    hipLaunchKernelGGL((prefill_kernel<D, PV, CAUSAL, false>), grid, dim3(kThreads), 0, s, a, nblk, total);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillLaunch &a, hipStream_t s, dim3 grid, int nblk, int total) {
  if (a.pv_mode == ATTN_Q_PV_FP8)
    return a.causal ? launch_t<D, ATTN_Q_PV_FP8, true>(a, s, grid, nblk, total)
                    : launch_t<D, ATTN_Q_PV_FP8, false>(a, s, grid, nblk, total);
  return a.causal ? launch_t<D, ATTN_Q_PV_INT8, true>(a, s, grid, nblk, total)
                  : launch_t<D, ATTN_Q_PV_INT8, false>(a, s, grid, nblk, total);
}

}  // namespace

size_t prefill_workspace_bytes(int q_gran) { return q_gran == ATTN_Q_GRAN_TENSOR ? 256 : 0; }

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t s) {
  if (a.q_len == 0) return hipSuccess;
  if (a.q_gran == ATTN_Q_GRAN_TENSOR) {
    hipLaunchKernelGGL(prefill_ws_init, dim3(1), dim3(1), 0, s, (uint32_t *)a.ws);
    const size_t n = (size_t)a.B * a.Hq * a.q_len * a.D;
    const int blocks = (int)std::min<size_t>((n + 255) / 256, 2048);
    hipLaunchKernelGGL(q_amax_kernel, dim3(blocks), dim3(256), 0, s, a.q, n, a.D, a.Hq, a.Hkv,
                       a.q_len, a.k_scales, (int)(a.k_gran == ATTN_Q_GRAN_CHANNEL), (uint32_t *)a.ws);
  }
  const int G = a.Hq / a.Hkv;
  const int nblk = (G * a.q_len + kRowsPerWG - 1) / kRowsPerWG;
  const int total = a.B * a.Hkv * nblk;
  dim3 grid((total + 7) / 8 * 8);
  return a.D == 128 ? launch_d<128>(a, s, grid, nblk, total) : launch_d<64>(a, s, grid, nblk, total);
}

// attn_q_v_operand: the PV operand of attn_q_prefill from the cache's int8 V codes.
//
// "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8", section "fp8 is not
// faster, it is shaped correctly": P and V enter the PV product as fp8.  The cache keeps V as
// int8 codes with per-channel or per-token scales; the e4m3 operand is derived from them once
// per cache (not per query tile):
//   per-channel V: e4m3(code) (the channel scale is applied after the product), or the code
//                  itself for the int8-PV comparison variant;
//   per-token V:   e4m3(code * f_n), f_n = fp32(s_V[n] * c_V), c_V = fp32(448 / fp32(127 V_max)),
//                  V_max the largest per-token scale of the head (written to the header), so
//                  every operand value stays within 448 and P keeps its static scale.
// The operand is laid out per 64-key tile as [channel][64 keys] in the order one matrix-core
// wave holds a tile of P (byte p <-> key perm(p)), so the prefill's V operand is one 16-byte
// read per lane.
//
// Two launches: the header reduction (per-token V only; one workgroup per (batch, kv-head)
// over its fp16 scales), then one workgroup per 64-key tile, each thread converting 4
// consecutive keys x 8 channels and writing them as one word per channel of the tile in LDS.
#include "common.h"

using namespace attnq;

namespace {

constexpr int kMaxThreads = 256;

__global__ __launch_bounds__(kMaxThreads) void vop_vmax_kernel(const uint16_t *__restrict__ v_scales, int n_keys,
                                                                int cap, float *__restrict__ v_scale_max) {
  const int bg = blockIdx.x, t = threadIdx.x;
  __shared__ float s_red[kMaxThreads / 64];
  float m = 0.0f;
  for (int n = t; n < n_keys; n += kMaxThreads)
    m = fmaxf(m, __half2float(__ushort_as_half(v_scales[(size_t)bg * cap + n])));
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((t & 63) == 0) s_red[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxThreads / 64; ++i) r = fmaxf(r, s_red[i]);
    v_scale_max[bg] = r;
  }
}

// inverse of the operand permutation: key r of a 64-key tile -> byte position
__device__ __forceinline__ int vop_pos(int r) {
  const int j = r >> 5, a = (r >> 3) & 3, h = (r >> 2) & 1, b = r & 3;
  return 32 * h + 16 * j + 4 * a + b;
}

// grid (cap / 64, B * Hkv), 2 * D threads: thread (part, rsub) owns channels 8 part .. +7 of
// keys 4 rsub .. 4 rsub + 3 of the tile
template <int D>
__global__ __launch_bounds__(2 * D) void vop_fill_kernel(const int8_t *__restrict__ v_codes,
                                                         const void *__restrict__ v_scales, int v_gran,
                                                         const float *__restrict__ v_scale_max, int n_keys,
                                                         int cap, int fmt, uint8_t *__restrict__ v_op) {
  constexpr int LPR = D / 8;
  const int bg = blockIdx.y, tile = blockIdx.x, t = threadIdx.x;
  const int part = t % LPR, rsub = t / LPR;
  __shared__ uint8_t s_vop[D * 64];
  const bool vtok = v_gran == ATTN_Q_GRAN_TOKEN;
  const float cv = vtok ? token_v_factor(v_scale_max[bg]) : 1.0f;
  uint32_t word[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = tile * 64 + rsub * 4 + i;
    const bool valid = n < n_keys;
    const int ns = valid ? n : 0;   // (an address inside the cache for the rows past n_keys)
    const uint2 raw = *(const uint2 *)(v_codes + ((size_t)bg * cap + ns) * D + part * 8);
    const float f = vtok ? __half2float(__ushort_as_half(((const uint16_t *)v_scales)[(size_t)bg * cap + ns])) * cv
                         : 1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int code = (int)(int8_t)(((e < 4 ? raw.x : raw.y) >> (8 * (e & 3))) & 0xFFu);
      uint32_t byte;
      if (fmt == ATTN_Q_PV_INT8) {
        byte = (uint32_t)code & 0xFFu;
      } else {
        // fp32(code * f_n), clamped to the e4m3 range (the conversion returns NaN above 448
        // where round-to-nearest with saturation gives 448)
        const float x = __builtin_amdgcn_fmed3f((float)code * f, -448.0f, 448.0f);
        byte = (uint32_t)cvt_pk_e4m3<false>(x, 0.0f, 0) & 0xFFu;
      }
      if (!valid) byte = 0u;
      word[e] |= byte << (8 * i);
    }
  }
  const int pos = vop_pos(rsub * 4);   // 4 consecutive keys -> 4 consecutive bytes
#pragma unroll
  for (int e = 0; e < 8; ++e) *(uint32_t *)&s_vop[(part * 8 + e) * 64 + pos] = word[e];
  __syncthreads();
  uint8_t *dst = v_op + ((size_t)bg * (cap / 64) + tile) * D * 64;
  for (int i = t; i < D * 64 / 16; i += 2 * D) ((v4i *)dst)[i] = ((const v4i *)s_vop)[i];
}

}  // namespace

hipError_t launch_v_operand(const VopLaunch &a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (a.v_gran == ATTN_Q_GRAN_TOKEN)
    hipLaunchKernelGGL(vop_vmax_kernel, dim3(BH), dim3(kMaxThreads), 0, s, (const uint16_t *)a.v_scales,
                       a.n_keys, a.cap, a.v_scale_max);
  const dim3 g(a.cap / 64, BH);
  if (a.D == 128)
    hipLaunchKernelGGL(vop_fill_kernel<128>, g, dim3(256), 0, s, a.v_codes, a.v_scales, a.v_gran, a.v_scale_max,
                       a.n_keys, a.cap, a.fmt, a.v_op);
  else
    hipLaunchKernelGGL(vop_fill_kernel<64>, g, dim3(128), 0, s, a.v_codes, a.v_scales, a.v_gran, a.v_scale_max,
                       a.n_keys, a.cap, a.fmt, a.v_op);
  return hipGetLastError();
}

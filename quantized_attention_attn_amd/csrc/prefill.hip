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
// gfx950 mapping.  A workgroup owns 128 query rows of one (batch, kv-head): rows are
// ordered position-major across the G query heads of the group, so all its waves share
// every K/V tile and nearly the same causal bound.  Key tiles are dealt to two streams
// (even / odd tiles); each stream has 4 waves of 32 rows, so there are 2 waves per SIMD
// to hide each other's latencies.  Each stream stages its tiles in LDS once (16-byte
// coalesced global loads, rows padded so the 16-byte operand reads hit distinct banks),
// double-buffered with one barrier per step.  Each wave computes S^T = K * Q^T with
// v_mfma_i32_32x32x32_i8: lane l holds query
// l%32 and 32 of the tile's 64 keys, so the row max and row sum are in-lane plus
// one exchange with lane l^32.  The running max is taken on the int32 accumulators
// (exact: the row's dequantization constant is uniform).  p = exp2(fma(c, acc,
// -(m - log2 448))) is converted to e4m3 in registers and fed, without leaving the
// registers, as the B operand of O^T = V^T * P^T on v_mfma_f32_32x32x64_f8f6f4; the V
// operand is pre-arranged by kv_quantize_i8 in exactly the order the lanes hold P.
#include "common.h"

using namespace attnq;

namespace {

constexpr int kStreams = ATTN_Q_KEY_STREAMS;      // key streams per row block
constexpr int kRowWaves = 4;                        // waves per stream (32 query rows each)
constexpr int kWaves = kRowWaves * kStreams;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kRowWaves * kRowsPerWave;
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

// Per-lane state of one wave's 32 query rows across key tiles.
template <int D>
struct RowState {
  static constexpr int NK = D / 32;
  v16f O[NK];     // O^T accumulators: lane holds query l%32, 16 channels per m-tile
  float l;        // row sum of the quantized P
  float m;        // running max (log2 units)
};

// LDS staging of one 64-key tile: K rows (D bytes, padded) and the V operand rows
// (64 bytes per channel, padded).  The pads make the 16-byte reads of 16 consecutive
// lanes (16 consecutive rows) fall on distinct banks.
template <int D>
struct Stage {
  static constexpr int KP = D + 16;          // K row pitch
  static constexpr int VP = KT + 16;         // V row pitch
  static constexpr int KBYTES = KT * KP;
  static constexpr int BYTES = KBYTES + D * VP;
  static constexpr int KCH = KT * D / 16;    // 16-byte pieces of a K tile
  static constexpr int VCH = D * KT / 16;    // ... of a V tile
  static constexpr int NCH = (KCH + VCH) / 256;   // pieces per thread of the stream
  static_assert(KCH % 256 == 0 && VCH % 256 == 0, "whole pieces per thread");
};

// global -> registers: the stream's 256 threads fetch K tile tk and V tile tv
template <int D>
__device__ __forceinline__ void stage_fetch(v4i (&r)[Stage<D>::NCH], const int8_t *kbase,
                                            const uint8_t *vbase, int tk, int tv, int tid) {
  constexpr int KU = Stage<D>::KCH / 256;
#pragma unroll
  for (int u = 0; u < Stage<D>::NCH; ++u) {
    if (u < KU) r[u] = *(const v4i *)(kbase + (size_t)tk * KT * D + (size_t)(tid + u * 256) * 16);
    else r[u] = *(const v4i *)(vbase + (size_t)tv * D * KT + (size_t)(tid + (u - KU) * 256) * 16);
  }
}
// registers -> LDS (padded layout): K into kbuf, V into vbuf
template <int D>
__device__ __forceinline__ void stage_store(const v4i (&r)[Stage<D>::NCH], uint8_t *kbuf, uint8_t *vbuf,
                                            int tid) {
  constexpr int KU = Stage<D>::KCH / 256;
#pragma unroll
  for (int u = 0; u < Stage<D>::NCH; ++u) {
    if (u < KU) {
      const int o = (tid + u * 256) * 16;
      *(v4i *)(kbuf + (o / D) * Stage<D>::KP + (o % D)) = r[u];
    } else {
      const int o = (tid + (u - KU) * 256) * 16;
      *(v4i *)(vbuf + (o / KT) * Stage<D>::VP + (o % KT)) = r[u];
    }
  }
}

template <int D>
struct StreamLds {
  uint8_t k[2][Stage<D>::KBYTES];
  uint8_t v[2][D * Stage<D>::VP];
};

// The QK accumulators start from the bit pattern of the fp32 value 1.5 * 2^23, so each
// result, read as fp32, is exactly 1.5 * 2^23 + acc (|acc| <= 127 * 127 * 128 < 2^22 keeps
// the sum inside one binade where the integer add lands in the mantissa): the int32 -> fp32
// conversion of the scores costs nothing.
constexpr int kBiasBits = 0x4B400000;
constexpr float kBias = 12582912.0f;

// S^T = K Q^T for one 64-key tile from LDS (int8, exact int32, biased by kBiasBits).
template <int D>
__device__ __forceinline__ void qk_tile(v16i (&S)[2], const uint8_t *kbuf, const v4i *qop, int n, int hh,
                                        const v16i &bias) {
  constexpr int NK = D / 32;
  const uint8_t *kb = kbuf + n * Stage<D>::KP + hh * 16;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const v4i k0 = *(const v4i *)(kb + kk * 32);
    const v4i k1 = *(const v4i *)(kb + 32 * Stage<D>::KP + kk * 32);
    S[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0, qop[kk], kk == 0 ? bias : S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1, qop[kk], kk == 0 ? bias : S[1], 0, 0, 0);
  }
}

// O^T += V^T P^T for one tile (V operand from LDS) and the row sum of its quantized P (a
// V^T operand of ones: e4m3 0x38, or int8 1 in INT8 mode).  Returns the row sum.
template <int D, int PV>
__device__ __forceinline__ float pv_tile(RowState<D> &st, const v8i &P, const uint8_t *vbuf, int n, int hh,
                                         const v8i &ones) {
  constexpr int NK = D / 32;
  const uint8_t *vb = vbuf + n * Stage<D>::VP + hh * 32;
  v8i vop[NK];
#pragma unroll
  for (int mt = 0; mt < NK; ++mt) vop[mt] = *(const v8i *)(vb + mt * 32 * Stage<D>::VP);
  if (PV == ATTN_Q_PV_FP8) {
#pragma unroll
    for (int mt = 0; mt < NK; ++mt)
      st.O[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mt], P, st.O[mt], 0, 0, 0, 0, 0, 0);
    const v16f lt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, P, v16f{}, 0, 0, 0, 0, 0, 0);
    return lt[0];   // every element of a lane holds its row's sum
  } else {
    const v4i P0 = v4i{P[0], P[1], P[2], P[3]}, P1 = v4i{P[4], P[5], P[6], P[7]};
#pragma unroll
    for (int mt = 0; mt < NK; ++mt) {
      v16i pv = v16i{};
      pv = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{vop[mt][0], vop[mt][1], vop[mt][2], vop[mt][3]}, P0, pv,
                                                 0, 0, 0);
      pv = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{vop[mt][4], vop[mt][5], vop[mt][6], vop[mt][7]}, P1, pv,
                                                 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) st.O[mt][q] += (float)pv[q];
    }
    v16i ls = v16i{};
    ls = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{ones[0], ones[1], ones[2], ones[3]}, P0, ls, 0, 0, 0);
    ls = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{ones[0], ones[1], ones[2], ones[3]}, P1, ls, 0, 0, 0);
    return (float)ls[0];
  }
}

// Online-softmax step of one tile: l += ladd, mask, int32 running max, the rescale of
// (O, l) when the max moves, p = exp2(c*acc - (m - log2 448)) and P to e4m3 (or int8) in
// registers.  P words: FP8 -- the B operand of the 32x32x64 fp8 MFMA; INT8 -- two 32x32x32
// B operands.  MASK: key key0 + 4*hh + off of the tile is visible iff off <= lim (off is a
// compile-time constant); lim < 0 masks the whole tile, which then leaves (m, l, O)
// unchanged.
template <int D, int PV, bool MASK, bool DEBUG>
__device__ __forceinline__ void softmax_tile(RowState<D> &st, v16i (&S)[2], v8i &P, float c, float Lsc, int key0,
                                             int hh, int lim, int32_t *ds, float ladd) {
  constexpr int NK = D / 32;
  st.l += ladd;   // row sum of the previous tile's P, which O already holds
  if (MASK) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int off = 32 * j + 8 * (q >> 2) + (q & 3);
        if (DEBUG && ds && off <= lim) ds[key0 + 4 * hh + off] = S[j][q] - kBiasBits;
        if (off > lim) S[j][q] = INT_MIN;
      }
  } else if (DEBUG && ds) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) ds[key0 + 32 * j + 8 * (q >> 2) + 4 * hh + (q & 3)] = S[j][q] - kBiasBits;
  }
  int mx = INT_MIN;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = max(mx, S[j][q]);
  mx = max_xor32(mx);
  // (the biased scores order like the scores; the max is exact as an fp32 difference)
  const float mt_ = (MASK && mx == INT_MIN) ? -INFINITY : c * (__int_as_float(mx) - kBias);
  const float mnew = fmaxf(st.m, mt_);
  if (__any(mnew != st.m)) {
    // 1 where the max did not move (also a row that has seen no key yet: -inf to -inf),
    // 0 on a row's first visible tile
    const float alpha = mnew == st.m ? 1.0f : fast_exp2(st.m - mnew);
    st.l *= alpha;
#pragma unroll
    for (int mt = 0; mt < NK; ++mt)
#pragma unroll
      for (int q = 0; q < 16; ++q) st.O[mt][q] *= alpha;
    st.m = mnew;
  }
  // exponent c*acc - (m - log2 448) evaluated as c*(bias + acc) + fp32(-(c*bias) - (m - log2 448))
  const float negK = __builtin_fmaf(-c, kBias, Lsc - st.m);
  float p[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float x = __builtin_fmaf(c, __int_as_float(S[j][q]), negK);
      if (MASK) x = S[j][q] == INT_MIN ? -INFINITY : x;
      p[j][q] = fast_exp2(x);
    }
  if (PV == ATTN_Q_PV_FP8) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int j = w >> 2, r0 = (w & 3) * 4;
      // the low half is written over whatever the word held; the high half follows
      const int word = cvt_pk_e4m3<false>(p[j][r0], p[j][r0 + 1], P[w]);
      P[w] = cvt_pk_e4m3<true>(p[j][r0 + 2], p[j][r0 + 3], word);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int j = w >> 2, r0 = (w & 3) * 4;
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pc = (int)fminf(__builtin_rintf(p[j][r0 + e]), 127.0f);
        word |= (uint32_t)pc << (8 * e);
      }
      P[w] = (int)word;
    }
  }
}

// Per-wave constants of the tile loop.
struct LoopArgs {
  const int8_t *kbase;
  const uint8_t *vbase;
  const v4i *qop;
  float c, Lsc;
  int n, hh, stid, stream;
  int nsteps, ntiles_wg, t_mask;
  int lim0;   // last key visible to the lane, minus 4*hh
  int32_t *ds;
};

// The tile loop of one key stream (tiles t_k = 2k + stream, ascending).  Step k is a
// matrix-core phase -- PV of tile t_{k-1} (V from LDS buffer (k+1)%2, P from registers)
// and QK of t_k (K from buffer k%2) -- followed by the vector phase, the softmax of t_k.
// Both streams run in step, so each SIMD interleaves its two waves' matrix-core work and
// then their vector work (the matrix cores and the vector unit of a SIMD barely overlap
// across waves, while two waves issuing vector work together double its rate).  The
// stream's threads fetch K tile t_{k+1} and V tile t_k into registers at the start of the
// step and store them to the other buffers at its end.  Steps run unconditionally: a tile
// beyond the wave's last visible key (and the empty "previous tile" of the first step) is
// computed fully masked, which leaves (m, l, O) unchanged; loads are clamped to the
// workgroup's last tile, whose data is valid, so such steps read only finite values.
template <int D, int PV, bool DEBUG>
__device__ __forceinline__ void stream_loop(RowState<D> &st, StreamLds<D> &lds, const LoopArgs &a,
                                            v4i (&pre)[Stage<D>::NCH]) {
  v16i S[2] = {v16i{}, v16i{}};
  v8i P = v8i{};
  const int one = PV == ATTN_Q_PV_FP8 ? 0x38383838 : 0x01010101;
  v8i ones = v8i{one, one, one, one, one, one, one, one};
  asm volatile("" : "+v"(ones));   // keep the constant operands resident in registers
  v16i bias;
#pragma unroll
  for (int e = 0; e < 16; ++e) bias[e] = kBiasBits;
  asm volatile("" : "+v"(bias));
  const int last = a.ntiles_wg - 1;
  for (int k = 0; k <= a.nsteps; ++k) {
    const int t = kStreams * k + a.stream;
    stage_fetch<D>(pre, a.kbase, a.vbase, min(t + kStreams, last), min(t, last), a.stid);
    const uint8_t *kbuf = lds.k[k & 1];
    const uint8_t *vprev = lds.v[(k + 1) & 1];
    const int key0 = t * KT;
    const int lim = a.lim0 - key0;
    const float lsum = pv_tile<D, PV>(st, P, vprev, a.n, a.hh, ones);
    qk_tile<D>(S, kbuf, a.qop, a.n, a.hh, bias);
    __builtin_amdgcn_sched_barrier(0);
    if (t < a.t_mask) softmax_tile<D, PV, false, DEBUG>(st, S, P, a.c, a.Lsc, key0, a.hh, lim, a.ds, lsum);
    else softmax_tile<D, PV, true, DEBUG>(st, S, P, a.c, a.Lsc, key0, a.hh, lim, a.ds, lsum);
    stage_store<D>(pre, lds.k[(k + 1) & 1], lds.v[k & 1], a.stid);
    __syncthreads();
  }
  // (the row sum of the last tile was added by the fully masked softmax of step nsteps)
}

template <int D, int PV, bool DEBUG>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillLaunch a, int nblk, int total) {
  constexpr int NK = D / 32;  // 32-wide d chunks = QK MFMAs per S tile = PV m-tiles
  __shared__ __attribute__((aligned(16))) StreamLds<D> s_stage[kStreams];
  const int L = xcd_linear(blockIdx.x, gridDim.x);
  if (L >= total) return;
  const int G = a.Hq / a.Hkv;
  int blk = L % nblk;
  const int bg = L / nblk;
  // (causal masking is a runtime flag: both cases share one code path and register budget)
  const bool causal = a.causal != 0;
  if (causal) blk = nblk - 1 - blk;  // heaviest (latest) query blocks first
  const int b = bg / a.Hkv, g = bg % a.Hkv;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rw = wave % kRowWaves, stream = wave / kRowWaves;
  const int stid = threadIdx.x % (kRowWaves * 64);   // thread index within the stream
  const int n = lane & 31, hh = lane >> 5;
  const int wrow0 = blk * kRowsPerWG + rw * kRowsPerWave;
  const int row = wrow0 + n;
  const int i = row / G;
  const int h = g * G + row % G;
  const bool row_valid = i < a.q_len;
  const int iq = row_valid ? i : a.q_len - 1;
  const size_t qrow = ((size_t)b * a.Hq + (row_valid ? h : g * G)) * a.q_len + iq;

  const int8_t *kbase = a.k_codes + (size_t)bg * a.cap * D;
  const uint8_t *vbase = a.v_op + (size_t)bg * (a.cap / KT) * D * KT;

  // ---- tiles of this workgroup (the bound of its last row) and of this wave
  const int i_wg_hi = min((blk * kRowsPerWG + kRowsPerWG - 1) / G, a.q_len - 1);
  const int ntiles_wg = ((causal ? min(a.kv_len, a.q_offset + i_wg_hi + 1) : a.kv_len) + KT - 1) / KT;
  const int nsteps = (ntiles_wg + kStreams - 1) / kStreams;
  // the first K tile goes out before the Q prologue so its latency is covered (its V part,
  // tile 0, only feeds the empty first step)
  v4i pre[Stage<D>::NCH];
  stage_fetch<D>(pre, kbase, vbase, min(stream, ntiles_wg - 1), 0, stid);

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
    amax = max_xor32(amax);
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

  // ---- this wave's tiles: [0, t_mask) need no mask, [t_mask, ntiles) do
  const int i_lo = min(wrow0 / G, a.q_len - 1);
  const int i_hi = min((wrow0 + kRowsPerWave - 1) / G, a.q_len - 1);
  const int kv_end = causal ? min(a.kv_len, a.q_offset + i_hi + 1) : a.kv_len;
  const int ntiles = (kv_end + KT - 1) / KT;
  int t_mask = min(ntiles, a.kv_len / KT);
  if (causal) t_mask = min(t_mask, (a.q_offset + i_lo + 1) / KT);
  const int vis_last = causal ? a.q_offset + iq : a.kv_len - 1;  // last visible key of the lane

  const float Lsc = PV == ATTN_Q_PV_FP8 ? kLog2_448 : kLog2_127;
  RowState<D> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int mt = 0; mt < NK; ++mt) st.O[mt] = v16f{};
  int32_t *ds = nullptr;
  if (DEBUG && row_valid) ds = a.debug_s + (((size_t)b * a.Hq + h) * a.q_len + i) * a.kv_len;

  // ---- the tile loop (K tile t_0 staged first; V tiles arrive one step after their K)
  stage_store<D>(pre, s_stage[stream].k[0], s_stage[stream].v[1], stid);
  __syncthreads();
  const LoopArgs la{kbase, vbase, qop, c, Lsc, n, hh, stid, stream, nsteps, ntiles_wg, t_mask,
                    min(vis_last, a.kv_len - 1) - 4 * hh, ds};
  stream_loop<D, PV, DEBUG>(st, s_stage[stream], la, pre);

  // ---- merge the key streams through LDS (reusing the staging buffers), one m-tile
  //      at a time: stream s > 0 hands (m, l, O) to stream 0
  float *xch = (float *)&s_stage[0];   // [kStreams-1][kRowWaves][18][64] floats
  static_assert((kStreams - 1) * kRowWaves * 18 * 64 * 4 <= sizeof(s_stage), "merge buffer");
  float f1 = 1.0f, f2[kStreams - 1];
#pragma unroll
  for (int mt = 0; mt < NK; ++mt) {
    if (stream > 0) {
      float *p = xch + (((stream - 1) * kRowWaves + rw) * 18) * 64 + lane;
      if (mt == 0) { p[0] = st.m; p[64] = st.l; }
#pragma unroll
      for (int q = 0; q < 16; ++q) p[(2 + q) * 64] = st.O[mt][q];
    }
    __syncthreads();
    if (stream == 0) {
#pragma unroll
      for (int sp = 0; sp < kStreams - 1; ++sp) {
        const float *p = xch + ((sp * kRowWaves + rw) * 18) * 64 + lane;
        if (mt == 0) {
          const float m2 = p[0], l2 = p[64];
          const float M = fmaxf(st.m, m2);
          f1 = st.m == -INFINITY ? 0.0f : fast_exp2(st.m - M);
          f2[sp] = m2 == -INFINITY ? 0.0f : fast_exp2(m2 - M);
          st.l = st.l * f1 + l2 * f2[sp];
          st.m = M;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) st.O[mt][q] = st.O[mt][q] * f1 + p[(2 + q) * 64] * f2[sp];
      }
    }
    __syncthreads();
  }
  if (stream > 0) return;

  // ---- epilogue: o = O * s_V / l
  const float inv = 1.0f / st.l;   // the MFMA row sum is complete in both lane halves
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
      for (int e = 0; e < 4; ++e) o[e] = st.O[mt][4 * r4 + e] * (vs[ch + e] * inv);
      if (a.out_f32) {
        *(float4 *)((float *)a.out + orow + ch) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        __half2 lo = __floats2half2_rn(o[0], o[1]), hi = __floats2half2_rn(o[2], o[3]);
        uint2 pk = make_uint2(*(uint32_t *)&lo, *(uint32_t *)&hi);
        *(uint2 *)((__half *)a.out + orow + ch) = pk;
      }
    }
}

template <int D, int PV>
hipError_t launch_t(const PrefillLaunch &a, hipStream_t s, dim3 grid, int nblk, int total) {
  if (a.debug_s)
    hipLaunchKernelGGL((prefill_kernel<D, PV, true>), grid, dim3(kThreads), 0, s, a, nblk, total);
  else
    hipLaunchKernelGGL((prefill_kernel<D, PV, false>), grid, dim3(kThreads), 0, s, a, nblk, total);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillLaunch &a, hipStream_t s, dim3 grid, int nblk, int total) {
  return a.pv_mode == ATTN_Q_PV_FP8 ? launch_t<D, ATTN_Q_PV_FP8>(a, s, grid, nblk, total)
                                    : launch_t<D, ATTN_Q_PV_INT8>(a, s, grid, nblk, total);
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

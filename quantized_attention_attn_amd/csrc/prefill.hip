// attn_q_prefill: fused int8-QK^T / fp32 online softmax / e4m3-P fp8-PV flash attention.
//
// Method: "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8" -- QK^T on
// int8 with int32 accumulation after K-mean subtraction; running row max m and
// exp(s - m) in fp32 so P <= 1 and its scale is a constant (section "The scale P
// needs is already sitting in a register"); P as e4m3 with static scale 448 and PV
// on fp8 (section "fp8 is not faster, it is shaped correctly").  The tiled loop over
// key blocks in ascending order with a running max (here one per row and key stream), the
// int32 row max and the exp2 with s_Q*s_K*d^-1/2*log2(e) folded in follow Algorithm 1 and
// eq. (3)-(4) of "QFlash: Bridging Quantization and Memory Efficiency in Vision
// Transformer Attention".
//
// gfx950 mapping.  A workgroup of 8 waves (two per SIMD) owns 128 query rows of one
// (batch, kv-head): rows are ordered position-major across the G query heads of the
// group, so all its waves share every K/V tile and nearly the same causal bound.  Key
// tiles are dealt to two streams (even / odd tiles, merged at the end); each stream has 4
// waves of 32 rows, one per SIMD.  Each stream's K and V tiles reach LDS by direct
// global->LDS loads, three steps ahead, in a ring of four slots per operand (swizzled so
// the operand reads are free of bank conflicts), with one barrier per step.  Each wave
// computes S^T = K * Q^T with v_mfma_i32_32x32x32_i8: lane l holds query l%32 and 32 of the tile's 64 keys, so the
// row max and row sum are in-lane plus one exchange with lane l^32.  The running max is
// taken on the int32 accumulators (exact: the row's dequantization constant is uniform);
// with one K scale per key (the fp16 scales reach LDS beside each K tile) the max is taken on
// the dequantized scores fp32(c_j * acc) and each exponent is fma(c_j, acc, -mL).
// p = exp2(c*acc - (m - log2 448)) is converted to e4m3 in registers and fed, without
// leaving the registers, as the B operand of O^T = V^T * P^T on
// v_mfma_f32_32x32x64_f8f6f4; the V operand is pre-arranged by kv_quantize_i8 in exactly
// the order the lanes hold P.  The tile loop is software-pipelined inside each wave: step
// k issues PV of the stream's tile k-1 and QK of its tile k+1 to the matrix core and
// meanwhile runs the softmax of tile k on the vector unit, which depends on neither; the
// two waves of a SIMD (one per stream) share the matrix core and together keep the vector
// unit busy.
#include "common.h"

using namespace attnq;

namespace {

constexpr int kStreams = ATTN_Q_KEY_STREAMS;        // key streams per row block
constexpr int kRowWaves = 4;                        // waves per stream (32 query rows each)
constexpr int kWaves = kRowWaves * kStreams;
constexpr int kThreads = kWaves * 64;
constexpr int kStreamThreads = kRowWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kRowWaves * kRowsPerWave;
constexpr int KT = ATTN_Q_KEY_TILE;  // 64
static_assert(kStreams == 2, "the two waves of a SIMD run the two key streams");

// How the key side of the dequantization constant is applied: folded into Q or the row constant
// (CHANNEL, TENSOR), one fp16 scale per key (TOKEN), or one fp32 scale per 64-key block, which
// is the key tile (BLOCK: a constant per tile).
constexpr int kKmRow = 0, kKmTok = 1, kKmBlk = 2;

// log2(448), log2(127) rounded once to fp32
constexpr float kLog2_448 = 8.807354922057604f;
constexpr float kLog2_127 = 6.988684686772166f;

__global__ void prefill_ws_init(uint32_t *ws) { *ws = 0u; }

// amax over all q' (q scaled per channel by s_K when K is per-channel), for q_gran TENSOR: a
// grid-stride loop over 16-byte loads (8 channels of one row; d is a multiple of 8), the
// workgroup's maximum through LDS and one atomic per workgroup (the fp32 bits of values >= 0
// order like the values).
constexpr int kAmaxThreads = 256;
constexpr int kAmaxBlocks = 512;
__global__ __launch_bounds__(kAmaxThreads) void q_amax_kernel(const uint16_t *__restrict__ q, size_t n, int D, int Hq,
                                                              int Hkv, int L, const float *__restrict__ k_scales,
                                                              int k_channel, uint32_t *ws) {
  float a = 0.0f;
  const int G = Hq / Hkv;
  const size_t n8 = n / 8;
  for (size_t i = (size_t)blockIdx.x * kAmaxThreads + threadIdx.x; i < n8; i += (size_t)gridDim.x * kAmaxThreads) {
    const v4i raw = ((const v4i *)q)[i];
    const uint16_t *h = (const uint16_t *)&raw;
    const float *ks = k_scales;
    if (k_channel) {
      const size_t e0 = i * 8, row = e0 / D;
      const int c0 = (int)(e0 - row * D);
      const int hq = (int)((row / L) % Hq), b = (int)(row / ((size_t)L * Hq));
      ks = k_scales + ((size_t)b * Hkv + hq / G) * D + c0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = __half2float(__ushort_as_half(h[e]));
      if (k_channel) x = x * ks[e];
      a = fmaxf(a, fabsf(x));
    }
  }
  for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m));
  __shared__ float s_w[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = s_w[0];
#pragma unroll
    for (int w = 1; w < kAmaxThreads / 64; ++w) m = fmaxf(m, s_w[w]);
    atomicMax(ws, __float_as_uint(m));
  }
}

// s_Q per block of 64 query positions of a (batch, head), for q_gran BLOCK: amax over the
// block's rows of q' (q scaled per channel by s_K when K is per-channel), fp32(amax / 127).
// grid (ceil(L / 64), B * Hq), 256 threads; ws fp32 [B][Hq][ceil(L / 64)].
__global__ __launch_bounds__(256) void q_block_scale_kernel(const uint16_t *__restrict__ q, int D, int Hq, int Hkv,
                                                            int L, const float *__restrict__ k_scales, int k_channel,
                                                            float *ws) {
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq, G = Hq / Hkv;
  const int i0 = blk * 64, i1 = min(L, i0 + 64);
  const uint16_t *qb = q + (size_t)bh * L * D;
  float a = 0.0f;
  for (int e = i0 * D + threadIdx.x; e < i1 * D; e += 256) {
    float x = __half2float(__ushort_as_half(qb[e]));
    if (k_channel) x = x * k_scales[((size_t)b * Hkv + h / G) * D + e % D];
    a = fmaxf(a, fabsf(x));
  }
  for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m));
  __shared__ float s_a[4];
  if ((threadIdx.x & 63) == 0) s_a[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) ws[(size_t)bh * gridDim.x + blk] = fmaxf(fmaxf(s_a[0], s_a[1]), fmaxf(s_a[2], s_a[3])) / 127.0f;
}

// Per-lane state of one wave's 32 query rows across key tiles.
template <int D>
struct RowState {
  static constexpr int NK = D / 32;
  v16f O[NK];     // O^T accumulators: lane holds query l%32, 16 channels per m-tile
  float l;        // row sum of the quantized P
  float m;        // running max (log2 units)
};

// LDS staging: K tiles (64 rows of D bytes) and V operand tiles (D rows of 64 bytes),
// unpadded.  The 16-byte chunk c of row r is stored in chunk slot c ^ f(r), which puts the
// 16-byte reads of 16 consecutive lanes (16 consecutive rows, one logical chunk) on
// distinct banks of the 64-bank LDS.  Tiles arrive by direct global->LDS loads
// (buffer_load_dwordx4 ... lds): one wave instruction fills 64 consecutive slots (1 KB),
// each lane fetching the global chunk that belongs in its slot, so no registers hold the
// tile.
template <int D>
struct Stage {
  static constexpr int KCPR = D / 16;        // 16-byte chunks per K row (8 or 4)
  static constexpr int VCPR = KT / 16;       // ... per V row (4)
  static constexpr int KBYTES = KT * D;
  static constexpr int VBYTES = D * KT;
  static constexpr int KU = KT * D / 16 / kStreamThreads;   // loads per thread of the stream, K tile
  static constexpr int VU = D * KT / 16 / kStreamThreads;   // ... V tile
  static_assert(KT * D / 16 % kStreamThreads == 0, "whole load instructions per thread");
};
// bytes between a lane's successive chunks of one tile load (kStreamThreads chunks)
constexpr uint32_t kChunkStride = kStreamThreads * 16;
static_assert(kChunkStride == 4096, "u-th chunk offset: rows of the same swizzle phase");

// Chunk slot of logical chunk c in row r for rows of cpr chunks.  16 consecutive rows span
// 2 (128-byte rows) or 4 (64-byte rows) bank phases; the rows sharing a phase get distinct
// slots.  The map is an involution, so it also gives the logical chunk of a slot.
__device__ __forceinline__ int swz_slot(int c, int r, int cpr) {
  return c ^ (cpr == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3));
}

// Slots per operand and stream.  The stream's j-th K tile and j-th V tile live in slot
// j % kRing; at step k its waves read its K tile k+1 and V tile k-1 (the hot step also the
// first operands of K tile k+2, at its end) and load its K tile k+kRing and V tile
// k+kRing-2, so each tile is requested at least two steps before it is read and a slot is
// refilled only after the barrier that follows its last read.
constexpr int kRing = 4;

template <int D>
struct Ring {
  uint8_t k[kRing][Stage<D>::KBYTES];
  uint8_t v[kRing][Stage<D>::VBYTES];
  uint8_t ks[kRing][256];   // per-token K: the fp16 scales of a K tile, in the order the lanes read them
};

// Per-lane byte offsets of the staging loads (source offset within a tile) and of the
// operand reads (LDS offset within a slot); loop invariant.
template <int D>
struct Offsets {
  // source offset of the lane's first chunk; its u-th load is kStreamThreads chunks later,
  // which is 4096 bytes further in both tiles (whole rows, and the row swizzle repeats)
  uint32_t ksrc, vsrc;
  int kop[D / 32];     // K operand of QK chunk kk (row n of the tile)
  int vop0, vop1;      // the two 16-byte halves of the V operand (row n)
};

template <int D>
__device__ __forceinline__ Offsets<D> make_offsets(int tid, int n, int hh) {
  Offsets<D> o;
  {
    const int r = tid / Stage<D>::KCPR, sl = tid % Stage<D>::KCPR;   // LDS chunk slot tid
    o.ksrc = (uint32_t)(r * D + swz_slot(sl, r, Stage<D>::KCPR) * 16);
  }
  {
    const int r = tid / Stage<D>::VCPR, sl = tid % Stage<D>::VCPR;
    o.vsrc = (uint32_t)(r * KT + swz_slot(sl, r, Stage<D>::VCPR) * 16);
  }
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) o.kop[kk] = n * D + swz_slot(2 * kk + hh, n, Stage<D>::KCPR) * 16;
  o.vop0 = n * KT + swz_slot(2 * hh, n, Stage<D>::VCPR) * 16;
  o.vop1 = n * KT + swz_slot(2 * hh + 1, n, Stage<D>::VCPR) * 16;
  return o;
}

#if defined(__HIP_DEVICE_COMPILE__)   // (the buffer builtins exist only in the device pass)
// Buffer resource of one tile (wave-uniform base, raw addressing, the tile's bytes as the
// range).  The loads below address a tile by the lane's 32-bit chunk offset plus a scalar
// offset, so no 64-bit per-lane address is formed or kept in registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *tile, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(tile), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(uint8_t *p) {
  return (__attribute__((address_space(3))) void *)p;
}
#endif

// The stream's waves load K tile t into a slot (global -> LDS) ...
template <int D>
__device__ __forceinline__ void stage_k(uint8_t *kbuf, const int8_t *kbase, int t, int wv, const Offsets<D> &o) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(kbase + (size_t)t * KT * D, KT * D);
#pragma unroll
  for (int u = 0; u < Stage<D>::KU; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(kbuf + (u * kStreamThreads + wv * 64) * 16), 16, o.ksrc,
                                             u * kChunkStride, 0, 0);
#endif
}
// ... and V operand tile t.
template <int D>
__device__ __forceinline__ void stage_v(uint8_t *vbuf, const uint8_t *vbase, int t, int wv, const Offsets<D> &o) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(vbase + (size_t)t * D * KT, D * KT);
#pragma unroll
  for (int u = 0; u < Stage<D>::VU; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(vbuf + (u * kStreamThreads + wv * 64) * 16), 16, o.vsrc,
                                             u * kChunkStride, 0, 0);
#endif
}

// ... and (per-token K) the 64 fp16 scales of K tile t, permuted so that lane half hh finds the
// 32 scales of its keys in 16 consecutive dwords: LDS dword 16hh + 8j + 2r + p holds the scales
// of keys 32j + 8r + 4hh + 2p and + 1, the keys of S elements [j][4r + 2p] and [j][4r + 2p + 1]
// of a lane of half hh.  One dword per lane (a lane's LDS dword is its lane index; lanes 32-63
// repeat lanes 0-31 into the unused upper half); every wave of the stream loads the same slot.
__device__ __forceinline__ void stage_ks(uint8_t *dst, const uint16_t *kscl, int t) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(kscl + (size_t)t * KT, KT * 2);
  const int ln = threadIdx.x & 31, hh = ln >> 4, idx = ln & 15;
  const int src = 16 * (idx >> 3) + 4 * ((idx >> 1) & 3) + 2 * hh + (idx & 1);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst), 4, src * 4, 0, 0, 0);
#endif
}

// The barrier between steps: the wave's LDS reads are complete (so other waves may refill
// their slots) and every wave has arrived.  Not __syncthreads: its workgroup fence would
// also wait for every outstanding tile load (they write LDS), draining the load pipeline
// that wait_tiles keeps two steps deep.
__device__ __forceinline__ void step_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until only the previous step's tile loads are in flight: the loads of step k-2 have
// landed, which covers the tiles step k reads (loaded at step k-3) and the K tile k+2 whose
// first operands the hot step reads at its end.  Debug builds also have global stores in
// flight, so they drain everything.
template <int D, bool DEBUG, bool KTOK>
__device__ __forceinline__ void wait_tiles() {
  constexpr int per_step = Stage<D>::KU + Stage<D>::VU + (KTOK ? 1 : 0);
  static_assert(per_step >= 2 && per_step <= 5, "vmcnt immediates below");
  if (DEBUG) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (per_step == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else if (per_step == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (per_step == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
}

// The QK accumulators start from zero (an inline constant of the MFMA, no registers):
// the int32 scores order like the scores they dequantize to (the row max is taken on them),
// and v_cvt_f32_i32 gives fp32(acc) exactly (|acc| <= 127 * 127 * 128 < 2^24).

// S^T = K Q^T for one 64-key tile from its LDS slot (int8, exact int32).
template <int D>
__device__ __forceinline__ void qk_tile(v16i (&S)[2], const uint8_t *kbuf, const Offsets<D> &o, const v4i *qop,
                                        const v16i &zero) {
  constexpr int NK = D / 32;
  v4i k0[NK], k1[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    k0[kk] = *(const v4i *)(kbuf + o.kop[kk]);
    k1[kk] = *(const v4i *)(kbuf + o.kop[kk] + 32 * D);
  }
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    S[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0[kk], qop[kk], kk == 0 ? zero : S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1[kk], qop[kk], kk == 0 ? zero : S[1], 0, 0, 0);
  }
}

// O^T += V^T P^T for one tile (V operand from its LDS slot) and the row sum of its
// quantized P.  FP8: one 16x16x128 MFMA reads the P registers as its B operand, whose
// lane l then holds keys 32*(l/16) .. +31 of column l%16; those are the keys of query l%32
// (the 32x32x64 layout), so column n mixes queries n and n+16, block by block.  The A
// operand (ones16) selects, for output rows 4g..4g+3, the blocks of parity g%2: lane l's
// result rows are then exactly the sum of query l%32.  INT8: two 32x32x32 MFMAs with an
// operand of ones.  Returns the row sum (held by every element of the lane's result).
template <int D, int PV>
__device__ __forceinline__ float pv_tile(RowState<D> &st, const v8i &P, const uint8_t *vbuf, const Offsets<D> &o,
                                         const v8i &ones) {
  constexpr int NK = D / 32;
  v8i vop[NK];
#pragma unroll
  for (int mt = 0; mt < NK; ++mt) {
    const v4i lo = *(const v4i *)(vbuf + o.vop0 + mt * 32 * KT);
    const v4i hi = *(const v4i *)(vbuf + o.vop1 + mt * 32 * KT);
    vop[mt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  if (PV == ATTN_Q_PV_FP8) {
#pragma unroll
    for (int mt = 0; mt < NK; ++mt)
      st.O[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mt], P, st.O[mt], 0, 0, 0, 0, 0, 0);
    const v4f lt = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P, v4f{}, 0, 0, 0, 0, 0, 0);
    return lt[0];
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

// Online-softmax step of one tile, without touching O or l (so it can run while the matrix
// core still accumulates the previous tile): mask, int32 running max, the new max m and
// the factor alpha = exp2(m_old - m) (1 where the max did not move), p = exp2(c*acc -
// (m - log2 448)) and P to e4m3 (or int8) in registers.  P words: FP8 -- the B operand of
// the 32x32x64 fp8 MFMA; INT8 -- two 32x32x32 B operands.  MASK: key key0 + 4*hh + off of
// the tile is visible iff off <= lim (off is a compile-time constant); lim < 0 masks the
// whole tile, which then leaves (m, l, O) unchanged.  Returns whether any row of the wave
// moved its max.
// fp32(c * s) for the fp16 scale in half `hi` of dword w (one rounding: the fp16 value is exact
// in fp32).  Written as fma(c, s, +0), which equals the product for the non-negative c and s
// here and which the compiler selects as one v_fma_mix_f32 reading the fp16 half in place.
__device__ __forceinline__ float c_times_half(float c, int w, int hi) {
  const uint16_t h = (uint16_t)(hi ? ((uint32_t)w >> 16) : ((uint32_t)w & 0xFFFFu));
  return __builtin_fmaf(c, __half2float(__ushort_as_half(h)), 0.0f);
}

template <int D, int PV, bool MASK, bool DEBUG, bool KTOK>
__device__ __forceinline__ bool softmax_tile(RowState<D> &st, v16i (&S)[2], v8i &P, float &alpha, float c,
                                             float Lsc, int key0, int hh, int lim, int32_t *ds, uint8_t *dp,
                                             const uint8_t *kss) {
  if (DEBUG && ds) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int off = 32 * j + 8 * (q >> 2) + (q & 3);
        if (!MASK || off <= lim) ds[key0 + 4 * hh + off] = S[j][q];
      }
  }
  // the scores to fp32 in place (exact: |acc| < 2^24); masked keys become -inf.  From here on
  // only the fp32 copy is live.
  float sf[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float f = (float)S[j][q];
      sf[j][q] = (MASK && 32 * j + 8 * (q >> 2) + (q & 3) > lim) ? -INFINITY : f;
    }
  // per-token K: each key has its own constant c_j = fp32(c * s_K[j]), and the row max is taken
  // over the dequantized scores fp32(c_j * acc_j) themselves (masked keys -inf).  The scales
  // come from the tile's scale slot (kss: the lane half's 16 dwords): the scale of S element
  // [j][q] is half q%2 of dword 8j + 2(q/4) + (q/2)%2.
  auto cjof = [&](int j, int q) -> float {
    const int dw = 8 * j + 2 * (q >> 2) + ((q >> 1) & 1);
    return c_times_half(c, *(const int *)(kss + 4 * dw), q & 1);
  };
  auto mxin = [&](int j, int q) -> float {
    if (!KTOK) return sf[j][q];
    return sf[j][q] == -INFINITY ? -INFINITY : cjof(j, q) * sf[j][q];
  };
  // (a tree of maxima: four independent chains, then their combination; the maximum of the
  // converted scores is the converted integer maximum)
  float mq[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) mq[r] = fmaxf(mxin(r >> 1, (r & 1) * 8), mxin(r >> 1, (r & 1) * 8 + 1));
#pragma unroll
  for (int e = 2; e < 8; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) mq[r] = fmaxf(mq[r], mxin(r >> 1, (r & 1) * 8 + e));
  float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
  mx = max_xor32(mx);
  const float mt_ = (MASK && mx == -INFINITY) ? -INFINITY : (KTOK ? mx : c * mx);
  const float mnew = fmaxf(st.m, mt_);
  const bool moved = mnew != st.m;
  // 1 where the max did not move (also a row that has seen no key yet: -inf to -inf),
  // 0 on a row's first visible tile
  alpha = fast_exp2(moved ? st.m - mnew : 0.0f);
  st.m = mnew;
  // exponent fp32(c*acc - mL) with one rounding, mL = fp32(m - log2 448); -mL = fp32(log2 448
  // - m) exactly (negation commutes with rounding to nearest); per-token K with c_j
  const float negmL = Lsc - st.m;
  float p[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float x = __builtin_fmaf(KTOK ? cjof(j, q) : c, sf[j][q], negmL);
      if (MASK) x = sf[j][q] == -INFINITY ? -INFINITY : x;
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
  if (DEBUG && dp) {
    // the P code of key key0 + 32j + 8(w%4) + 4hh + e is byte e of word w
#pragma unroll
    for (int w = 0; w < 8; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int off = 32 * (w >> 2) + 8 * (w & 3) + e;
        if (!MASK || off <= lim) dp[key0 + 4 * hh + off] = (uint8_t)((uint32_t)P[w] >> (8 * e));
      }
  }
  return __any(moved);
}

// Per-wave constants of the tile loop.
struct LoopArgs {
  const int8_t *kbase;
  const uint8_t *vbase;
  const v4i *qop;
  float c, Lsc;
  int hh, wv, stream;   // wv: wave index within the stream
  int ntiles_wg, nsteps, t_mask;
  int lim0;   // last key visible to the lane, minus 4*hh
  int32_t *ds;
  uint8_t *dp;
  const uint16_t *kscl;   // per-token K: the fp16 scales of this (batch, kv-head)
  const float *kblk;      // per-block K: the fp32 scales of this (batch, kv-head), one per tile
};

// What the softmax of a tile leaves for the next step, which applies it to (O, l) just
// before adding the tile's PV: the rescale factor, whether any row needs it, and the row
// sum of the P of the tile before (from the matrix core).
struct Carry {
  float alpha;
  float lsum;
  bool any_moved;
};

// Step k of the stream's tile loop (0 <= k < nsteps; the stream's tile k is tile
// kStreams*k + stream of the row block), as one basic block so the scheduler can interleave
// matrix-core and vector work.  On entry Sc holds S of tile k (computed in the previous
// step), Pp the e4m3 P of tile k-1, and cr the softmax results of tile k-1.  The step
// issues QK(k+1) into Sn; runs the softmax of tile k into Pc; applies tile k-1's rescale to
// (O, l) (RESCALE: some row moved its max) and adds the row sum of tile k-2; then issues
// PV(k-1) and the row sum of tile k-1.  Tiles beyond the wave's last visible key are
// computed fully masked, which leaves (m, l, O) unchanged; loads are clamped to the
// workgroup's last tile, whose data is valid, so such steps read only finite values (at
// k = 0, PV reads the finite V data of the stream's first tile with P = 0).
template <int D, int PV, bool MASK, bool RESCALE, bool DEBUG, bool KTOK>
__device__ __forceinline__ void tile_step(RowState<D> &st, v16i (&Sc)[2], v16i (&Sn)[2], const v8i &Pp, v8i &Pc,
                                          Carry &cr, Ring<D> &ring, const Offsets<D> &o, const LoopArgs &a,
                                          int k, const v16i &zero, const v8i &ones, float c) {
  const int key0 = (kStreams * k + a.stream) * KT;
  qk_tile<D>(Sn, ring.k[(k + 1) % kRing], o, a.qop, zero);
  float alpha;
  // (per-token K: the scales of this tile's keys come from its scale slot, which is not refilled
  // in this step)
  const bool moved = softmax_tile<D, PV, MASK, DEBUG, KTOK>(st, Sc, Pc, alpha, c, a.Lsc, key0, a.hh,
                                                            a.lim0 - key0, a.ds, a.dp, ring.ks[k % kRing] + 64 * a.hh);
  st.l += cr.lsum;
  if (RESCALE) {
    st.l *= cr.alpha;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int q = 0; q < 16; ++q) st.O[mt][q] *= cr.alpha;
  }
  cr.lsum = pv_tile<D, PV>(st, Pp, ring.v[(k > 0 ? k - 1 : 0) % kRing], o, ones);
  cr.alpha = alpha;
  cr.any_moved = moved;
}

// The same step for the hot case (d = 128, e4m3 PV, no mask, no debug output) with the
// instruction order fixed by hand.  The 13 MFMAs -- QK(k+1) x8 (32 cycles each), then
// PV(k-1) x4 and its row sum (64 cycles each) -- each open a slot whose vector work runs
// while the MFMA executes; the sched_barriers keep the compiler from regrouping them, which
// would stall the wave on MFMA issue or leave the matrix core idle.  The vector work of tile
// k: the row max (slots 0-1), the new max, exponent offset and the wave's rescale flag (slot
// 2), the row-sum update (slot 3), and (RESCALE) the rescale of O for tile k-1, eight
// accumulators per QK slot, all before PV reads O; the 32 exp2 with their e4m3 packing fill
// the remaining capacity (kExpPerSlot).  The tile loads of the step are issued in slots 1
// and 2.  The arithmetic is that of tile_step.
#define ATTN_Q_FENCE __builtin_amdgcn_sched_barrier(0)
template <bool RESCALE>
struct ExpPlan {
  static constexpr int n[13] = {0, 0, 0, RESCALE ? 1 : 2, RESCALE ? 1 : 2, RESCALE ? 1 : 2, RESCALE ? 1 : 2,
                                RESCALE ? 1 : 2, RESCALE ? 5 : 4, RESCALE ? 5 : 4, RESCALE ? 6 : 5,
                                RESCALE ? 6 : 5, RESCALE ? 5 : 4};
  static constexpr int begin(int slot) {
    int b = 0;
    for (int i = 0; i < slot; ++i) b += n[i];
    return b;
  }
  static_assert(begin(13) == 32, "every exponential in exactly one slot");
  // the slot of exponential e
  static constexpr int slot_of(int e) {
    int i = 0;
    while (begin(i + 1) <= e) ++i;
    return i;
  }
  // (per-token K) the slot that reads scale chunk cc again for exponentials 8cc .. 8cc+7: the
  // slot before the first of them (a table, so the comparison with the unrolled slot index folds)
  static constexpr int read_slot[4] = {slot_of(0) - 1, slot_of(8) - 1, slot_of(16) - 1, slot_of(24) - 1};
  static_assert(read_slot[0] >= 2, "after the max phase's first reads");
};

struct StageArgs {
  uint8_t *kdst, *vdst, *ksdst;
  const int8_t *kbase;
  const uint8_t *vbase;
  const uint16_t *kscl;
  int tk, tv, tks, wv;
};

// Per-token K in the hot step: the scale slot of tile k and the lane's offset in it (16 dwords
// at 64*hh).  A chunk is one 16-byte read: the scales of S elements [cc/2][8(cc%2) ..
// 8(cc%2)+7].
struct TokArgs {
  const uint8_t *ksc;
  int kso;
};

// DEBUG: the step also stores the tile's int32 scores (ds) and P codes (dp) of the lane's row
// at keys koff + 32j + 8r + e (koff = the tile's first key + 4*hh); the kernels that take these
// exports are separate instantiations, so the arithmetic they check is the hot step's own.
template <bool RESCALE, bool KTOK, bool DEBUG>
__device__ __forceinline__ void tile_step_d128(RowState<128> &st, v16i (&Sc)[2], v16i (&Sn)[2], const v8i &Pp,
                                               v8i &Pc, Carry &cr, const uint8_t *kbuf, const uint8_t *vbuf,
                                               const Offsets<128> &o, const v4i *qop, float c, float Lsc,
                                               const v16i &zero, const v8i &ones, const StageArgs &sa,
                                               v4i (&kpre)[2], const uint8_t *knext, const TokArgs &ta,
                                               int32_t *ds, uint8_t *dp, int koff) {
  constexpr int NK = 4;
  using Plan = ExpPlan<RESCALE>;
  // The operand offsets are derived in the step from two registers (the K offsets of chunks
  // kk > 0 and the upper V half differ from the first by an xor of one bit); the opaque asm
  // keeps the derived values from being hoisted out of the loop, where the register
  // allocator would spill them -- and a spill reload waits for every outstanding load,
  // the tile loads in flight included.
  int kop0 = o.kop[0], vop0 = o.vop0;
  asm volatile("" : "+v"(kop0), "+v"(vop0));
  v4i k0[NK], k1[NK];
  v8i vop[NK];
  k0[0] = kpre[0];   // (read at the end of the previous step)
  k1[0] = kpre[1];
  // (per-token K) the tile's scale chunks.  Max phase: slot 0 reads chunks 0 and 1 and converts
  // all 32 scores to fp32 in place; slot 1 takes the max of the dequantized scores
  // fp32(c_j * acc_j) of chains 0 and 1, then reads chunks 2 and 3 into the same registers (a
  // fence keeps the reads after the work that frees them); slot 2 does chains 2 and 3 and the
  // row max.  Exponent phase: each chunk is read again (ke) in the slot before its first
  // exponential, through an opaque offset so the read is not merged with the first one, and c_j
  // is formed again for the fma.
  v4i kc[2], ke[4];
#pragma unroll
  for (int kk = 1; kk < NK; ++kk) {
    const int ko = kop0 ^ (kk << 5);
    k0[kk] = *(const v4i *)(kbuf + ko);
    k1[kk] = *(const v4i *)(kbuf + ko + 32 * 128);
  }
  ATTN_Q_FENCE;
  const float a_prev = cr.alpha;
  float mq[4];
  float negmL = 0.0f, alpha = 1.0f;
  bool any_moved = false;
  float p[2][16];
#pragma unroll
  for (int i = 0; i < 13; ++i) {
    // ---- the slot's MFMA
    if (i < 2 * NK) {
      const int kk = i >> 1;
      if ((i & 1) == 0) Sn[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0[kk], qop[kk], kk == 0 ? zero : Sn[0], 0, 0, 0);
      else Sn[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1[kk], qop[kk], kk == 0 ? zero : Sn[1], 0, 0, 0);
    } else if (i < 3 * NK) {
      const int mt = i - 2 * NK;
      st.O[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mt], Pp, st.O[mt], 0, 0, 0, 0, 0, 0);
    } else {
      cr.lsum = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, Pp, v4f{}, 0, 0, 0, 0, 0, 0)[0];
    }
    ATTN_Q_FENCE;
    // ---- its vector work (the empty asm statements pin each input to its slot, so the
    //      arithmetic is not hoisted above the slot's MFMA)
    if (DEBUG && i == 0 && ds) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) ds[koff + 32 * j + 8 * (q >> 2) + (q & 3)] = Sc[j][q];
    }
    if (KTOK && i == 0) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) kc[cc] = *(const v4i *)(ta.ksc + ta.kso + 16 * cc);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          asm volatile("" : "+v"(Sc[j][q]));
          Sc[j][q] = __float_as_int((float)Sc[j][q]);
        }
    }
    if (KTOK && (i == 1 || i == 2)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // chains 2(i-1), 2(i-1)+1: the max of fp32(c_j * acc_j)
        const int r = 2 * (i - 1) + h, j = r >> 1, b0 = (r & 1) * 8;
        auto dq = [&](int e) {
          return c_times_half(c, kc[h][2 * (e >> 2) + ((e >> 1) & 1)], e & 1) * __int_as_float(Sc[j][b0 + e]);
        };
        float m0 = fmaxf(dq(0), dq(1));
#pragma unroll
        for (int e = 2; e < 8; ++e) m0 = fmaxf(m0, dq(e));
        mq[r] = m0;
      }
      if (i == 1) {
        ATTN_Q_FENCE;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) kc[cc] = *(const v4i *)(ta.ksc + ta.kso + 32 + 16 * cc);
      }
    }
    if (!KTOK && i < 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // 8 scores of tile k to fp32 in place, their max (chains 2i, 2i+1)
        const int r = 2 * i + h, j = r >> 1, b0 = (r & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          asm volatile("" : "+v"(Sc[j][b0 + e]));
          Sc[j][b0 + e] = __float_as_int((float)Sc[j][b0 + e]);
        }
        float m0 = fmaxf(__int_as_float(Sc[j][b0]), __int_as_float(Sc[j][b0 + 1]));
#pragma unroll
        for (int e = 2; e < 8; ++e) m0 = fmaxf(m0, __int_as_float(Sc[j][b0 + e]));
        mq[r] = m0;
      }
    }
    if (i == 1) {
      stage_k<128>(sa.kdst, sa.kbase, sa.tk, sa.wv, o);
      if (KTOK) stage_ks(sa.ksdst, sa.kscl, sa.tks);
    }
    if (i == 4 || i == 8) {
      // V operands of PV, two m-tiles at a time, once the K operands of two QK chunks are
      // consumed (their registers are reused) and ahead of the PV slots that need them
#pragma unroll
      for (int mt = (i - 4) / 2; mt < (i - 4) / 2 + 2; ++mt) {
        const v4i lo = *(const v4i *)(vbuf + vop0 + mt * 32 * KT);
        const v4i hi = *(const v4i *)(vbuf + (vop0 ^ 16) + mt * 32 * KT);
        vop[mt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    if (i == 12) {
      // the first K operands of the next step's QK (K tile k+2, landed before this step's
      // barrier), so that step's first MFMA does not wait on LDS
      kpre[0] = *(const v4i *)(knext + kop0);
      kpre[1] = *(const v4i *)(knext + kop0 + 32 * 128);
    }

    if (i == 2) {
      float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
      mx = max_xor32(mx);
      const float mt_ = KTOK ? mx : c * mx;   // (per-token K: mx is already dequantized)
      const float mnew = fmaxf(st.m, mt_);
      const bool moved = mnew != st.m;
      alpha = fast_exp2(moved ? st.m - mnew : 0.0f);
      st.m = mnew;
      negmL = Lsc - st.m;
      any_moved = __any(moved);
      stage_v<128>(sa.vdst, sa.vbase, sa.tv, sa.wv, o);
    }
    if (i == 3) {
      st.l += cr.lsum;
      if (RESCALE) st.l *= a_prev;
    }
    if (RESCALE && i < 2 * NK) {
      // O *= alpha of tile k-1: m-tile i/2, half i%2
#pragma unroll
      for (int q = 0; q < 8; ++q) st.O[i >> 1][(i & 1) * 8 + q] *= a_prev;
    }
    if constexpr (KTOK) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        if (i == Plan::read_slot[cc]) {
          int off = ta.kso;
          asm volatile("" : "+v"(off));
          ke[cc] = *(const v4i *)(ta.ksc + off + 16 * cc);
        }
    }
    // exponentials of this slot, then the e4m3 words they complete
#pragma unroll
    for (int e = Plan::begin(i); e < Plan::begin(i + 1); ++e) {
      const int j = e >> 4, q = e & 15;
      asm volatile("" : "+v"(Sc[j][q]));
      float cj = c;
      if constexpr (KTOK) cj = c_times_half(c, ke[e >> 3][2 * ((q >> 2) & 1) + ((q >> 1) & 1)], q & 1);
      const float x = __builtin_fmaf(cj, __int_as_float(Sc[j][q]), negmL);
      p[j][q] = fast_exp2(x);
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int last_e = (w >> 2) * 16 + (w & 3) * 4 + 3;
      if (last_e >= Plan::begin(i) && last_e < Plan::begin(i + 1)) {
        const int j = w >> 2, r0 = (w & 3) * 4;
        const int word = cvt_pk_e4m3<false>(p[j][r0], p[j][r0 + 1], Pc[w]);
        Pc[w] = cvt_pk_e4m3<true>(p[j][r0 + 2], p[j][r0 + 3], word);
      }
    }
    ATTN_Q_FENCE;
  }
  cr.alpha = alpha;
  cr.any_moved = any_moved;
  if (DEBUG && dp) {
#pragma unroll
    for (int w = 0; w < 8; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[koff + 32 * (w >> 2) + 8 * (w & 3) + e] = (uint8_t)((uint32_t)Pc[w] >> (8 * e));
  }
}

// the instantiation whose unmasked steps take tile_step_d128
template <int D, int PV, bool DEBUG, int KM>
constexpr bool kHotStep = D == 128 && PV == ATTN_Q_PV_FP8;

template <int D, int PV, bool DEBUG, int KM>
__device__ __forceinline__ void step(RowState<D> &st, v16i (&Sc)[2], v16i (&Sn)[2], const v8i &Pp, v8i &Pc,
                                     Carry &cr, Ring<D> &ring, const Offsets<D> &o, const LoopArgs &a, int k,
                                     const v16i &zero, const v8i &ones, v4i (&kpre)[2]) {
  const int last = a.ntiles_wg - 1;
  const int t = kStreams * k + a.stream;                        // tile of the row block
  const int tk = min(kStreams * (k + kRing) + a.stream, last);  // K tile loaded in this step
  const int tv = min(kStreams * (k + kRing - 2) + a.stream, last);
  // (per-token K: the scales of K tile k+kRing-1, into the slot of tile k-1, whose scales the
  //  previous step read last; so the scales of tiles k and k+1 stay in place during the step)
  const int tks = min(kStreams * (k + kRing - 1) + a.stream, last);
  uint8_t *ksdst = ring.ks[(k + kRing - 1) % kRing];
  constexpr bool KTOK = KM == kKmTok;
  // the row constant of this tile's keys: c, or fp32(c * s_K[tile]) for per-block K (the
  // scale requested before the barrier, so its latency passes there)
  float ct = a.c;
  if constexpr (KM == kKmBlk) ct = a.c * a.kblk[min(t, last)];
  // the tiles read in this step have landed in every wave, and every wave is done with
  // the slots refilled below
  wait_tiles<D, DEBUG, KTOK>();
  step_barrier();
  // (t_mask lives in a scalar register; the copy into a vector register, made here every step,
  //  keeps the branch in the form the register allocator handles well without a loop-long
  //  vector register for it -- which it would spill, and a spill reload waits for every
  //  outstanding tile load)
  int tmv;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tmv) : "s"(a.t_mask));
  if constexpr (kHotStep<D, PV, DEBUG, KM>) {
    if (t < tmv) {
      // (this path issues the step's tile loads itself, between its MFMAs)
      const StageArgs sa{ring.k[k % kRing], ring.v[(k + kRing - 2) % kRing], ksdst, a.kbase, a.vbase, a.kscl,
                         tk, tv, tks, a.wv};
      const uint8_t *kbuf = ring.k[(k + 1) % kRing], *vbuf = ring.v[(k > 0 ? k - 1 : 0) % kRing];
      const uint8_t *knext = ring.k[(k + 2) % kRing];
      const TokArgs ta{ring.ks[k % kRing], 64 * a.hh};
      const int koff = t * KT + 4 * a.hh;
      if (cr.any_moved)
        tile_step_d128<true, KTOK, DEBUG>(st, Sc, Sn, Pp, Pc, cr, kbuf, vbuf, o, a.qop, ct, a.Lsc, zero, ones, sa,
                                          kpre, knext, ta, a.ds, a.dp, koff);
      else
        tile_step_d128<false, KTOK, DEBUG>(st, Sc, Sn, Pp, Pc, cr, kbuf, vbuf, o, a.qop, ct, a.Lsc, zero, ones, sa,
                                           kpre, knext, ta, a.ds, a.dp, koff);
      return;
    }
  }
  stage_k<D>(ring.k[k % kRing], a.kbase, tk, a.wv, o);
  stage_v<D>(ring.v[(k + kRing - 2) % kRing], a.vbase, tv, a.wv, o);
  if (KTOK) stage_ks(ksdst, a.kscl, tks);
  if (t < tmv) {
    if (cr.any_moved) tile_step<D, PV, false, true, DEBUG, KTOK>(st, Sc, Sn, Pp, Pc, cr, ring, o, a, k, zero, ones, ct);
    else tile_step<D, PV, false, false, DEBUG, KTOK>(st, Sc, Sn, Pp, Pc, cr, ring, o, a, k, zero, ones, ct);
  } else {
    if (cr.any_moved) tile_step<D, PV, true, true, DEBUG, KTOK>(st, Sc, Sn, Pp, Pc, cr, ring, o, a, k, zero, ones, ct);
    else tile_step<D, PV, true, false, DEBUG, KTOK>(st, Sc, Sn, Pp, Pc, cr, ring, o, a, k, zero, ones, ct);
  }
}

template <int D, int PV, bool DEBUG, int KM>
__device__ __forceinline__ void tile_loop(RowState<D> &st, Ring<D> &ring, const Offsets<D> &o,
                                          const LoopArgs &a) {
  // (FP8: e4m3 1.0 where output row block (l%16)/4 and key block l/16 have the same parity,
  //  0 elsewhere; INT8: 1 everywhere)
  const int ln = threadIdx.x & 63;
  const int one = PV == ATTN_Q_PV_FP8 ? ((((ln & 15) >> 2) & 1) == ((ln >> 4) & 1) ? 0x38383838 : 0) : 0x01010101;
  v8i ones = v8i{one, one, one, one, one, one, one, one};
  asm volatile("" : "+v"(ones));   // keep the constant operands resident in registers
  const v16i zero = v16i{};
  const int n_k = a.nsteps, last = a.ntiles_wg - 1;
  // prologue: the stream's K tiles 0 .. kRing-1 and V tiles 0 .. kRing-3, then QK of its
  // tile 0
#pragma unroll
  for (int j = 0; j < kRing; ++j) stage_k<D>(ring.k[j], a.kbase, min(kStreams * j + a.stream, last), a.wv, o);
#pragma unroll
  for (int j = 0; j < kRing - 2; ++j) stage_v<D>(ring.v[j], a.vbase, min(kStreams * j + a.stream, last), a.wv, o);
  if constexpr (KM == kKmTok) {
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j) stage_ks(ring.ks[j], a.kscl, min(kStreams * j + a.stream, last));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  v16i Sa[2], Sb[2];
  qk_tile<D>(Sa, ring.k[0], o, a.qop, zero);
  // (hot steps: the first K operands of step 0's QK, which reads the stream's tile 1; every
  //  hot step reads those of the next one.  Hot steps form a prefix of the loop.)
  v4i kpre[2] = {v4i{}, v4i{}};
  if constexpr (kHotStep<D, PV, DEBUG, KM>) {
    kpre[0] = *(const v4i *)(ring.k[1] + o.kop[0]);
    kpre[1] = *(const v4i *)(ring.k[1] + o.kop[0] + 32 * D);
  }
  v8i Pa = v8i{}, Pb = v8i{};
  Carry cr{1.0f, 0.0f, false};
  // two steps per iteration so the S and P buffers swap roles without copies
  for (int k = 0; k < n_k; k += 2) {
    step<D, PV, DEBUG, KM>(st, Sa, Sb, Pb, Pa, cr, ring, o, a, k, zero, ones, kpre);
    if (k + 1 < n_k) step<D, PV, DEBUG, KM>(st, Sb, Sa, Pa, Pb, cr, ring, o, a, k + 1, zero, ones, kpre);
  }
  // the stream's last tile: its rescale, the row sum of the tile before, its PV and row
  // sum; no load may still be landing afterwards (the ring is reused for the merge)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  st.l += cr.lsum;
  if (cr.any_moved) {
    st.l *= cr.alpha;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int q = 0; q < 16; ++q) st.O[mt][q] *= cr.alpha;
  }
  st.l += pv_tile<D, PV>(st, (n_k & 1) ? Pa : Pb, ring.v[(n_k - 1) % kRing], o, ones);
  __syncthreads();
}

template <int D, int PV, bool DEBUG, int KM>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillLaunch a, int nblk, int total) {
  constexpr bool KTOK = KM == kKmTok;
  constexpr int NK = D / 32;  // 32-wide d chunks = QK MFMAs per S tile = PV m-tiles
  __shared__ __attribute__((aligned(16))) Ring<D> s_ring[kStreams];
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
  const int stid = threadIdx.x % kStreamThreads;   // thread index within the stream
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
      const float *ks = (const float *)a.k_scales + (size_t)bg * D + kk * 32 + hh * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) qf[kk][e] = qf[kk][e] * ks[e];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(qf[kk][e]));
  }
  float sq;
  if (a.q_gran == ATTN_Q_GRAN_TENSOR) {
    sq = __uint_as_float(*(const uint32_t *)a.ws) / 127.0f;
  } else if (a.q_gran == ATTN_Q_GRAN_BLOCK) {
    sq = ((const float *)a.ws)[((size_t)b * a.Hq + (row_valid ? h : g * G)) * ((a.q_len + 63) / 64) + iq / 64];
  } else {
    amax = max_xor32(amax);
    sq = amax / 127.0f;
  }
  float c = sq * a.kconst;
  if (a.k_gran == ATTN_Q_GRAN_TENSOR) c = c * ((const float *)a.k_scales)[0];
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

  // ---- this wave's tiles: [0, t_mask) of the row block need no mask, the rest do
  const int i_lo = min(wrow0 / G, a.q_len - 1);
  const int i_hi = min((wrow0 + kRowsPerWave - 1) / G, a.q_len - 1);
  const int kv_end = causal ? min(a.kv_len, a.q_offset + i_hi + 1) : a.kv_len;
  int t_mask = min((kv_end + KT - 1) / KT, a.kv_len / KT);
  if (causal) t_mask = min(t_mask, (a.q_offset + i_lo + 1) / KT);
  const int vis_last = causal ? a.q_offset + iq : a.kv_len - 1;  // last visible key of the lane

  const float Lsc = PV == ATTN_Q_PV_FP8 ? kLog2_448 : kLog2_127;
  RowState<D> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int mt = 0; mt < NK; ++mt) st.O[mt] = v16f{};
  int32_t *ds = nullptr;
  uint8_t *dp = nullptr;
  if (DEBUG && row_valid && a.debug_s) ds = a.debug_s + (((size_t)b * a.Hq + h) * a.q_len + i) * a.kv_len;
  if (DEBUG && row_valid && a.debug_p) dp = a.debug_p + (((size_t)b * a.Hq + h) * a.q_len + i) * a.kv_len;

  const Offsets<D> o = make_offsets<D>(stid, n, hh);
  const int nsteps = (ntiles_wg + kStreams - 1) / kStreams;
  const LoopArgs la{kbase, vbase, qop, c, Lsc, hh, rw, stream, ntiles_wg, nsteps, t_mask,
                    min(vis_last, a.kv_len - 1) - 4 * hh, ds, dp,
                    (const uint16_t *)a.k_scales + (KTOK ? (size_t)bg * a.cap : 0),
                    (const float *)a.k_scales + (KM == kKmBlk ? (size_t)bg * (a.cap / KT) : 0)};
  {
    // (the stream is uniform across the wave; taking its ring and tile bases through
    //  readfirstlane lets the per-step addresses be scalar)
    LoopArgs lu = la;
    lu.kbase = (const int8_t *)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)kbase >> 32)) << 32) |
                                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)kbase));
    lu.vbase = (const uint8_t *)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)vbase >> 32)) << 32) |
                                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)vbase));
    if constexpr (KTOK)
      lu.kscl = (const uint16_t *)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)la.kscl >> 32)) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)la.kscl));
    lu.stream = __builtin_amdgcn_readfirstlane(stream);
    lu.wv = __builtin_amdgcn_readfirstlane(rw);
    // (wave-uniform: the step's branch on it is scalar and it stays in a scalar register)
    lu.t_mask = __builtin_amdgcn_readfirstlane(t_mask);
    tile_loop<D, PV, DEBUG, KM>(st, s_ring[lu.stream], o, lu);
  }

  // ---- merge the key streams through LDS (reusing the staging ring), one m-tile at a
  //      time: stream 1 hands (m, l, O) to stream 0
  float *xch = (float *)&s_ring[0];   // [kRowWaves][18][64] floats
  static_assert(kRowWaves * 18 * 64 * 4 <= sizeof(s_ring), "merge buffer");
  float f1 = 1.0f, f2 = 0.0f;
#pragma unroll
  for (int mt = 0; mt < NK; ++mt) {
    float *xp = xch + (rw * 18) * 64 + lane;
    if (stream == 1) {
      if (mt == 0) { xp[0] = st.m; xp[64] = st.l; }
#pragma unroll
      for (int q = 0; q < 16; ++q) xp[(2 + q) * 64] = st.O[mt][q];
    }
    __syncthreads();
    if (stream == 0) {
      if (mt == 0) {
        const float m2 = xp[0], l2 = xp[64];
        const float M = fmaxf(st.m, m2);
        f1 = st.m == -INFINITY ? 0.0f : fast_exp2(st.m - M);
        f2 = m2 == -INFINITY ? 0.0f : fast_exp2(m2 - M);
        st.l = st.l * f1 + l2 * f2;
        st.m = M;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) st.O[mt][q] = st.O[mt][q] * f1 + xp[(2 + q) * 64] * f2;
    }
    __syncthreads();
  }
  if (stream > 0) return;

  // ---- epilogue: o = O * g / l with g = s_V[c] (per-channel V) or 1 / c_V (per-token V, whose
  //      operand carries s_V[n] * c_V); lse = m + log2(l) - log2(static scale)
  const float inv = 1.0f / st.l;   // the MFMA row sum is complete in both lane halves
  if (!row_valid) return;
  if (a.lse && hh == 0) a.lse[((size_t)b * a.Hq + h) * a.q_len + i] = st.m + (__builtin_amdgcn_logf(st.l) - Lsc);
  const size_t orow = (((size_t)b * a.Hq + h) * a.q_len + i) * D;
  const bool vtok = a.v_gran == ATTN_Q_GRAN_TOKEN;
  const float *vs = a.v_scales + (vtok ? 0 : (size_t)bg * D);
  const float gtok = vtok ? token_v_gain(a.v_scale_max[bg]) * inv : 0.0f;
#pragma unroll
  for (int mt = 0; mt < NK; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int ch = mt * 32 + 8 * r4 + 4 * hh;
      float ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = st.O[mt][4 * r4 + e] * (vtok ? gtok : vs[ch + e] * inv);
      if (a.out_f32) {
        *(float4 *)((float *)a.out + orow + ch) = make_float4(ov[0], ov[1], ov[2], ov[3]);
      } else {
        __half2 lo = __floats2half2_rn(ov[0], ov[1]), hi = __floats2half2_rn(ov[2], ov[3]);
        uint2 pk = make_uint2(*(uint32_t *)&lo, *(uint32_t *)&hi);
        *(uint2 *)((__half *)a.out + orow + ch) = pk;
      }
    }
}

template <int D, int PV, int KM>
hipError_t launch_k(const PrefillLaunch &a, hipStream_t s, dim3 grid, int nblk, int total) {
  if (a.debug_s || a.debug_p)
    hipLaunchKernelGGL((prefill_kernel<D, PV, true, KM>), grid, dim3(kThreads), 0, s, a, nblk, total);
  else
    hipLaunchKernelGGL((prefill_kernel<D, PV, false, KM>), grid, dim3(kThreads), 0, s, a, nblk, total);
  return hipGetLastError();
}

template <int D, int PV>
hipError_t launch_t(const PrefillLaunch &a, hipStream_t s, dim3 grid, int nblk, int total) {
  if (a.k_gran == ATTN_Q_GRAN_TOKEN) return launch_k<D, PV, kKmTok>(a, s, grid, nblk, total);
  if (a.k_gran == ATTN_Q_GRAN_BLOCK) return launch_k<D, PV, kKmBlk>(a, s, grid, nblk, total);
  return launch_k<D, PV, kKmRow>(a, s, grid, nblk, total);
}

template <int D>
hipError_t launch_d(const PrefillLaunch &a, hipStream_t s, dim3 grid, int nblk, int total) {
  return a.pv_mode == ATTN_Q_PV_FP8 ? launch_t<D, ATTN_Q_PV_FP8>(a, s, grid, nblk, total)
                                    : launch_t<D, ATTN_Q_PV_INT8>(a, s, grid, nblk, total);
}

}  // namespace

size_t prefill_workspace_bytes(int q_gran, int B, int Hq, int q_len) {
  if (q_gran == ATTN_Q_GRAN_TENSOR) return 256;
  if (q_gran == ATTN_Q_GRAN_BLOCK) return ((size_t)B * Hq * ((q_len + 63) / 64) * 4 + 255) / 256 * 256;
  return 0;
}

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t s) {
  if (a.q_len == 0) return hipSuccess;
  if (a.q_gran == ATTN_Q_GRAN_TENSOR) {
    hipLaunchKernelGGL(prefill_ws_init, dim3(1), dim3(1), 0, s, (uint32_t *)a.ws);
    const size_t n = (size_t)a.B * a.Hq * a.q_len * a.D;
    const int blocks = (int)std::min<size_t>((n / 8 + kAmaxThreads - 1) / kAmaxThreads, kAmaxBlocks);
    hipLaunchKernelGGL(q_amax_kernel, dim3(blocks), dim3(kAmaxThreads), 0, s, a.q, n, a.D, a.Hq, a.Hkv,
                       a.q_len, (const float *)a.k_scales, (int)(a.k_gran == ATTN_Q_GRAN_CHANNEL), (uint32_t *)a.ws);
  } else if (a.q_gran == ATTN_Q_GRAN_BLOCK) {
    hipLaunchKernelGGL(q_block_scale_kernel, dim3((a.q_len + 63) / 64, a.B * a.Hq), dim3(256), 0, s, a.q, a.D, a.Hq,
                       a.Hkv, a.q_len, (const float *)a.k_scales, (int)(a.k_gran == ATTN_Q_GRAN_CHANNEL), (float *)a.ws);
  }
  const int G = a.Hq / a.Hkv;
  const int nblk = (G * a.q_len + kRowsPerWG - 1) / kRowsPerWG;
  const int total = a.B * a.Hkv * nblk;
  dim3 grid((total + 7) / 8 * 8);
  return a.D == 128 ? launch_d<128>(a, s, grid, nblk, total) : launch_d<64>(a, s, grid, nblk, total);
}

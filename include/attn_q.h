/*
 * attn_q.h -- C ABI of libattn_q.so: quantized flash attention for MI355X (gfx950).
 *
 * The method ("int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8",
 * zolotukhin.ai): the QK^T product runs on int8 with int32 accumulation after K's
 * per-channel mean is subtracted (exact, because softmax ignores a constant added
 * to every score of a row -- section "Why does subtracting K's channel mean not
 * change the attention output?"); the online softmax keeps its running row max
 * m and exp(s - m) in fp32, so every probability is <= 1 and P needs no
 * max-finding reduction (section "The scale P needs is already sitting in a
 * register"); P is stored as OCP e4m3 with the static scale 448 and the PV
 * product runs on fp8 (section "fp8 is not faster, it is shaped correctly");
 * decode streams the int8 KV cache (section "What actually changed for decode").
 * The int8 quantizer is symmetric with scale amax/127 (eq. (1)-(2) of "QFlash:
 * Bridging Quantization and Memory Efficiency in Vision Transformer Attention").
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates device memory, never synchronizes, and keeps no mutable
 *    global state apart from a per-device cache of the device's architecture.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream).
 *    Asynchronous faults surface at the caller's next synchronization.
 *  - Arguments are validated before any HIP call; a negative attn_q_status is
 *    returned and nothing is launched.  No entry point aborts or throws.
 *  - fp16 means IEEE binary16, e4m3 means OCP FP8 E4M3 (bias 7, max 448, NaN =
 *    0x7F/0xFF), int8 codes lie in [-127, 127], rounding is to nearest-even.
 *  - Tensors are dense row-major in the order written in brackets.  Code rows
 *    (head_dim bytes) must be 16-byte aligned; head_dim is 64 or 128.
 *  - Results are deterministic: the same inputs give identical bytes.
 */
#ifndef ATTN_Q_H
#define ATTN_Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_Q_ABI_VERSION 6
/* Keys per online-softmax step of attn_q_prefill (the B_c of the tiled loop over
 * key blocks in QFlash's Algorithm 1).  P codes depend on the running max, so
 * this width is part of the numerical contract. */
#define ATTN_Q_KEY_TILE 64
/* Key tiles are dealt round-robin to this many streams (tile t to stream t % 2); each
 * stream runs its own online softmax over its tiles in ascending order and the streams
 * are merged at the end: M = max_s m_s, O = sum_s 2^(m_s - M) O_s, l likewise.  Also
 * part of the numerical contract (P codes depend on the stream's running max). */
#define ATTN_Q_KEY_STREAMS 2

typedef enum {
  ATTN_Q_OK = 0,
  ATTN_Q_E_NULL = -1,        /* a required pointer is NULL                      */
  ATTN_Q_E_SHAPE = -2,       /* inconsistent or out-of-range sizes               */
  ATTN_Q_E_UNSUPPORTED = -3, /* valid but not implemented (granularity, head_dim)*/
  ATTN_Q_E_ALIGN = -4,       /* a pointer is not aligned as documented           */
  ATTN_Q_E_WORKSPACE = -5,   /* workspace NULL or smaller than *_workspace_size  */
  ATTN_Q_E_DEVICE = -6,      /* current device is not gfx950 or HIP query failed */
  ATTN_Q_E_LAUNCH = -7,      /* a kernel launch returned an error                */
  ATTN_Q_E_SCRATCH = -8      /* larger than the static scratch of a no-allocation call */
} attn_q_status;

/* Quantization granularity: which elements share one int8 scale. */
typedef enum {
  ATTN_Q_GRAN_TENSOR = 0,  /* one fp32 scale for the whole tensor (QFlash section 3.3, C3) */
  ATTN_Q_GRAN_BLOCK = 1,   /* one fp32 scale per block of ATTN_Q_BLOCK consecutive tokens of a
                              (batch, head): QFlash's per-block quantization (section 3.3, C3)
                              with the blocks of its tiled loop -- for K the 64-key tile        */
  ATTN_Q_GRAN_TOKEN = 2,   /* one scale per token row                                        */
  ATTN_Q_GRAN_CHANNEL = 3  /* one fp32 scale per (batch, kv-head, channel)                    */
} attn_q_gran;

/* Tokens per ATTN_Q_GRAN_BLOCK scale (keys of K, query positions of Q). */
#define ATTN_Q_BLOCK 64

typedef enum {
  ATTN_Q_PV_FP8 = 0,     /* P and V as e4m3 on the fp8 matrix cores (P scale 448)           */
  ATTN_Q_PV_INT8 = 1,    /* comparison variant: P as int8 with static scale 127, int8 PV    */
  ATTN_Q_PV_SPLIT24 = 2  /* precision mode: int8 K and V codes as stored; q and p split into
                            three exact 8-bit parts (24 bits), int8 matrix cores for both
                            products, parts combined in fp32 (attn_q_prefill only)           */
} attn_q_pv_mode;

typedef enum { ATTN_Q_OUT_F16 = 0, ATTN_Q_OUT_F32 = 1 } attn_q_out_dtype;

/* ------------------------------------------------------------------------ */
/* kv_quantize_i8: fp16 K/V -> int8 KV cache.
 *
 * K mean (k_mean): one vector per (batch, kv-head) over all seq_len keys,
 *   mu_c = fp32( S_c / (seq_len * 2^24) ) with S_c = sum_n k[n][c] * 2^24 taken
 *   exactly in int64 (every fp16 times 2^24 is an integer).  It is the constant
 *   shift of the page's mean subtraction; zeros when subtract_k_mean == 0.
 * K codes: x = fp32(k) - mu (fp32); scale over the granularity set
 *   s = fp32(amax / 127), rounded to its storage type; code = clamp(rint(x / s_stored),
 *   -127, 127) with an IEEE fp32 division; a zero scale gives code 0.  k_gran BLOCK: the set
 *   is a block of ATTN_Q_BLOCK keys (its keys below seq_len, all channels); requires
 *   capacity % ATTN_Q_BLOCK == 0.
 * V codes: the same without a mean.
 * v_op (optional, NULL = not written): the V operand of attn_q_prefill,
 *   uint8 [B][Hkv][capacity/64][head_dim][64].  Byte p of channel c in key tile T
 *   holds key 64*T + perm(p), perm(p) = 32*((p%32)/16) + 8*((p%16)/4) + 4*(p/32) + p%4;
 *   keys >= seq_len (up to capacity) are 0.  Requires capacity % 64 == 0.  (The permutation
 *   is the order in which one 64-wide matrix-core wave holds a 64-key tile of P, so the PV
 *   operand needs no transposition on the hot path.)  Contents:
 *   - v_gran CHANNEL: e4m3(fp32(code)) for v_op_format ATTN_Q_PV_FP8, or the int8 code for
 *     ATTN_Q_PV_INT8 (the channel scale s_V[c] is applied after the product);
 *   - v_gran TOKEN (ATTN_Q_PV_FP8 only): e4m3(fp32(code * f_n)), f_n = fp32(s_V[n] * c_V),
 *     c_V = fp32(448 / fp32(127 * V_max)) (0 if V_max = 0), where V_max = max_n s_V[n] over
 *     the seq_len keys is the cache header written to v_scale_max (fp32 [B][Hkv]); every
 *     value then lies within 448, so P keeps its static scale, and the prefill multiplies
 *     its output by fp32(1 / c_V).  ("int8 Flash Attention on RDNA4", section "fp8 is not
 *     faster, it is shaped correctly": P and V enter the PV product as fp8.)
 *   attn_q_v_operand rebuilds the operand (and the header) from the codes and scales, e.g.
 *   after attn_q_kv_append_i8 has grown the cache.
 *
 * k_sum (optional, NULL = not written): int64 [B][Hkv][d] receives S_c itself (computed
 *   also when subtract_k_mean == 0), the cache header from which attn_q_kv_append_i8
 *   continues the running mean.
 *
 * Buffers: k, v fp16 [B][Hkv][seq_len][d]; k_codes, v_codes int8 [B][Hkv][capacity][d]
 *   (rows >= seq_len untouched; v_codes may be NULL when v_op is written with per-channel V:
 *   a cache that serves attn_q_prefill's fp8 PV only -- attn_q_decode, attn_q_v_operand and
 *   the int8 PV modes read the V codes); k_scales: TOKEN fp16 [B][Hkv][capacity], CHANNEL fp32
 *   [B][Hkv][d], BLOCK fp32 [B][Hkv][capacity / 64] (blocks past seq_len untouched), TENSOR
 *   fp32 [1]; v_scales: TOKEN fp16 [B][Hkv][capacity], CHANNEL
 *   fp32 [B][Hkv][d]; k_mean fp32 [B][Hkv][d].  batch * kv_heads <= 65535.
 *   workspace: kv_quantize_i8_workspace_size
 *   bytes of accumulators; it must be zero-filled before its first use, and every call
 *   leaves it zero-filled again, so it may be reused by later calls with the same
 *   (batch, kv_heads, head_dim) on the same stream.  seq_len >= 1.  Calls are
 *   stream-ordered; concurrent calls on different streams need separate workspaces.
 */
typedef struct {
  int32_t batch, kv_heads, seq_len, head_dim, capacity;
  const void *k, *v;
  int32_t subtract_k_mean;
  int32_t k_gran;                 /* TOKEN | CHANNEL | BLOCK | TENSOR */
  int32_t v_gran;                 /* TOKEN | CHANNEL                  */
  int8_t *k_codes, *v_codes;
  void *k_scales, *v_scales;
  float *k_mean;
  int64_t *k_sum;                 /* optional header output */
  uint8_t *v_op;
  int32_t v_op_format;            /* ATTN_Q_PV_FP8 | ATTN_Q_PV_INT8 */
  float *v_scale_max;             /* header V_max, fp32 [B][Hkv] (v_op with v_gran TOKEN) */
  void *workspace;
  size_t workspace_bytes;
} attn_q_kvq_args;

/* ------------------------------------------------------------------------ */
/* attn_q_v_operand: (re)build the prefill's V operand v_op of a cache from its int8 V codes
 * and scales over keys [0, n_keys) -- exactly as kv_quantize_i8 writes it (see v_op above),
 * including, for per-token V, the header V_max (v_scale_max, written here).  A cache grown by
 * attn_q_kv_append_i8 (per-token scales) is brought to attn_q_prefill this way.
 * Buffers: v_codes int8 [B][Hkv][capacity][d]; v_scales TOKEN fp16 [B][Hkv][capacity] or
 *   CHANNEL fp32 [B][Hkv][d]; v_op uint8 [B][Hkv][capacity/64][d][64] (every tile written;
 *   keys >= n_keys are 0); v_scale_max fp32 [B][Hkv] (TOKEN only).
 * Requirements: 1 <= n_keys <= capacity, capacity % 64 == 0; v_op_format ATTN_Q_PV_FP8, or
 *   ATTN_Q_PV_INT8 with v_gran CHANNEL.  No workspace.
 */
typedef struct {
  int32_t batch, kv_heads, head_dim, capacity, n_keys;
  const int8_t *v_codes;
  const void *v_scales;
  int32_t v_gran;                 /* TOKEN | CHANNEL */
  uint8_t *v_op;
  int32_t v_op_format;            /* ATTN_Q_PV_FP8 | ATTN_Q_PV_INT8 */
  float *v_scale_max;
} attn_q_vop_args;
int attn_q_v_operand(const attn_q_vop_args *a, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* attn_q_kv_append_i8: append new_tokens fp16 K/V rows to an int8 cache at row seq_len,
 * keeping the running per-channel K mean in the cache header (the decode-time cache of
 * "int8 Flash Attention on RDNA4", section "K's outliers, and the subtraction softmax
 * does not notice": K arrives one token at a time, the mean lags by one token, so the
 * shift differs slightly from key to key -- a difference below fp16 round-off on
 * LLM-like keys when the appended tokens are few next to the prompt).
 *
 * Header k_sum: int64 [B][Hkv][d], S_c = sum of k[n][c] * 2^24 (exact) over the seq_len
 *   keys already in the cache.  kv_quantize_i8 writes it through its k_sum field; an
 *   empty cache starts from zeros.  On return it holds the sum over seq_len + new_tokens.
 * Token n = seq_len + t (t = 0 .. new_tokens-1, in order): S_n is the header sum over the
 *   n keys before it, mu_n = fp32(S_n / (n * 2^24)) (IEEE fp64 division) and mu_0 = 0;
 *   x = fp32(k) - mu_n (fp32); s_K = fp16(fp32(max_c |x_c| / 127)); code = clamp(rint(x /
 *   s_K), -127, 127) with an IEEE fp32 division, 0 for a zero scale.  V: the same without
 *   a shift.  (These are the per-token scales of kv_quantize_i8's TOKEN granularity: a
 *   shift that moves with n leaves no fixed per-channel range.)
 * k_mean (optional, NULL = not written): fp32 [B][Hkv][d] = fp32(S / (n_total * 2^24)) of
 *   the header after the append.
 * The cache is read by attn_q_decode with k_gran = v_gran = ATTN_Q_GRAN_TOKEN; a prompt
 *   placed by kv_quantize_i8 must use TOKEN for K and V too.
 *
 * Buffers: k, v fp16 [B][Hkv][new_tokens][d]; k_codes, v_codes int8 [B][Hkv][capacity][d]
 *   (rows seq_len .. seq_len + new_tokens - 1 written, every other row untouched);
 *   k_scales, v_scales fp16 [B][Hkv][capacity] (same rows).
 * Requirements: seq_len >= 0, new_tokens >= 0 (0 = no-op), seq_len + new_tokens <=
 *   capacity.  workspace: attn_q_kv_append_i8_workspace_size bytes (0 when new_tokens <=
 *   64: then NULL is allowed); contents need not be initialised.  Calls that overlap in
 *   time must not share a workspace or a cache.
 */
typedef struct {
  int32_t batch, kv_heads, head_dim, capacity;
  int32_t seq_len, new_tokens;
  const void *k, *v;
  int64_t *k_sum;
  int8_t *k_codes, *v_codes;
  void *k_scales, *v_scales;
  float *k_mean;
  void *workspace;
  size_t workspace_bytes;
} attn_q_kv_append_args;

/* ------------------------------------------------------------------------ */
/* attn_q_prefill: fused quantized flash-attention forward for a chunk of queries.
 *
 * Query row (b, h, i), kv-head g = h / (q_heads / kv_heads), sees key j iff
 * j < kv_len and (causal == 0 or j <= q_offset + i).  Per row:
 *   q' = fp32(q) * s_K[c] (K CHANNEL) or fp32(q); s_Q = fp32(amax(q')/127) per row
 *   (q_gran TOKEN), per block of ATTN_Q_BLOCK query positions of the (batch, head) (BLOCK;
 *   a pass before the kernel writes them to the workspace) or over the whole tensor
 *   (TENSOR); q_code = clamp(rint(q'/s_Q)).
 *   acc_j = sum_c q_code_c * k_code_{j,c}                      exact int32
 *   c_j = fp32(s_Q * kconst) (K CHANNEL), fp32(fp32(s_Q * kconst) * s_K) (K TENSOR) or
 *   fp32(fp32(s_Q * kconst) * s_K[j]) (K TOKEN: one fp16 scale per key; K BLOCK: the fp32 scale
 *   of j's 64-key block, constant over a key tile; nothing folded into q for either),
 *   kconst = fp32(sm_scale * log2 e) in fp64 rounded once (sm_scale <= 0: 1/sqrt(d)).
 *   Per key stream (see ATTN_Q_KEY_STREAMS), for each of its key tiles in ascending order:
 *     m = max(m, max_j fp32(c_j * acc_j)) ; mL = fp32(m - log2(448))  (log2(127) for INT8)
 *     p_j = exp2(fp32(c_j * acc_j - mL)), the argument rounded once (a fused multiply-add)
 *         (= 448 * exp(s_j - m) <= 448, fp32)
 *     P_j = e4m3(p_j) (FP8) or rint(p_j) (INT8) ; l = alpha*l + sum dec(P_j) ;
 *     O = alpha*O + sum_j dec(P_j) * vop_j, alpha = exp2(m_old - m)
 *   streams merged as above; out_c = O_c * s_V[c] / l.
 * l sums the quantized weights, so mass whose P code is zero drops out of the normalization.
 *
 * pv_mode ATTN_Q_PV_SPLIT24 (the precision mode of the "Strata" int8-KV prompt attention,
 * which keeps K and V as stored int8 codes and splits the other operand of each product into
 * three exact 8-bit parts): X_c = rint(q'_c / s_Q * 2^16) and W_j = rint(p_j / p_max * 127 * 2^16)
 * (p_max the largest p of the row in the 64-key tile, so every tile keeps 24 bits) are
 * written as 2^16 h + 2^8 l + m with signed-byte digits; each digit's product with the int8
 * codes is an exact int32 sum on the matrix core; the three sums are combined in fp32.  The
 * online softmax is as above, with p_j unquantized in the exponent and l the sum of W_j.  The
 * result approaches fp64 attention over the dequantized cache (codes times scales) to about
 * 1e-5 relative.  Requires q_gran TOKEN, k_gran CHANNEL or TENSOR, debug_s NULL and v_op written by kv_quantize_i8 with
 * v_op_format ATTN_Q_PV_INT8.
 * The exp2 is the hardware fp32 exp2; P codes may differ from a correctly rounded
 * exp2 in the last place in rare cases, and the fp32 sums are in matrix-core order.
 *
 * Output: out_c = O_c * g_c / l with g_c = s_V[c] (v_gran CHANNEL) or g = fp32(1 / c_V)
 *   (v_gran TOKEN, whose V operand carries f_n = fp32(s_V[n] * c_V) -- see kv_quantize_i8's
 *   v_op).  lse (optional, NULL = not written) receives the base-2 log-sum-exp of the row,
 *   m + log2(l) - log2(448) (log2(127) for INT8), in the units of c * acc: the merge
 *   weight of the row's result when chunks of keys are attended separately
 *   (out = sum_k 2^(lse_k - LSE) out_k with LSE = log2 sum_k 2^lse_k).  (QFlash,
 *   Algorithm 1: the output step normalizes by l; the log-sum-exp is the standard
 *   companion the blocked loop keeps.)
 * Buffers: q fp16 [B][Hq][q_len][d]; k_codes int8 [B][Hkv][capacity][d]; k_scales
 *   fp32 [B][Hkv][d] (CHANNEL), fp32 [1] (TENSOR), fp16 [B][Hkv][capacity] (TOKEN, the
 *   per-token scales of kv_quantize_i8 and attn_q_kv_append_i8) or fp32 [B][Hkv][capacity/64]
 *   (BLOCK); v_op as written by kv_quantize_i8
 *   with the matching format; v_scales fp32 [B][Hkv][d] (V CHANNEL; unused for TOKEN);
 *   v_scale_max fp32 [B][Hkv] (V TOKEN, the header kv_quantize_i8 writes with v_op);
 *   out [B][Hq][q_len][d] fp16 or fp32; lse fp32 [B][Hq][q_len];
 *   debug_s (optional, NULL = off) int32 [B][Hq][q_len][kv_len] receives acc_j for every
 *   visible pair, debug_p (optional) uint8 the same shape receives the P code of every
 *   visible pair (e4m3 bits for FP8, the int8 code for INT8); other entries untouched.
 * Requirements: capacity >= kv_len rounded up to 64; q_heads % kv_heads == 0;
 *   kv_len >= 1; q_len >= 0 (0 = no-op); causal requires q_offset + q_len <= kv_len.
 * workspace: attn_q_prefill_workspace_size bytes (may be 0, then NULL is allowed): the
 *   per-tensor or per-block Q scales (TENSOR, BLOCK); contents need not be initialised.
 */
typedef struct {
  int32_t batch, q_heads, kv_heads, head_dim;
  int32_t q_len, kv_len, q_offset, causal;
  float sm_scale;
  const void *q;
  int32_t q_gran;                 /* TOKEN | BLOCK | TENSOR  */
  const int8_t *k_codes;
  const void *k_scales;
  int32_t k_gran;                 /* CHANNEL | TENSOR | TOKEN | BLOCK */
  const uint8_t *v_op;
  const float *v_scales;          /* V CHANNEL: fp32 [B][Hkv][d] */
  int32_t v_gran;                 /* CHANNEL | TOKEN */
  const float *v_scale_max;       /* V TOKEN: the cache header V_max, fp32 [B][Hkv] */
  int32_t pv_mode;                /* attn_q_pv_mode */
  int32_t capacity;
  void *out;
  int32_t out_dtype;              /* attn_q_out_dtype */
  float *lse;                     /* optional: fp32 [B][Hq][q_len] */
  int32_t *debug_s;
  uint8_t *debug_p;               /* optional: P codes, uint8 [B][Hq][q_len][kv_len] */
  void *workspace;
  size_t workspace_bytes;
} attn_q_prefill_args;

/* ------------------------------------------------------------------------ */
/* attn_q_decode: one query token per head against the int8 KV cache
 * (memory-bound: the cache is streamed once, each 16-byte load serving every
 * query head of its kv-head).
 *   q' = fp32(q) * s_K[c] (K CHANNEL) or fp32(q); s_Q = fp32(amax(q')/127) per head;
 *   q_code = clamp(rint(q'/s_Q)); acc_n = sum_c q_code_c * k_code_{n,c} (exact int32);
 *   s_n = fp32(c_n * acc_n), c_n = fp32(fp32(s_Q * kconst) * s_K[n]) (K TOKEN; K BLOCK: the
 *   scale of n's 64-key block) or fp32(s_Q * kconst) (K CHANNEL); p_n = 2^(s_n - max) in fp32 (max over a 64-key group);
 *   out = sum_n p_n * s_V * v_code_n / sum_n p_n, with the weights w_n = p_n (V CHANNEL) or
 *   p_n * s_V[n] (V TOKEN) multiplied by a power of two that puts the group's largest in
 *   [1, 2) and rounded to fp16, the products w_n * v_code_n exact and summed in fp32; each
 *   split of 512 keys computes its own max, sums and weighted V sum, and a second small
 *   kernel merges the splits (log-sum-exp).  Max relative error against the fp64 sum of the
 *   fp32 weights: a few 1e-5 on LLM-like caches, within 1e-3 in every tested case.
 * Ragged batch: with kv_lens (device int32 [B], optional) batch row b attends over its first
 *   kv_lens[b] keys (values are clamped to [1, kv_len]); kv_len is then the largest length,
 *   which sizes the launch and the workspace.  Splits past a row's length exit at once.
 * Buffers: q fp16 [B][Hq][d]; k_codes/v_codes int8 [B][Hkv][capacity][d]; k_scales
 *   TOKEN fp16 [B][Hkv][capacity], CHANNEL fp32 [B][Hkv][d] or BLOCK fp32 [B][Hkv][capacity/64]
 *   (capacity % 64 == 0); v_scales TOKEN or CHANNEL likewise;
 *   out [B][Hq][d]; debug_qk (optional) int32 [B][Hq][kv_len] (row stride kv_len).  capacity % 8 == 0;
 *   per-token scale arrays 16-byte aligned (they are read in groups of 8 keys; entries
 *   of keys >= kv_len may hold anything).
 * workspace: attn_q_decode_workspace_size bytes of per-split partials; contents need
 *   not be initialised.  Calls that overlap in time must not share it.
 */
typedef struct {
  int32_t batch, q_heads, kv_heads, head_dim, kv_len, capacity;
  const int32_t *kv_lens;         /* optional, device int32 [B]: keys of each batch row */
  float sm_scale;
  const void *q;
  const int8_t *k_codes;
  const void *k_scales;
  int32_t k_gran;                 /* TOKEN | CHANNEL | BLOCK */
  const int8_t *v_codes;
  const void *v_scales;
  int32_t v_gran;                 /* TOKEN | CHANNEL */
  void *out;
  int32_t out_dtype;
  int32_t *debug_qk;
  void *workspace;
  size_t workspace_bytes;
} attn_q_decode_args;

/* ------------------------------------------------------------------------ */
/* attn_q_decode_noalloc: attn_q_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid hipMalloc).  The same
 * kernels and the same result bits as attn_q_decode; the split partials go to a static
 * scratch array of the library (8 MiB per GPU, held until the process ends) instead of the
 * caller's workspace.  The workspace fields of `a` are ignored.  Nothing is allocated: no
 * hipMalloc, hipFree or allocating library call, on any call.
 * Limit: decode_workspace_size(a) must not exceed 8 MiB (batch * q_heads * ceil(kv_len /
 *   512) * (4 * head_dim + 8) bytes, rounded up to 256 twice) -- else ATTN_Q_E_SCRATCH and
 *   nothing is launched.  Every call on one GPU shares that GPU's array: calls that overlap
 *   in time on one GPU (different streams, or host threads) race and must not be issued;
 *   calls ordered on one stream are safe.  Nothing in the array needs to start at zero.
 */
int attn_q_decode_noalloc(const attn_q_decode_args *a, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* attn_q_decode_append: the decode step of a growing cache in one launch -- the new token's
 * K and V appended with the running K mean of the cache header (as attn_q_kv_append_i8 with
 * new_tokens = 1), then attn_q_decode with the new token as the last key.  The workgroup of
 * the decode that holds that key computes its row, writes it to the cache and the header,
 * and uses it at once; the result is bit for bit that of the two calls in sequence (cache
 * rows, scales, header, mean and output).  It saves the append's launch (the decode step of
 * "int8 Flash Attention on RDNA4", section "K's outliers, and the subtraction softmax does
 * not notice": the key arrives, is shifted by the lagging mean, and is attended at once).
 * Requirements: both argument blocks valid on their own; app->new_tokens == 1,
 *   app->seq_len == dec->kv_len - 1; the same batch, kv_heads, head_dim and capacity; the
 *   same cache buffers (k_codes, v_codes, k_scales, v_scales); dec->k_gran and dec->v_gran
 *   TOKEN; dec->kv_lens NULL.  app->workspace is not used.  Errors as for the two calls; nothing is launched
 *   on an error.
 */
int attn_q_decode_append(const attn_q_decode_args *dec, const attn_q_kv_append_args *app, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* attn_q_short_fused: quantized attention for short sequences in one pass over HBM, one
 * workgroup per (batch, head), for the vision shapes of "QFlash: Bridging Quantization and
 * Memory Efficiency in Vision Transformer Attention" (Table 1: ViT/DeiT heads of 197
 * tokens with d = 64, Swin windows of 49 tokens with d = 32).  The head's quantization
 * runs inside the kernel, so fp16 Q, K, V are read once and O written once.
 *
 * Per head (b, h), all N keys visible (non-causal):
 *   K: mu_c = fp32(S_c / (N * 2^24)) from the exact int64 sum S_c of k * 2^24; x = fp32(k) - mu;
 *      s_K[c] = fp32(max_n |x| / 127); k_code = clamp(rint(x / s_K[c]))   (per channel)
 *   V: s_V[c] = fp32(max_n |v| / 127); v_code likewise; operand e4m3(fp32(v_code))
 *   Q: q' = fp32(q) * s_K[c]; s_Q = fp32(max_c |q'| / 127) per row; q_code = clamp(rint(q'/s_Q))
 *   acc_j = sum_c q_code_c * k_code_{j,c} (exact int32); c = fp32(s_Q * kconst);
 *   m = max_j fp32(c * acc_j) over ALL keys (one key block: the row max is exact, nothing
 *   is rescaled); p_j, P_j, l and out exactly as attn_q_prefill with one key stream and
 *   one tile spanning the head: p_j = exp2(fp32(c * acc_j - fp32(m - log2 448))) (one rounding),
 *   P_j = e4m3(p_j), l = sum_j dec(P_j), out_c = (sum_j dec(P_j) * dec(v_op_jc)) * s_V[c] / l.
 *   These are the granularities of kv_quantize_i8 with K and V CHANNEL and of attn_q_prefill
 *   with q_gran TOKEN, taken per head.  The divisions are IEEE fp32 (fp64 for mu).
 * Buffers: q, k, v fp16 [B][H][seq_len][d]; out [B][H][seq_len][d] fp16 or fp32; debug_s
 *   (optional, NULL = off) int32 [B][H][seq_len][seq_len] receives acc_j for every pair.
 * Requirements: head_dim 32 or 64; 1 <= seq_len <= 256; 16-byte aligned q, k, v, out.
 *   No workspace.
 */
typedef struct {
  int32_t batch, heads, seq_len, head_dim;
  float sm_scale;                 /* <= 0: 1/sqrt(head_dim) */
  const void *q, *k, *v;
  void *out;
  int32_t out_dtype;              /* attn_q_out_dtype */
  int32_t *debug_s;
} attn_q_short_args;

/* ------------------------------------------------------------------------ */
/* Q and K below 8 bits: MX operands on the matrix core's fp6 / fp4 types.
 *
 * "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8" ends on the question
 * whether Q and K survive four bits (an accuracy question to ask of the grid before the
 * hardware).  gfx950 has no int4 matrix-core instruction; its 64-deep f8f6f4 MFMA takes
 * fp6 (E2M3) and fp4 (E2M1) operands with one E8M0 scale per lane, and each lane feeds one
 * block of 32 consecutive channels: the block of the OCP MX formats (Microscaling Formats
 * v1.0).  These calls put Q and K in those formats; softmax, P and PV are attn_q_prefill's.
 *
 * Encoding of a row, per block of 32 consecutive channels with largest magnitude amax:
 *   X = 2^e, e = floor(log2 amax) - 2 (amax = 0: e = 0), stored as the E8M0 byte 127 + e;
 *   element x / X (exact) rounded to the nearest value of the element grid, ties to the even
 *   code, magnitudes above the largest (6 for E2M1, 7.5 for E2M3) saturating; the code is
 *   sign | exponent field (bias 1, 0 = subnormal) | mantissa, with the sign bit (bit 3 of an
 *   E2M1 code, bit 5 of an E2M3 code) set for negative x of nonzero magnitude (a zero element
 *   is +0).  Packed codes: a row of d channels is d * bits / 8 bytes, element c at bits
 *   [bits*c, bits*c + bits) of the row read as a little-endian bit string.
 */
typedef enum {
  ATTN_Q_MX_FP6 = 2,   /* E2M3 elements, 6-bit codes (the MFMA's fp6 operand type) */
  ATTN_Q_MX_FP4 = 4    /* E2M1 elements, 4-bit codes (the MFMA's fp4 operand type) */
} attn_q_mx_format;

/* attn_q_k_quantize_mx: K rows shifted by the cache's per-channel mean and MX-encoded:
 *   x = fp32(k) - k_mean[c] (fp32, the shift of kv_quantize_i8's K codes), encoded as above.
 * Buffers: k fp16 [B][Hkv][seq_len][d]; k_mean fp32 [B][Hkv][d] (kv_quantize_i8's k_mean, or
 *   zeros for no shift); k_mx uint8 [B][Hkv][capacity][d * bits / 8]; k_mx_scales uint8
 *   [B][Hkv][capacity][d / 32] (E8M0 bytes); rows >= seq_len untouched.  k_mx 16-byte aligned.
 * Requirements: head_dim 64 or 128; 1 <= seq_len <= capacity; B * Hkv * seq_len * d / 32 <
 *   2^31.  No workspace.
 */
typedef struct {
  int32_t batch, kv_heads, seq_len, head_dim, capacity;
  int32_t fmt;                    /* attn_q_mx_format */
  const void *k;
  const float *k_mean;
  void *k_mx, *k_mx_scales;
} attn_q_k_mx_args;

/* attn_q_prefill_mx: attn_q_prefill with Q and K as MX operands.
 * Row (b, h, i) sees the keys attn_q_prefill's row sees.  q is MX-encoded per row (no shift)
 *   in q_fmt inside the kernel; K is attn_q_k_quantize_mx's, in k_fmt.
 *   s_j = sum over the row's blocks of X_q * X_k * (sum over the block of the products of the
 *     element values), on the scaled 64-deep MFMA with fp32 accumulation (each block's sum
 *     is exact; blocks of different scales are added in the matrix core's order);
 *   c = kconst (the block scales carry the magnitudes), kconst as attn_q_prefill's.
 *   Per key stream (ATTN_Q_KEY_STREAMS, merged as attn_q_prefill's), for each of its 64-key
 *   tiles in ascending order,
 *     m = max(m, max_j fp32(c * s_j)); mL = fp32(m - log2(448));
 *     p_j = exp2(fp32(c * s_j - mL)) (one rounding); P_j = e4m3(p_j);
 *     l = alpha*l + sum dec(P_j); O = alpha*O + sum_j dec(P_j) * vop_j, alpha = exp2(m_old - m);
 *   streams merged; out_c = O_c * s_V[c] / l.
 * V: per-channel, the e4m3 operand v_op (v_op_format ATTN_Q_PV_FP8) and v_scales of
 *   kv_quantize_i8.
 * Buffers: q fp16 [B][Hq][q_len][d]; k_mx, k_mx_scales as attn_q_k_quantize_mx writes them
 *   (capacity rows); v_op uint8 [B][Hkv][capacity/64][d][64]; v_scales fp32 [B][Hkv][d];
 *   out [B][Hq][q_len][d] fp16 or fp32; debug_s (optional, NULL = off) fp32
 *   [B][Hq][q_len][kv_len] receives s_j of every visible pair, other entries untouched.
 * Requirements: head_dim 64 or 128; q_heads % kv_heads == 0; kv_len >= 1; capacity a
 *   multiple of 64 and >= kv_len; q_len >= 0 (0 = no-op); causal requires q_offset + q_len
 *   <= kv_len; ceil(q_len / 128) * batch * q_heads < 2^31; q, k_mx, v_scales, out 16-byte aligned, v_op
 *   32-byte aligned.  No workspace.
 */
typedef struct {
  int32_t batch, q_heads, kv_heads, head_dim;
  int32_t q_len, kv_len, q_offset, causal;
  float sm_scale;                 /* <= 0: 1/sqrt(head_dim) */
  const void *q;
  int32_t q_fmt;                  /* attn_q_mx_format */
  const void *k_mx, *k_mx_scales;
  int32_t k_fmt;                  /* attn_q_mx_format */
  int32_t capacity;
  const void *v_op;
  const float *v_scales;
  void *out;
  int32_t out_dtype;              /* attn_q_out_dtype */
  float *debug_s;
} attn_q_prefill_mx_args;

int attn_q_k_quantize_mx(const attn_q_k_mx_args *a, void *hip_stream);
int attn_q_prefill_mx(const attn_q_prefill_mx_args *a, void *hip_stream);

int kv_quantize_i8(const attn_q_kvq_args *a, void *hip_stream);
int attn_q_prefill(const attn_q_prefill_args *a, void *hip_stream);
int attn_q_decode(const attn_q_decode_args *a, void *hip_stream);
int attn_q_kv_append_i8(const attn_q_kv_append_args *a, void *hip_stream);
int attn_q_short_fused(const attn_q_short_args *a, void *hip_stream);

/* Workspace sizes in bytes for the given arguments (only sizes and enums are
 * read); 0 if the arguments are invalid. */
size_t kv_quantize_i8_workspace_size(const attn_q_kvq_args *a);
size_t attn_q_prefill_workspace_size(const attn_q_prefill_args *a);
size_t attn_q_decode_workspace_size(const attn_q_decode_args *a);
size_t attn_q_kv_append_i8_workspace_size(const attn_q_kv_append_args *a);

/* Static string for a status code; never NULL. */
const char *attn_q_status_string(int status);
/* ATTN_Q_ABI_VERSION of the loaded library. */
int attn_q_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_Q_H */

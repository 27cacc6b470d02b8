// Host side of the C ABI declared in include/attn_q.h: argument validation (before any
// HIP call), device check, workspace sizing and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "common.h"

namespace {

constexpr int kMaxDevices = 64;
// per-device architecture check: 0 = unknown, 1 = gfx950, 2 = other / failed
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_Q_E_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    st = 2;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
      st = 1;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? ATTN_Q_OK : ATTN_Q_E_DEVICE;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }

int validate_kvq(const attn_q_kvq_args *a) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->kv_heads < 1 || a->seq_len < 1 || a->capacity < a->seq_len)
    return ATTN_Q_E_SHAPE;
  if (!head_dim_ok(a->head_dim)) return ATTN_Q_E_UNSUPPORTED;
  if ((int64_t)a->batch * a->kv_heads * a->capacity * a->head_dim > ((int64_t)1 << 40)) return ATTN_Q_E_SHAPE;
  if ((int64_t)a->batch * a->kv_heads > 65535) return ATTN_Q_E_SHAPE;   // grid y
  if (a->k_gran != ATTN_Q_GRAN_TOKEN && a->k_gran != ATTN_Q_GRAN_CHANNEL && a->k_gran != ATTN_Q_GRAN_TENSOR &&
      a->k_gran != ATTN_Q_GRAN_BLOCK)
    return ATTN_Q_E_UNSUPPORTED;
  if (a->k_gran == ATTN_Q_GRAN_BLOCK && a->capacity % ATTN_Q_BLOCK) return ATTN_Q_E_SHAPE;
  if (a->v_gran != ATTN_Q_GRAN_TOKEN && a->v_gran != ATTN_Q_GRAN_CHANNEL) return ATTN_Q_E_UNSUPPORTED;
  if (!a->k || !a->v || !a->k_codes || !a->k_scales || !a->v_scales || !a->k_mean) return ATTN_Q_E_NULL;
  // the V codes may be left out of a cache that serves only the prefill (its per-channel e4m3
  // operand is written from the quantized values directly)
  if (!a->v_codes && !(a->v_op && a->v_gran == ATTN_Q_GRAN_CHANNEL)) return ATTN_Q_E_NULL;
  if (a->v_op) {
    if (a->capacity % ATTN_Q_KEY_TILE) return ATTN_Q_E_SHAPE;
    if (a->v_op_format != ATTN_Q_PV_FP8 && a->v_op_format != ATTN_Q_PV_INT8) return ATTN_Q_E_UNSUPPORTED;
    // a per-token operand is e4m3 (it carries s_V[n] * c_V) and writes the V_max header
    if (a->v_gran == ATTN_Q_GRAN_TOKEN && a->v_op_format != ATTN_Q_PV_FP8) return ATTN_Q_E_UNSUPPORTED;
    if (a->v_gran == ATTN_Q_GRAN_TOKEN && !a->v_scale_max) return ATTN_Q_E_NULL;
    if (!aligned(a->v_op, 16) || !aligned(a->v_scale_max, 4)) return ATTN_Q_E_ALIGN;
  }
  if (!aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->k_codes, 16) || !aligned(a->v_codes, 16) ||
      !aligned(a->k_scales, 4) || !aligned(a->v_scales, 4) || !aligned(a->k_mean, 4) || !aligned(a->k_sum, 8))
    return ATTN_Q_E_ALIGN;
  const size_t need = kvq_workspace_bytes(a->batch, a->kv_heads, a->head_dim);
  if (!a->workspace || a->workspace_bytes < need) return ATTN_Q_E_WORKSPACE;
  if (!aligned(a->workspace, 16)) return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

int validate_vop(const attn_q_vop_args *a) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->kv_heads < 1 || a->n_keys < 1 || a->capacity < a->n_keys) return ATTN_Q_E_SHAPE;
  if (a->capacity % ATTN_Q_KEY_TILE) return ATTN_Q_E_SHAPE;
  if (!head_dim_ok(a->head_dim)) return ATTN_Q_E_UNSUPPORTED;
  if ((int64_t)a->batch * a->kv_heads > 65535) return ATTN_Q_E_SHAPE;   // grid y
  if (a->v_gran != ATTN_Q_GRAN_TOKEN && a->v_gran != ATTN_Q_GRAN_CHANNEL) return ATTN_Q_E_UNSUPPORTED;
  if (a->v_op_format != ATTN_Q_PV_FP8 && a->v_op_format != ATTN_Q_PV_INT8) return ATTN_Q_E_UNSUPPORTED;
  if (a->v_gran == ATTN_Q_GRAN_TOKEN && a->v_op_format != ATTN_Q_PV_FP8) return ATTN_Q_E_UNSUPPORTED;
  if (!a->v_codes || !a->v_op || (a->v_gran == ATTN_Q_GRAN_TOKEN && (!a->v_scales || !a->v_scale_max)))
    return ATTN_Q_E_NULL;
  if (!aligned(a->v_codes, 16) || !aligned(a->v_op, 16) || !aligned(a->v_scales, 2) || !aligned(a->v_scale_max, 4))
    return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

int validate_prefill(const attn_q_prefill_args *a) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->q_heads < 1 || a->kv_heads < 1 || a->q_heads % a->kv_heads) return ATTN_Q_E_SHAPE;
  if (!head_dim_ok(a->head_dim)) return ATTN_Q_E_UNSUPPORTED;
  if (a->q_len < 0 || a->kv_len < 1 || a->q_offset < 0) return ATTN_Q_E_SHAPE;
  const int64_t cap_need = ((int64_t)a->kv_len + ATTN_Q_KEY_TILE - 1) / ATTN_Q_KEY_TILE * ATTN_Q_KEY_TILE;
  if (a->capacity < cap_need || a->capacity % ATTN_Q_KEY_TILE) return ATTN_Q_E_SHAPE;
  if (a->causal && (int64_t)a->q_offset + a->q_len > a->kv_len) return ATTN_Q_E_SHAPE;
  if ((int64_t)a->q_heads / a->kv_heads * a->q_len > ((int64_t)1 << 30)) return ATTN_Q_E_SHAPE;
  if (a->q_gran != ATTN_Q_GRAN_TOKEN && a->q_gran != ATTN_Q_GRAN_TENSOR && a->q_gran != ATTN_Q_GRAN_BLOCK)
    return ATTN_Q_E_UNSUPPORTED;
  if (a->k_gran != ATTN_Q_GRAN_CHANNEL && a->k_gran != ATTN_Q_GRAN_TENSOR && a->k_gran != ATTN_Q_GRAN_TOKEN &&
      a->k_gran != ATTN_Q_GRAN_BLOCK)
    return ATTN_Q_E_UNSUPPORTED;
  if (a->pv_mode != ATTN_Q_PV_FP8 && a->pv_mode != ATTN_Q_PV_INT8 && a->pv_mode != ATTN_Q_PV_SPLIT24)
    return ATTN_Q_E_UNSUPPORTED;
  if (a->pv_mode == ATTN_Q_PV_SPLIT24 &&
      (a->q_gran != ATTN_Q_GRAN_TOKEN || a->debug_s || a->k_gran == ATTN_Q_GRAN_TOKEN ||
       a->k_gran == ATTN_Q_GRAN_BLOCK))
    return ATTN_Q_E_UNSUPPORTED;
  if (a->out_dtype != ATTN_Q_OUT_F16 && a->out_dtype != ATTN_Q_OUT_F32) return ATTN_Q_E_UNSUPPORTED;
  if (a->v_gran != ATTN_Q_GRAN_CHANNEL && a->v_gran != ATTN_Q_GRAN_TOKEN) return ATTN_Q_E_UNSUPPORTED;
  // per-token V: the e4m3 operand carries s_V[n] * c_V (the int8 variants keep bare codes)
  if (a->v_gran == ATTN_Q_GRAN_TOKEN && a->pv_mode != ATTN_Q_PV_FP8) return ATTN_Q_E_UNSUPPORTED;
  if (a->pv_mode == ATTN_Q_PV_SPLIT24 && (a->lse || a->debug_p)) return ATTN_Q_E_UNSUPPORTED;
  if (a->q_len == 0) return ATTN_Q_OK;  // nothing to read or write
  if (!a->q || !a->k_codes || !a->k_scales || !a->v_op || !a->out) return ATTN_Q_E_NULL;
  if (a->v_gran == ATTN_Q_GRAN_CHANNEL ? !a->v_scales : !a->v_scale_max) return ATTN_Q_E_NULL;
  if (!aligned(a->q, 16) || !aligned(a->k_codes, 16) || !aligned(a->v_op, 32) || !aligned(a->k_scales, 16) ||
      !aligned(a->v_scales, 16) || !aligned(a->v_scale_max, 4) || !aligned(a->out, 16) ||
      !aligned(a->debug_s, 4) || !aligned(a->lse, 4))
    return ATTN_Q_E_ALIGN;
  const size_t need = prefill_workspace_bytes(a->q_gran, a->batch, a->q_heads, a->q_len);
  if (need && (!a->workspace || a->workspace_bytes < need)) return ATTN_Q_E_WORKSPACE;
  if (need && !aligned(a->workspace, 16)) return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

int validate_decode(const attn_q_decode_args *a, bool own_workspace = true) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->q_heads < 1 || a->kv_heads < 1 || a->q_heads % a->kv_heads) return ATTN_Q_E_SHAPE;
  const int G = a->q_heads / a->kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ATTN_Q_E_UNSUPPORTED;
  if (!head_dim_ok(a->head_dim)) return ATTN_Q_E_UNSUPPORTED;
  if (a->kv_len < 1 || a->capacity < a->kv_len || a->capacity % 8) return ATTN_Q_E_SHAPE;
  if ((int64_t)a->batch * a->kv_heads > 65535) return ATTN_Q_E_SHAPE;   // grid y, arrival counters
  if (a->k_gran != ATTN_Q_GRAN_TOKEN && a->k_gran != ATTN_Q_GRAN_CHANNEL && a->k_gran != ATTN_Q_GRAN_BLOCK)
    return ATTN_Q_E_UNSUPPORTED;
  if (a->k_gran == ATTN_Q_GRAN_BLOCK && a->capacity % ATTN_Q_BLOCK) return ATTN_Q_E_SHAPE;
  if (a->v_gran != ATTN_Q_GRAN_TOKEN && a->v_gran != ATTN_Q_GRAN_CHANNEL) return ATTN_Q_E_UNSUPPORTED;
  if (a->out_dtype != ATTN_Q_OUT_F16 && a->out_dtype != ATTN_Q_OUT_F32) return ATTN_Q_E_UNSUPPORTED;
  if (!a->q || !a->k_codes || !a->k_scales || !a->v_codes || !a->v_scales || !a->out) return ATTN_Q_E_NULL;
  // per-token scales are read as 16-byte groups of 8 keys
  const size_t ks_align = a->k_gran == ATTN_Q_GRAN_TOKEN ? 16 : 4;
  const size_t vs_align = a->v_gran == ATTN_Q_GRAN_TOKEN ? 16 : 4;
  if (!aligned(a->q, 4) || !aligned(a->k_codes, 16) || !aligned(a->v_codes, 16) || !aligned(a->k_scales, ks_align) ||
      !aligned(a->v_scales, vs_align) || !aligned(a->out, 4) || !aligned(a->debug_qk, 4) || !aligned(a->kv_lens, 4))
    return ATTN_Q_E_ALIGN;
  const size_t need = decode_workspace_bytes(a->batch, a->q_heads, a->kv_heads, a->head_dim, a->kv_len);
  if (!own_workspace) return need > decode_scratch_bytes() ? ATTN_Q_E_SCRATCH : ATTN_Q_OK;
  if (!a->workspace || a->workspace_bytes < need) return ATTN_Q_E_WORKSPACE;
  if (!aligned(a->workspace, 256)) return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

int validate_append(const attn_q_kv_append_args *a) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->kv_heads < 1 || a->capacity < 1 || a->seq_len < 0 || a->new_tokens < 0)
    return ATTN_Q_E_SHAPE;
  if (!head_dim_ok(a->head_dim)) return ATTN_Q_E_UNSUPPORTED;
  if ((int64_t)a->seq_len + a->new_tokens > a->capacity) return ATTN_Q_E_SHAPE;
  if ((int64_t)a->batch * a->kv_heads * a->capacity * a->head_dim > ((int64_t)1 << 40)) return ATTN_Q_E_SHAPE;
  const int64_t chunks = ((int64_t)a->new_tokens + 63) / 64;
  if ((int64_t)a->batch * a->kv_heads * (chunks > 0 ? chunks : 1) > INT32_MAX) return ATTN_Q_E_SHAPE;  // grid x
  if (a->new_tokens == 0) return ATTN_Q_OK;  // nothing to read or write
  if (!a->k || !a->v || !a->k_sum || !a->k_codes || !a->v_codes || !a->k_scales || !a->v_scales)
    return ATTN_Q_E_NULL;
  if (!aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->k_codes, 16) || !aligned(a->v_codes, 16) ||
      !aligned(a->k_sum, 8) || !aligned(a->k_scales, 2) || !aligned(a->v_scales, 2) || !aligned(a->k_mean, 4))
    return ATTN_Q_E_ALIGN;
  const size_t need = kv_append_workspace_bytes(a->batch, a->kv_heads, a->head_dim, a->new_tokens);
  if (need && (!a->workspace || a->workspace_bytes < need)) return ATTN_Q_E_WORKSPACE;
  if (need && !aligned(a->workspace, 16)) return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

int validate_short(const attn_q_short_args *a) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->heads < 1 || a->seq_len < 1) return ATTN_Q_E_SHAPE;
  if (a->head_dim != 32 && a->head_dim != 64) return ATTN_Q_E_UNSUPPORTED;
  if (a->seq_len > 256) return ATTN_Q_E_UNSUPPORTED;   // one workgroup holds the head
  if ((int64_t)a->batch * a->heads > INT32_MAX) return ATTN_Q_E_SHAPE;   // grid x
  if (a->out_dtype != ATTN_Q_OUT_F16 && a->out_dtype != ATTN_Q_OUT_F32) return ATTN_Q_E_UNSUPPORTED;
  if (!a->q || !a->k || !a->v || !a->out) return ATTN_Q_E_NULL;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->out, 16) ||
      !aligned(a->debug_s, 4))
    return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

bool mx_fmt_ok(int f) { return f == ATTN_Q_MX_FP4 || f == ATTN_Q_MX_FP6; }

int validate_k_mx(const attn_q_k_mx_args *a) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->kv_heads < 1 || a->seq_len < 1 || a->capacity < a->seq_len) return ATTN_Q_E_SHAPE;
  if (!head_dim_ok(a->head_dim) || !mx_fmt_ok(a->fmt)) return ATTN_Q_E_UNSUPPORTED;
  if ((int64_t)a->batch * a->kv_heads * a->seq_len * (a->head_dim / 32) >= ((int64_t)1 << 31)) return ATTN_Q_E_SHAPE;
  if (!a->k || !a->k_mean || !a->k_mx || !a->k_mx_scales) return ATTN_Q_E_NULL;
  if (!aligned(a->k, 16) || !aligned(a->k_mean, 4) || !aligned(a->k_mx, 16)) return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

int validate_prefill_mx(const attn_q_prefill_mx_args *a) {
  if (!a) return ATTN_Q_E_NULL;
  if (a->batch < 1 || a->q_heads < 1 || a->kv_heads < 1 || a->q_heads % a->kv_heads) return ATTN_Q_E_SHAPE;
  if (!head_dim_ok(a->head_dim) || !mx_fmt_ok(a->q_fmt) || !mx_fmt_ok(a->k_fmt)) return ATTN_Q_E_UNSUPPORTED;
  if (a->q_len < 0 || a->kv_len < 1 || a->q_offset < 0) return ATTN_Q_E_SHAPE;
  if (a->capacity < a->kv_len || a->capacity % ATTN_Q_KEY_TILE) return ATTN_Q_E_SHAPE;
  if (a->causal && (int64_t)a->q_offset + a->q_len > a->kv_len) return ATTN_Q_E_SHAPE;
  if (((int64_t)a->q_len + 127) / 128 * a->batch * a->q_heads >= ((int64_t)1 << 31)) return ATTN_Q_E_SHAPE;  // grid
  if (a->out_dtype != ATTN_Q_OUT_F16 && a->out_dtype != ATTN_Q_OUT_F32) return ATTN_Q_E_UNSUPPORTED;
  if (a->q_len == 0) return ATTN_Q_OK;
  if (!a->q || !a->k_mx || !a->k_mx_scales || !a->v_op || !a->v_scales || !a->out) return ATTN_Q_E_NULL;
  if (!aligned(a->q, 16) || !aligned(a->k_mx, 16) || !aligned(a->k_mx_scales, 4) || !aligned(a->v_op, 32) ||
      !aligned(a->v_scales, 16) || !aligned(a->out, 16) || !aligned(a->debug_s, 4))
    return ATTN_Q_E_ALIGN;
  return ATTN_Q_OK;
}

}  // namespace

extern "C" {

int attn_q_version(void) { return ATTN_Q_ABI_VERSION; }

const char *attn_q_status_string(int status) {
  switch (status) {
    case ATTN_Q_OK: return "ok";
    case ATTN_Q_E_NULL: return "a required pointer is NULL";
    case ATTN_Q_E_SHAPE: return "inconsistent or out-of-range sizes";
    case ATTN_Q_E_UNSUPPORTED: return "unsupported granularity, mode, dtype or head_dim";
    case ATTN_Q_E_ALIGN: return "misaligned pointer";
    case ATTN_Q_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_Q_E_DEVICE: return "current device is not gfx950 or the HIP query failed";
    case ATTN_Q_E_LAUNCH: return "kernel launch failed";
    case ATTN_Q_E_SCRATCH: return "the call needs more than the library's static scratch (attn_q_decode_noalloc)";
    default: return "unknown status";
  }
}

size_t kv_quantize_i8_workspace_size(const attn_q_kvq_args *a) {
  if (!a || a->batch < 1 || a->kv_heads < 1 || !head_dim_ok(a->head_dim)) return 0;
  return kvq_workspace_bytes(a->batch, a->kv_heads, a->head_dim);
}

size_t attn_q_prefill_workspace_size(const attn_q_prefill_args *a) {
  if (!a || a->batch < 1 || a->q_heads < 1 || a->q_len < 0) return 0;
  return prefill_workspace_bytes(a->q_gran, a->batch, a->q_heads, a->q_len);
}

size_t attn_q_decode_workspace_size(const attn_q_decode_args *a) {
  if (!a || a->batch < 1 || a->kv_heads < 1 || a->q_heads < 1 || a->q_heads % a->kv_heads ||
      !head_dim_ok(a->head_dim) || a->kv_len < 1)
    return 0;
  return decode_workspace_bytes(a->batch, a->q_heads, a->kv_heads, a->head_dim, a->kv_len);
}

size_t attn_q_kv_append_i8_workspace_size(const attn_q_kv_append_args *a) {
  if (!a || a->batch < 1 || a->kv_heads < 1 || !head_dim_ok(a->head_dim) || a->new_tokens < 0) return 0;
  return kv_append_workspace_bytes(a->batch, a->kv_heads, a->head_dim, a->new_tokens);
}

int kv_quantize_i8(const attn_q_kvq_args *a, void *hip_stream) {
  int st = validate_kvq(a);
  if (st != ATTN_Q_OK) return st;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  KvqLaunch l;
  l.B = a->batch; l.H = a->kv_heads; l.N = a->seq_len; l.D = a->head_dim; l.cap = a->capacity;
  l.k = (const uint16_t *)a->k; l.v = (const uint16_t *)a->v;
  l.subtract_mean = a->subtract_k_mean != 0; l.k_gran = a->k_gran; l.v_gran = a->v_gran;
  l.k_codes = a->k_codes; l.v_codes = a->v_codes; l.k_scales = a->k_scales; l.v_scales = a->v_scales;
  l.k_mean = a->k_mean; l.k_sum = a->k_sum; l.v_op = a->v_op; l.v_op_format = a->v_op_format;
  l.v_scale_max = a->v_scale_max; l.ws = a->workspace;
  return launch_kv_quantize(l, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_v_operand(const attn_q_vop_args *a, void *hip_stream) {
  int st = validate_vop(a);
  if (st != ATTN_Q_OK) return st;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  VopLaunch l;
  l.B = a->batch; l.H = a->kv_heads; l.D = a->head_dim; l.cap = a->capacity; l.n_keys = a->n_keys;
  l.v_codes = a->v_codes; l.v_scales = a->v_scales; l.v_gran = a->v_gran; l.fmt = a->v_op_format;
  l.v_op = a->v_op; l.v_scale_max = a->v_scale_max;
  return launch_v_operand(l, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_prefill(const attn_q_prefill_args *a, void *hip_stream) {
  int st = validate_prefill(a);
  if (st != ATTN_Q_OK) return st;
  if (a->q_len == 0) return ATTN_Q_OK;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  PrefillLaunch l;
  l.B = a->batch; l.Hq = a->q_heads; l.Hkv = a->kv_heads; l.D = a->head_dim;
  l.q_len = a->q_len; l.kv_len = a->kv_len; l.q_offset = a->q_offset; l.causal = a->causal != 0;
  l.cap = a->capacity; l.kconst = attnq::host_kconst(a->sm_scale, a->head_dim);
  l.q = (const uint16_t *)a->q; l.q_gran = a->q_gran; l.k_codes = a->k_codes; l.k_scales = a->k_scales;
  l.k_gran = a->k_gran; l.v_op = a->v_op; l.v_scales = a->v_scales; l.v_gran = a->v_gran;
  l.v_scale_max = a->v_scale_max; l.pv_mode = a->pv_mode;
  l.out = a->out; l.out_f32 = a->out_dtype == ATTN_Q_OUT_F32; l.lse = a->lse; l.debug_s = a->debug_s;
  l.debug_p = a->debug_p; l.ws = a->workspace;
  const hipError_t e = a->pv_mode == ATTN_Q_PV_SPLIT24 ? launch_prefill_split24(l, (hipStream_t)hip_stream)
                                                        : launch_prefill(l, (hipStream_t)hip_stream);
  return e == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

static DecodeLaunch decode_launch(const attn_q_decode_args *a) {
  DecodeLaunch l;
  l.B = a->batch; l.Hq = a->q_heads; l.Hkv = a->kv_heads; l.D = a->head_dim; l.kv_len = a->kv_len;
  l.cap = a->capacity; l.kconst = attnq::host_kconst(a->sm_scale, a->head_dim);
  l.q = (const uint16_t *)a->q; l.k_codes = a->k_codes; l.k_scales = a->k_scales;
  l.v_codes = a->v_codes; l.v_scales = a->v_scales; l.out = a->out;
  l.flags = (a->k_gran == ATTN_Q_GRAN_TOKEN ? kDecKTok : 0) | (a->v_gran == ATTN_Q_GRAN_TOKEN ? kDecVTok : 0) |
            (a->out_dtype == ATTN_Q_OUT_F32 ? kDecOutF32 : 0) | (a->k_gran == ATTN_Q_GRAN_BLOCK ? kDecKBlk : 0);
  l.debug_qk = a->debug_qk; l.ws = a->workspace; l.kv_lens = a->kv_lens;
  return l;
}

int attn_q_decode(const attn_q_decode_args *a, void *hip_stream) {
  int st = validate_decode(a);
  if (st != ATTN_Q_OK) return st;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  const DecodeLaunch l = decode_launch(a);
  return launch_decode(l, nullptr, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_decode_noalloc(const attn_q_decode_args *a, void *hip_stream) {
  int st = validate_decode(a, false);
  if (st != ATTN_Q_OK) return st;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  void *ws = nullptr;
  if (decode_scratch_ptr(&ws) != hipSuccess || !ws) return ATTN_Q_E_DEVICE;
  DecodeLaunch l = decode_launch(a);
  l.ws = ws;
  return launch_decode(l, nullptr, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_decode_append(const attn_q_decode_args *d, const attn_q_kv_append_args *a, void *hip_stream) {
  int st = validate_decode(d);
  if (st != ATTN_Q_OK) return st;
  if ((st = validate_append(a)) != ATTN_Q_OK) return st;
  // one new token, at the row the decode reads last, in the same cache (one length for all rows)
  if (a->new_tokens != 1 || a->seq_len != d->kv_len - 1 || d->kv_lens) return ATTN_Q_E_SHAPE;
  if (a->batch != d->batch || a->kv_heads != d->kv_heads || a->head_dim != d->head_dim ||
      a->capacity != d->capacity)
    return ATTN_Q_E_SHAPE;
  if (d->k_gran != ATTN_Q_GRAN_TOKEN || d->v_gran != ATTN_Q_GRAN_TOKEN) return ATTN_Q_E_UNSUPPORTED;
  if ((const void *)a->k_codes != (const void *)d->k_codes || (const void *)a->v_codes != (const void *)d->v_codes ||
      (const void *)a->k_scales != d->k_scales || (const void *)a->v_scales != d->v_scales)
    return ATTN_Q_E_SHAPE;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  const DecodeLaunch l = decode_launch(d);
  DecodeAppendLaunch ap;
  ap.k = (const uint16_t *)a->k; ap.v = (const uint16_t *)a->v;
  ap.k_sum = (long long *)a->k_sum; ap.k_mean = a->k_mean;
  ap.k_codes = a->k_codes; ap.v_codes = a->v_codes;
  ap.k_scales = (__half *)a->k_scales; ap.v_scales = (__half *)a->v_scales;
  return launch_decode(l, &ap, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_kv_append_i8(const attn_q_kv_append_args *a, void *hip_stream) {
  int st = validate_append(a);
  if (st != ATTN_Q_OK) return st;
  if (a->new_tokens == 0) return ATTN_Q_OK;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  KvAppendLaunch l;
  l.B = a->batch; l.H = a->kv_heads; l.D = a->head_dim; l.cap = a->capacity;
  l.n_before = a->seq_len; l.T = a->new_tokens;
  l.k = (const uint16_t *)a->k; l.v = (const uint16_t *)a->v; l.k_sum = a->k_sum;
  l.k_codes = a->k_codes; l.v_codes = a->v_codes;
  l.k_scales = (uint16_t *)a->k_scales; l.v_scales = (uint16_t *)a->v_scales;
  l.k_mean = a->k_mean; l.ws = a->workspace;
  return launch_kv_append(l, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_k_quantize_mx(const attn_q_k_mx_args *a, void *hip_stream) {
  int st = validate_k_mx(a);
  if (st != ATTN_Q_OK) return st;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  KMxLaunch l;
  l.BH = a->batch * a->kv_heads; l.N = a->seq_len; l.D = a->head_dim; l.cap = a->capacity; l.fmt = a->fmt;
  l.k = (const uint16_t *)a->k; l.k_mean = a->k_mean;
  l.k_mx = (uint8_t *)a->k_mx; l.k_sc = (uint8_t *)a->k_mx_scales;
  return launch_k_mx(l, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_prefill_mx(const attn_q_prefill_mx_args *a, void *hip_stream) {
  int st = validate_prefill_mx(a);
  if (st != ATTN_Q_OK) return st;
  if (a->q_len == 0) return ATTN_Q_OK;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  PrefillMxLaunch l;
  l.B = a->batch; l.Hq = a->q_heads; l.Hkv = a->kv_heads; l.D = a->head_dim;
  l.q_len = a->q_len; l.kv_len = a->kv_len; l.q_offset = a->q_offset; l.causal = a->causal != 0;
  l.cap = a->capacity; l.q_fmt = a->q_fmt; l.k_fmt = a->k_fmt; l.out_f32 = a->out_dtype == ATTN_Q_OUT_F32;
  l.kconst = attnq::host_kconst(a->sm_scale, a->head_dim);
  l.q = (const uint16_t *)a->q; l.k_mx = (const uint8_t *)a->k_mx; l.k_sc = (const uint8_t *)a->k_mx_scales;
  l.v_op = (const uint8_t *)a->v_op; l.v_scales = a->v_scales; l.out = a->out; l.debug_s = a->debug_s;
  return launch_prefill_mx(l, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

int attn_q_short_fused(const attn_q_short_args *a, void *hip_stream) {
  int st = validate_short(a);
  if (st != ATTN_Q_OK) return st;
  if ((st = check_device()) != ATTN_Q_OK) return st;
  ShortLaunch l;
  l.B = a->batch; l.H = a->heads; l.N = a->seq_len; l.D = a->head_dim;
  l.kconst = attnq::host_kconst(a->sm_scale, a->head_dim);
  l.q = (const uint16_t *)a->q; l.k = (const uint16_t *)a->k; l.v = (const uint16_t *)a->v;
  l.out = a->out; l.out_f32 = a->out_dtype == ATTN_Q_OUT_F32; l.debug_s = a->debug_s;
  return launch_short_fused(l, (hipStream_t)hip_stream) == hipSuccess ? ATTN_Q_OK : ATTN_Q_E_LAUNCH;
}

}  // extern "C"

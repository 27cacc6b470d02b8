"""CPU oracle for quantized flash attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``liboracle_attn.so`` (built from
``oracle_attn.cpp`` with g++; no code shared with the GPU library) through
ctypes and adds numpy-only diagnostics (``oracle.diagnostics``).

The functions here follow "int8 Flash Attention on RDNA4: QK Wants Integers, PV
Wants FP8" (the method) and the quantizer / integer-score equations (1)-(4) and
Algorithm 1 of "QFlash: Bridging Quantization and Memory Efficiency in Vision
Transformer Attention"; the C++ source cites the section behind each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_attn.cpp")
_LIB = os.path.join(_HERE, "liboracle_attn.so")

GRAN_TENSOR, GRAN_BLOCK, GRAN_TOKEN, GRAN_CHANNEL = 0, 1, 2, 3
BLOCK_N = 64   # tokens per BLOCK-granularity scale
PV_FP8, PV_INT8 = 0, 1
KEY_TILE = 64     # keys per online-softmax step emulated by default
KEY_STREAMS = 2   # interleaved online-softmax streams emulated by default


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.orc_e4m3_encode.argtypes = [P, P, i64]
        L.orc_e4m3_decode.argtypes = [P, P, i64]
        L.orc_half_to_double.argtypes = [P, P, i64]
        L.orc_float_to_half.argtypes = [P, P, i64]
        L.orc_quant_i8.argtypes = [P, f32, P, i64]
        L.orc_log2_448.restype = f32
        L.orc_kconst.argtypes = [f32, i32]
        L.orc_kconst.restype = f32
        L.orc_int_dots.argtypes = [P, P, P, i32, i32, i32]
        L.orc_int_dots.restype = i32
        L.orc_kv_quantize.argtypes = [i32, i32, i32, i32, i32, P, P, i32, i32, i32,
                                      P, P, P, P, P, P, i32, P, P]
        L.orc_v_operand.argtypes = [i32, i32, i32, i32, i32, P, P, i32, i32, P, P]
        L.orc_quantize_q.argtypes = [i32, i32, i32, i32, i32, P, P, i32, P, P]
        L.orc_kv_append.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.orc_prefill_emulate.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                          P, P, P, P, i32, P, P, i32, P, i32, P, i64, P, P, P, P, i32, P, P,
                                          P, P, P]
        L.orc_prefill_emulate.restype = i64
        L.orc_decode_emulate.argtypes = [i32, i32, i32, i32, i32, i32, f32, P, P, P, i32,
                                         P, P, i32, P, P]
        L.orc_attn_exact.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, f64,
                                     P, P, P, P, P, i64, P]
        L.orc_attn_dequant.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, f64,
                                       P, P, P, i32, P, P, P, i64, P]
        L.orc_attn_lowbit.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, f64, P, P, P, i32, i32, P, i64, P]
        L.orc_lowbit_element.argtypes = [P, i64, i32, P, P]
        L.orc_lowbit_row.argtypes = [P, i32, i32, P]
        L.orc_mx_quantize.argtypes = [P, i64, i32, i32, P, P, P]
        L.orc_mx_quantize.restype = i32
        L.orc_num_threads.restype = i32
        L.orc_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a: np.ndarray) -> np.ndarray:
    assert a.dtype == np.float16
    return np.ascontiguousarray(a).view(np.uint16)


# ------------------------------------------------------------------ codecs
def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode(_p(x), _p(out), x.size)
    return out


def e4m3_decode(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    out = np.empty(b.shape, np.float64)
    lib().orc_e4m3_decode(_p(b), _p(out), b.size)
    return out


def half_to_double(h: np.ndarray) -> np.ndarray:
    u = _u16(h)
    out = np.empty(u.shape, np.float64)
    lib().orc_half_to_double(_p(u), _p(out), u.size)
    return out


def float_to_half(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.uint16)
    lib().orc_float_to_half(_p(x), _p(out), x.size)
    return out.view(np.float16)


def quant_i8(x, s: float) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.int8)
    lib().orc_quant_i8(_p(x), float(s), _p(out), x.size)
    return out


def int_dots(a: np.ndarray, b: np.ndarray):
    """int8 [m][d] x int8 [n][d] -> (int32 [m][n], overflowed?)"""
    a = np.ascontiguousarray(a, dtype=np.int8)
    b = np.ascontiguousarray(b, dtype=np.int8)
    m, d = a.shape
    n = b.shape[0]
    acc = np.empty((m, n), np.int32)
    ov = lib().orc_int_dots(_p(a), _p(b), _p(acc), m, n, d)
    return acc, bool(ov)


def kconst(sm_scale: float, d: int) -> float:
    return float(lib().orc_kconst(sm_scale, d))


# ------------------------------------------------------------ quantizers
@dataclass
class KVCache:
    k_codes: np.ndarray
    v_codes: np.ndarray
    k_scales: np.ndarray      # fp32 [B][H][d] (CHANNEL) / fp16 [B][H][cap] (TOKEN) /
                              # fp32 [B][H][cap/64] (BLOCK) / fp32 [1]
    v_scales: np.ndarray
    k_mean: np.ndarray        # fp32 [B][H][d]
    v_op: Optional[np.ndarray]
    k_gran: int
    v_gran: int
    capacity: int
    seq_len: int
    v_scale_max: Optional[np.ndarray] = None   # fp32 [B][H]: header V_max of a per-token V operand


def kv_quantize(k: np.ndarray, v: np.ndarray, k_gran: int, v_gran: int,
                subtract_mean: bool = True, capacity: Optional[int] = None,
                v_op_format: Optional[int] = None,
                k_sum: Optional[np.ndarray] = None) -> KVCache:
    """k_sum (optional int64 [B][Hkv][d]) receives the exact header sum S of the keys,
    from which kv_append continues the running mean."""
    B, H, N, d = k.shape
    if k_sum is not None:
        assert k_sum.dtype == np.int64 and k_sum.shape == (B, H, d) and k_sum.flags.c_contiguous
    cap = capacity if capacity is not None else N
    k_codes = np.zeros((B, H, cap, d), np.int8)
    v_codes = np.zeros((B, H, cap, d), np.int8)
    if k_gran == GRAN_CHANNEL:
        ks = np.zeros((B, H, d), np.float32)
    elif k_gran == GRAN_TOKEN:
        ks = np.zeros((B, H, cap), np.float16)
    elif k_gran == GRAN_BLOCK:
        assert cap % BLOCK_N == 0
        ks = np.zeros((B, H, cap // BLOCK_N), np.float32)
    else:
        ks = np.zeros((1,), np.float32)
    vs = np.zeros((B, H, d), np.float32) if v_gran == GRAN_CHANNEL else np.zeros((B, H, cap), np.float16)
    km = np.zeros((B, H, d), np.float32)
    v_op = None
    vmax = np.zeros((B, H), np.float32) if v_gran == GRAN_TOKEN else None
    if v_op_format is not None:
        assert cap % 64 == 0
        v_op = np.zeros((B, H, cap // 64, d, 64), np.uint8)
    lib().orc_kv_quantize(B, H, N, d, cap, _p(_u16(k)), _p(_u16(v)), int(subtract_mean),
                          k_gran, v_gran, _p(k_codes), _p(v_codes), _p(ks), _p(vs), _p(km),
                          _p(v_op), 0 if v_op_format is None else v_op_format, _p(k_sum),
                          _p(vmax) if v_op is not None else None)
    if v_op is None:
        vmax = None
    return KVCache(k_codes, v_codes, ks, vs, km, v_op, k_gran, v_gran, cap, N, vmax)


def v_operand(cache: KVCache, n_keys: int, v_op_format: int = PV_FP8) -> KVCache:
    """(Re)build the cache's PV operand over its first n_keys keys from the V codes and
    scales (and, for per-token V, the header V_max): see v_operand in oracle_attn.cpp."""
    B, H, cap, d = cache.v_codes.shape
    assert cap % 64 == 0 and n_keys <= cap
    cache.v_op = np.zeros((B, H, cap // 64, d, 64), np.uint8)
    vs = np.ascontiguousarray(cache.v_scales)
    vs = vs.view(np.uint16) if vs.dtype == np.float16 else vs
    cache.v_scale_max = np.zeros((B, H), np.float32) if cache.v_gran == GRAN_TOKEN else None
    lib().orc_v_operand(B, H, d, cap, n_keys, _p(cache.v_codes), _p(vs), cache.v_gran, v_op_format,
                        _p(cache.v_op), _p(cache.v_scale_max))
    return cache


def empty_append_cache(B: int, H: int, capacity: int, d: int) -> KVCache:
    """An empty cache for kv_append (per-token K and V scales, header sum zero)."""
    return KVCache(np.zeros((B, H, capacity, d), np.int8), np.zeros((B, H, capacity, d), np.int8),
                   np.zeros((B, H, capacity), np.float16), np.zeros((B, H, capacity), np.float16),
                   np.zeros((B, H, d), np.float32), None, GRAN_TOKEN, GRAN_TOKEN, capacity, 0)


def kv_append(k: np.ndarray, v: np.ndarray, cache: KVCache, k_sum: np.ndarray) -> KVCache:
    """Append k, v fp16 [B][Hkv][T][d] at cache.seq_len with the running channel mean of K
    (see orc_kv_append); k_sum int64 [B][Hkv][d] is the cache header, updated in place."""
    B, H, T, d = k.shape
    assert cache.k_gran == GRAN_TOKEN and cache.v_gran == GRAN_TOKEN
    assert cache.seq_len + T <= cache.capacity and k_sum.dtype == np.int64
    assert k_sum.flags.c_contiguous and k_sum.shape == (B, H, d)
    lib().orc_kv_append(B, H, T, d, cache.capacity, cache.seq_len, _p(_u16(k)), _p(_u16(v)), _p(k_sum),
                        _p(cache.k_codes), _p(cache.v_codes), _p(cache.k_scales.view(np.uint16)),
                        _p(cache.v_scales.view(np.uint16)), _p(cache.k_mean))
    cache.seq_len += T
    return cache


def quantize_q(q: np.ndarray, hkv: int, q_gran: int, k_scales_channel: Optional[np.ndarray]):
    B, Hq, L, d = q.shape
    codes = np.empty((B, Hq, L, d), np.int8)
    scales = np.empty((B, Hq, L), np.float32)
    ksc = None if k_scales_channel is None else np.ascontiguousarray(k_scales_channel, np.float32)
    lib().orc_quantize_q(B, Hq, hkv, L, d, _p(_u16(q)), _p(ksc), q_gran, _p(codes), _p(scales))
    return codes, scales


# ------------------------------------------------------------- attention
@dataclass
class PrefillResult:
    out: np.ndarray                    # fp64 [B][Hq][q_len][d] (rows not listed stay 0)
    s_i32: Optional[np.ndarray]
    p_codes: Optional[np.ndarray]
    n_p: int
    n_flushed: int
    lse: np.ndarray                    # fp64 [B][Hq][q_len]: base-2 log-sum-exp of the row
    flushed_mass: np.ndarray           # fp64 [B][Hq][q_len]: softmax mass on keys with P code 0


def prefill_emulate(q: np.ndarray, cache: KVCache, *, kv_len: int, q_offset: int, causal: bool,
                    q_gran: int = GRAN_TOKEN, sm_scale: float = 0.0, pv_mode: int = PV_FP8,
                    block_c: int = KEY_TILE, n_streams: int = KEY_STREAMS,
                    rows: Optional[np.ndarray] = None,
                    want_s: bool = False, want_p: bool = False,
                    norm_fp32: bool = False, mx: Optional["MXOperands"] = None,
                    q_quant: Optional[tuple] = None) -> PrefillResult:
    """norm_fp32: normalize by the sum of the unquantized p instead of the quantized P.
    mx: Q and K below 8 bits (mx_operands); the scores are then the fp32 MX dots and
    ``s_i32`` holds them as float32 when want_s.  q_quant: (int8 codes [B][Hq][L][d], fp32
    scales [B][Hq][L]) used instead of quantizing q (for pins that fix the codes)."""
    B, Hq, L, d = q.shape
    H = cache.k_codes.shape[1]
    if mx is None:
        ksc = cache.k_scales if cache.k_gran == GRAN_CHANNEL else None
        if q_quant is None:
            qc, qs = quantize_q(q, H, q_gran, ksc)
        else:
            qc, qs = (np.ascontiguousarray(q_quant[0], np.int8), np.ascontiguousarray(q_quant[1], np.float32))
        qv = kv = None
    else:
        qc, qs = None, None
        qv, kv = np.ascontiguousarray(mx.q_values), np.ascontiguousarray(mx.k_values)
        assert qv.shape == q.shape and kv.shape == cache.k_codes.shape
    out = np.zeros((B, Hq, L, d), np.float64)
    s_i32 = np.zeros((B, Hq, L, kv_len), np.int32) if want_s and mx is None else None
    s_f32 = np.zeros((B, Hq, L, kv_len), np.float32) if want_s and mx is not None else None
    p_codes = np.zeros((B, Hq, L, kv_len), np.uint8) if want_p else None
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    flushed = ctypes.c_int64(0)
    ks = np.ascontiguousarray(cache.k_scales)
    ks = ks.view(np.uint16) if ks.dtype == np.float16 else ks.astype(np.float32, copy=False)
    vs = np.ascontiguousarray(cache.v_scales)
    vs = vs.view(np.uint16) if vs.dtype == np.float16 else vs.astype(np.float32, copy=False)
    vmax = None
    if cache.v_gran == GRAN_TOKEN:
        assert pv_mode == PV_FP8, "per-token V feeds the e4m3 operand only"
        # the header V_max the cache's operand was built against (else over the keys read)
        vmax = cache.v_scale_max if cache.v_scale_max is not None else \
            cache.v_scales[:, :, :kv_len].astype(np.float32).max(axis=2)
        vmax = np.ascontiguousarray(vmax, np.float32)
    lse = np.zeros((B, Hq, L), np.float64)
    fmass = np.zeros((B, Hq, L), np.float64)
    n = lib().orc_prefill_emulate(B, Hq, H, d, L, kv_len, cache.capacity, q_offset, int(causal),
                                  float(sm_scale), block_c, n_streams, _p(qc), _p(qs), _p(cache.k_codes),
                                  _p(ks), cache.k_gran, _p(cache.v_codes), _p(vs), cache.v_gran, _p(vmax),
                                  pv_mode, _p(rows_arr), 0 if rows_arr is None else rows_arr.size,
                                  _p(out), _p(s_i32), _p(p_codes), ctypes.byref(flushed), int(norm_fp32),
                                  _p(lse), _p(fmass), _p(qv), _p(kv), _p(s_f32))
    return PrefillResult(out, s_i32 if mx is None else s_f32, p_codes, int(n), int(flushed.value), lse, fmass)


def decode_emulate(q: np.ndarray, cache: KVCache, *, kv_len: int, sm_scale: float = 0.0,
                   want_qk: bool = False):
    """q fp16 [B][Hq][d] -> (out fp64 [B][Hq][d], int32 dots [B][Hq][kv_len] or None)."""
    B, Hq, d = q.shape
    H = cache.k_codes.shape[1]
    out = np.zeros((B, Hq, d), np.float64)
    dbg = np.zeros((B, Hq, kv_len), np.int32) if want_qk else None
    ks = cache.k_scales if cache.k_gran == GRAN_TOKEN else np.ascontiguousarray(cache.k_scales, np.float32)
    vs = cache.v_scales if cache.v_gran == GRAN_TOKEN else np.ascontiguousarray(cache.v_scales, np.float32)
    ks = ks.view(np.uint16) if ks.dtype == np.float16 else ks
    vs = vs.view(np.uint16) if vs.dtype == np.float16 else vs
    lib().orc_decode_emulate(B, Hq, H, d, kv_len, cache.capacity, float(sm_scale), _p(_u16(q)),
                             _p(cache.k_codes), _p(np.ascontiguousarray(ks)), cache.k_gran,
                             _p(cache.v_codes), _p(np.ascontiguousarray(vs)), cache.v_gran,
                             _p(out), _p(dbg))
    return out, dbg


def attn_exact(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool = False,
               q_offset: int = 0, sm_scale: float = 0.0, kmu: Optional[np.ndarray] = None,
               rows: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 attention from fp16 inputs; q [B][Hq][L][d], k/v [B][Hkv][N][d]."""
    B, Hq, L, d = q.shape
    H, N = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, L, d), np.float64)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    mu = None if kmu is None else np.ascontiguousarray(kmu, np.float64)
    lib().orc_attn_exact(B, Hq, H, d, L, N, q_offset, int(causal), float(sm_scale),
                         _p(_u16(q)), _p(_u16(k)), _p(_u16(v)), _p(mu), _p(rows_arr),
                         0 if rows_arr is None else rows_arr.size, _p(out))
    return out


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on."""
    lib().orc_set_threads(int(n))


def attn_dequant(q: np.ndarray, cache: KVCache, *, kv_len: int, q_offset: int = 0, causal: bool = False,
                 sm_scale: float = 0.0, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 attention over the dequantized int8 cache (see orc_attn_dequant): K codes times
    their per-channel / per-tensor scales, V codes times their per-channel scales.
    q fp16 [B][Hq][L][d] -> out fp64 [B][Hq][L][d] (rows not listed stay 0)."""
    B, Hq, L, d = q.shape
    H = cache.k_codes.shape[1]
    assert cache.v_gran == GRAN_CHANNEL and cache.k_gran in (GRAN_CHANNEL, GRAN_TENSOR)
    out = np.zeros((B, Hq, L, d), np.float64)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    lib().orc_attn_dequant(B, Hq, H, d, L, kv_len, cache.capacity, q_offset, int(causal), float(sm_scale),
                           _p(_u16(q)), _p(cache.k_codes), _p(np.ascontiguousarray(cache.k_scales, np.float32)),
                           cache.k_gran, _p(cache.v_codes), _p(np.ascontiguousarray(cache.v_scales, np.float32)),
                           _p(rows_arr), 0 if rows_arr is None else rows_arr.size, _p(out))
    return out


# sub-8-bit grids for Q and K (see orc_attn_lowbit)
LB_INT8_ROW, LB_INT8_BLOCK, LB_INT4_BLOCK, LB_MXFP6, LB_MXFP4 = 0, 1, 2, 3, 4


def attn_lowbit(q: np.ndarray, k: np.ndarray, v: np.ndarray, fmt_q: int, fmt_k: int, *, causal: bool = False,
                q_offset: int = 0, sm_scale: float = 0.0, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 attention with Q and (mean-shifted) K replaced by their values in the given grids."""
    B, Hq, L, d = q.shape
    H, N = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, L, d), np.float64)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    lib().orc_attn_lowbit(B, Hq, H, d, L, N, q_offset, int(causal), float(sm_scale), _p(_u16(q)), _p(_u16(k)),
                          _p(_u16(v)), fmt_q, fmt_k, _p(rows_arr), 0 if rows_arr is None else rows_arr.size, _p(out))
    return out


def lowbit_element(x: np.ndarray, fmt: int):
    """Round to the E2M1 (fmt LB_MXFP4) or E2M3 (LB_MXFP6) grid with unit scale -> (values, codes)."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty_like(x)
    codes = np.empty(x.shape, np.int32)
    lib().orc_lowbit_element(_p(x), x.size, fmt, _p(out), _p(codes))
    return out, codes


@dataclass
class MXEncoded:
    codes: np.ndarray        # uint8 [..., d]: sign bit | magnitude code, one per element
    scale_bytes: np.ndarray  # uint8 [..., d/32]: E8M0 exponent bytes (127 + e)
    values: np.ndarray       # fp64 [..., d]: the dequantized values


def mx_quantize(x: np.ndarray, fmt: int) -> MXEncoded:
    """MX encoding of fp32 rows (last axis a multiple of 32) in LB_MXFP6 / LB_MXFP4."""
    x = np.ascontiguousarray(x, np.float32)
    d = x.shape[-1]
    rows = x.size // d
    codes = np.zeros(x.shape, np.uint8)
    sb = np.zeros(x.shape[:-1] + (d // 32,), np.uint8)
    vals = np.zeros(x.shape, np.float64)
    rc = lib().orc_mx_quantize(_p(x), rows, d, fmt, _p(codes), _p(sb), _p(vals))
    assert rc == 0, "a block scale outside the E8M0 range"
    return MXEncoded(codes, sb, vals)


def k_quantize_mx(k: np.ndarray, k_mean: np.ndarray, fmt: int, capacity: Optional[int] = None) -> MXEncoded:
    """K fp16 [B][H][N][d] shifted by the cache's per-channel mean (fp32(k) - mu, as the int8
    path) and MX-encoded; rows N .. capacity-1 are zero codes with scale byte 0."""
    B, H, N, d = k.shape
    cap = capacity or N
    x = k.astype(np.float32) - np.asarray(k_mean, np.float32)[:, :, None, :]
    e = mx_quantize(x, fmt)
    codes = np.zeros((B, H, cap, d), np.uint8)
    sb = np.zeros((B, H, cap, d // 32), np.uint8)
    vals = np.zeros((B, H, cap, d), np.float64)
    codes[:, :, :N], sb[:, :, :N], vals[:, :, :N] = e.codes, e.scale_bytes, e.values
    return MXEncoded(codes, sb, vals)


@dataclass
class MXOperands:
    q_values: np.ndarray   # fp64 [B][Hq][L][d]
    k_values: np.ndarray   # fp64 [B][Hkv][cap][d]


def mx_operands(q: np.ndarray, q_fmt: int, k_enc: MXEncoded) -> MXOperands:
    """Q fp16 MX-encoded per row (no shift) beside the encoded K, for prefill_emulate(mx=...)."""
    return MXOperands(mx_quantize(q.astype(np.float32), q_fmt).values, k_enc.values)


def lowbit_row(x: np.ndarray, fmt: int) -> np.ndarray:
    """Dequantized values of one fp32 row in a format."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.float64)
    lib().orc_lowbit_row(_p(x), x.size, fmt, _p(out))
    return out

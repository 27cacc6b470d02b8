"""ctypes binding of libattn_q.so (include/attn_q.h).

Argument marshalling only: PyTorch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  The entry
points keep the C names: ``kv_quantize_i8``, ``attn_q_prefill``, ``attn_q_decode``,
``attn_q_kv_append_i8``, ``attn_q_decode_append``, ``attn_q_short_fused``,
``attn_q_k_quantize_mx`` and ``attn_q_prefill_mx``.  If the
library is missing this module raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_q.so")

# enums (attn_q.h)
OK, E_NULL, E_SHAPE, E_UNSUPPORTED, E_ALIGN, E_WORKSPACE, E_DEVICE, E_LAUNCH, E_SCRATCH = \
    0, -1, -2, -3, -4, -5, -6, -7, -8
GRAN_TENSOR, GRAN_BLOCK, GRAN_TOKEN, GRAN_CHANNEL = 0, 1, 2, 3
BLOCK = 64   # tokens per BLOCK-granularity scale (ATTN_Q_BLOCK)
PV_FP8, PV_INT8, PV_SPLIT24 = 0, 1, 2
MX_FP6, MX_FP4 = 2, 4   # attn_q_mx_format: E2M3 / E2M1 elements, one E8M0 scale per 32 channels
MX_BITS = {MX_FP6: 6, MX_FP4: 4}
OUT_F16, OUT_F32 = 0, 1
KEY_TILE = 64

P = ctypes.c_void_p
i32 = ctypes.c_int32


class KvqArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("kv_heads", i32), ("seq_len", i32), ("head_dim", i32),
                ("capacity", i32), ("k", P), ("v", P), ("subtract_k_mean", i32),
                ("k_gran", i32), ("v_gran", i32), ("k_codes", P), ("v_codes", P),
                ("k_scales", P), ("v_scales", P), ("k_mean", P), ("k_sum", P), ("v_op", P),
                ("v_op_format", i32), ("v_scale_max", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t)]


class VopArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("kv_heads", i32), ("head_dim", i32), ("capacity", i32), ("n_keys", i32),
                ("v_codes", P), ("v_scales", P), ("v_gran", i32), ("v_op", P), ("v_op_format", i32),
                ("v_scale_max", P)]


class KvAppendArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("kv_heads", i32), ("head_dim", i32), ("capacity", i32),
                ("seq_len", i32), ("new_tokens", i32), ("k", P), ("v", P), ("k_sum", P),
                ("k_codes", P), ("v_codes", P), ("k_scales", P), ("v_scales", P), ("k_mean", P),
                ("workspace", P), ("workspace_bytes", ctypes.c_size_t)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("q_heads", i32), ("kv_heads", i32), ("head_dim", i32),
                ("q_len", i32), ("kv_len", i32), ("q_offset", i32), ("causal", i32),
                ("sm_scale", ctypes.c_float), ("q", P), ("q_gran", i32), ("k_codes", P),
                ("k_scales", P), ("k_gran", i32), ("v_op", P), ("v_scales", P),
                ("v_gran", i32), ("v_scale_max", P),
                ("pv_mode", i32), ("capacity", i32), ("out", P), ("out_dtype", i32), ("lse", P),
                ("debug_s", P), ("debug_p", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("q_heads", i32), ("kv_heads", i32), ("head_dim", i32),
                ("kv_len", i32), ("capacity", i32), ("kv_lens", P), ("sm_scale", ctypes.c_float), ("q", P),
                ("k_codes", P), ("k_scales", P), ("k_gran", i32), ("v_codes", P),
                ("v_scales", P), ("v_gran", i32), ("out", P), ("out_dtype", i32),
                ("debug_qk", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t)]


class ShortArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("heads", i32), ("seq_len", i32), ("head_dim", i32),
                ("sm_scale", ctypes.c_float), ("q", P), ("k", P), ("v", P), ("out", P),
                ("out_dtype", i32), ("debug_s", P)]


class KMxArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("kv_heads", i32), ("seq_len", i32), ("head_dim", i32), ("capacity", i32),
                ("fmt", i32), ("k", P), ("k_mean", P), ("k_mx", P), ("k_mx_scales", P)]


class PrefillMxArgs(ctypes.Structure):
    _fields_ = [("batch", i32), ("q_heads", i32), ("kv_heads", i32), ("head_dim", i32),
                ("q_len", i32), ("kv_len", i32), ("q_offset", i32), ("causal", i32),
                ("sm_scale", ctypes.c_float), ("q", P), ("q_fmt", i32), ("k_mx", P), ("k_mx_scales", P),
                ("k_fmt", i32), ("capacity", i32), ("v_op", P), ("v_scales", P), ("out", P),
                ("out_dtype", i32), ("debug_s", P)]


EXPORTS = ["kv_quantize_i8", "attn_q_v_operand", "attn_q_prefill", "attn_q_decode", "attn_q_decode_noalloc", "attn_q_kv_append_i8",
           "attn_q_decode_append",
           "attn_q_short_fused", "attn_q_k_quantize_mx", "attn_q_prefill_mx",
           "kv_quantize_i8_workspace_size", "attn_q_prefill_workspace_size",
           "attn_q_decode_workspace_size", "attn_q_kv_append_i8_workspace_size",
           "attn_q_status_string", "attn_q_version"]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_attention_attn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kv_quantize_i8.argtypes = [ctypes.POINTER(KvqArgs), P]
        L.attn_q_v_operand.argtypes = [ctypes.POINTER(VopArgs), P]
        L.attn_q_prefill.argtypes = [ctypes.POINTER(PrefillArgs), P]
        L.attn_q_decode.argtypes = [ctypes.POINTER(DecodeArgs), P]
        L.attn_q_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), P]
        L.attn_q_kv_append_i8.argtypes = [ctypes.POINTER(KvAppendArgs), P]
        L.attn_q_decode_append.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(KvAppendArgs), P]
        L.attn_q_short_fused.argtypes = [ctypes.POINTER(ShortArgs), P]
        L.attn_q_k_quantize_mx.argtypes = [ctypes.POINTER(KMxArgs), P]
        L.attn_q_prefill_mx.argtypes = [ctypes.POINTER(PrefillMxArgs), P]
        for f, t in [("kv_quantize_i8_workspace_size", KvqArgs),
                     ("attn_q_prefill_workspace_size", PrefillArgs),
                     ("attn_q_decode_workspace_size", DecodeArgs),
                     ("attn_q_kv_append_i8_workspace_size", KvAppendArgs)]:
            getattr(L, f).argtypes = [ctypes.POINTER(t)]
            getattr(L, f).restype = ctypes.c_size_t
        L.attn_q_status_string.argtypes = [ctypes.c_int]
        L.attn_q_status_string.restype = ctypes.c_char_p
        L.attn_q_version.restype = ctypes.c_int
        _lib = L
    return _lib


class AttnQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib().attn_q_status_string(status).decode()} ({status})")
        self.status = status


def _check(status: int, where: str):
    if status != OK:
        raise AttnQError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libattn_q must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t: torch.Tensor, name: str, dtype, shape, device):
    """Argument check before any pointer reaches the library (dtype, shape, device, layout)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out_dtype(out: Optional[torch.Tensor], out_dtype: int) -> int:
    """The output mode of a caller-supplied out tensor is its dtype."""
    if out is None:
        return out_dtype
    if out.dtype == torch.float32:
        return OUT_F32
    if out.dtype == torch.float16:
        return OUT_F16
    raise ValueError(f"out must be float16 or float32, got {out.dtype}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ws_cache = {}


def workspace(nbytes: int, device, key: str = "", zero: bool = False) -> torch.Tensor:
    """Device scratch owned by the binding (allocated once per size and purpose)."""
    k = (str(device), key)
    ws = _ws_cache.get(k)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device) if zero else \
            torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[k] = ws
    return ws


@dataclass
class KVCache:
    """Device buffers of the int8 KV cache written by kv_quantize_i8."""
    k_codes: torch.Tensor
    v_codes: Optional[torch.Tensor]   # None: a cache that serves the prefill's fp8 PV only
    k_scales: torch.Tensor
    v_scales: torch.Tensor
    k_mean: torch.Tensor
    v_op: Optional[torch.Tensor]
    v_op_format: int
    k_gran: int
    v_gran: int
    capacity: int
    seq_len: int
    k_sum: Optional[torch.Tensor] = None   # int64 [B][Hkv][d] header of attn_q_kv_append_i8
    v_scale_max: Optional[torch.Tensor] = None   # fp32 [B][Hkv] header V_max (per-token V operand)

    @property
    def shape(self):
        return self.k_codes.shape


def alloc_cache(batch, kv_heads, capacity, head_dim, k_gran, v_gran, device,
                v_op_format: Optional[int] = PV_FP8, seq_len: int = 0, header: bool = False,
                v_codes: bool = True) -> KVCache:
    """Zero-filled cache buffers; header=True adds the int64 K-sum header that
    kv_quantize_i8 fills and attn_q_kv_append_i8 continues (a zero header is an
    empty cache); v_codes=False leaves out the int8 V codes (per-channel V with the e4m3
    operand: a cache for attn_q_prefill's fp8 PV only)."""
    B, H, C, D = batch, kv_heads, capacity, head_dim
    z = dict(device=device)
    k_codes = torch.zeros((B, H, C, D), dtype=torch.int8, **z)
    if not v_codes and (v_op_format != PV_FP8 or v_gran != GRAN_CHANNEL):
        raise ValueError("only a per-channel cache with the e4m3 V operand may leave out the V codes")
    vc = torch.zeros((B, H, C, D), dtype=torch.int8, **z) if v_codes else None
    if k_gran == GRAN_TOKEN:
        ks = torch.zeros((B, H, C), dtype=torch.float16, **z)
    elif k_gran == GRAN_CHANNEL:
        ks = torch.zeros((B, H, D), dtype=torch.float32, **z)
    elif k_gran == GRAN_BLOCK:
        ks = torch.zeros((B, H, C // BLOCK), dtype=torch.float32, **z)
    else:
        ks = torch.zeros((4,), dtype=torch.float32, **z)
    vs = torch.zeros((B, H, C), dtype=torch.float16, **z) if v_gran == GRAN_TOKEN else \
        torch.zeros((B, H, D), dtype=torch.float32, **z)
    km = torch.zeros((B, H, D), dtype=torch.float32, **z)
    v_op = None
    if v_op_format is not None:
        v_op = torch.zeros((B, H, C // KEY_TILE, D, KEY_TILE), dtype=torch.uint8, **z)
    k_sum = torch.zeros((B, H, D), dtype=torch.int64, **z) if header else None
    vmax = torch.zeros((B, H), dtype=torch.float32, **z) if v_gran == GRAN_TOKEN else None
    return KVCache(k_codes, vc, ks, vs, km, v_op, -1 if v_op_format is None else v_op_format,
                   k_gran, v_gran, C, seq_len, k_sum, vmax)


def kv_quantize_i8(k: torch.Tensor, v: torch.Tensor, cache: KVCache, *, subtract_k_mean: bool = True,
                   stream=None) -> KVCache:
    """k, v: fp16 [B][Hkv][N][d] on the GPU -> fills `cache` (see attn_q.h)."""
    if k.dim() != 4:
        raise ValueError("k must be [B][Hkv][N][d]")
    B, H, N, D = k.shape
    _expect(k, "k", torch.float16, None, cache.k_codes.device)
    _expect(v, "v", torch.float16, k.shape, cache.k_codes.device)
    a = KvqArgs(B, H, N, D, cache.capacity, _ptr(k), _ptr(v), int(subtract_k_mean), cache.k_gran,
                cache.v_gran, _ptr(cache.k_codes), _ptr(cache.v_codes), _ptr(cache.k_scales),
                _ptr(cache.v_scales), _ptr(cache.k_mean), _ptr(cache.k_sum), _ptr(cache.v_op),
                max(cache.v_op_format, 0), _ptr(cache.v_scale_max), None, 0)
    nbytes = lib().kv_quantize_i8_workspace_size(ctypes.byref(a))
    # zero-filled once; every call leaves its accumulators zeroed (one buffer per shape)
    ws = workspace(nbytes, k.device, f"kvq{B}x{H}x{D}", zero=True)
    a.workspace, a.workspace_bytes = _ptr(ws), ws.numel()
    _check(lib().kv_quantize_i8(ctypes.byref(a), stream or _stream(k.device)), "kv_quantize_i8")
    cache.seq_len = N
    return cache


def attn_q_v_operand(cache: KVCache, *, n_keys: Optional[int] = None, v_op_format: Optional[int] = None,
                     stream=None) -> KVCache:
    """(Re)build cache.v_op (and, for per-token V, the header cache.v_scale_max) from the V codes
    and scales of keys [0, n_keys) (default: cache.seq_len), e.g. after appends (attn_q.h)."""
    if cache.v_codes is None:
        raise ValueError("attn_q_v_operand rebuilds the operand from the V codes, which this cache leaves out")
    B, H, cap, D = cache.v_codes.shape
    dev = cache.v_codes.device
    fmt = v_op_format if v_op_format is not None else (cache.v_op_format if cache.v_op_format >= 0 else PV_FP8)
    if cache.v_op is None:
        cache.v_op = torch.zeros((B, H, cap // KEY_TILE, D, KEY_TILE), dtype=torch.uint8, device=dev)
    if cache.v_gran == GRAN_TOKEN and cache.v_scale_max is None:
        cache.v_scale_max = torch.zeros((B, H), dtype=torch.float32, device=dev)
    n = cache.seq_len if n_keys is None else n_keys
    a = VopArgs(B, H, D, cap, n, _ptr(cache.v_codes), _ptr(cache.v_scales), cache.v_gran, _ptr(cache.v_op), fmt,
                _ptr(cache.v_scale_max))
    _check(lib().attn_q_v_operand(ctypes.byref(a), stream or _stream(dev)), "attn_q_v_operand")
    cache.v_op_format = fmt
    return cache


def attn_q_prefill(q: torch.Tensor, cache: KVCache, *, kv_len: int, q_offset: int = 0,
                   causal: bool = False, q_gran: int = GRAN_TOKEN, pv_mode: int = PV_FP8,
                   out_dtype: int = OUT_F16, sm_scale: float = 0.0,
                   out: Optional[torch.Tensor] = None, debug_s: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, debug_p: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """q fp16 [B][Hq][q_len][d] -> out [B][Hq][q_len][d] (fp16 or fp32); lse (optional) fp32
    [B][Hq][q_len] receives the rows' base-2 log-sum-exp; debug_s / debug_p (optional) int32 /
    uint8 [B][Hq][q_len][kv_len] receive the int32 scores / P codes (tests)."""
    if q.dim() != 4:
        raise ValueError("q must be [B][Hq][q_len][d]")
    B, Hq, L, D = q.shape
    H = cache.k_codes.shape[1]
    _expect(q, "q", torch.float16, None, cache.k_codes.device)
    out_dtype = _out_dtype(out, out_dtype)
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=torch.float32 if out_dtype == OUT_F32 else torch.float16,
                          device=q.device)
    _expect(out, "out", None, (B, Hq, L, D), q.device)
    want_op = PV_FP8 if pv_mode == PV_FP8 else PV_INT8   # INT8 and SPLIT24 read int8 V operands
    if cache.v_op is None or cache.v_op_format != want_op:
        raise ValueError(f"pv_mode {pv_mode} needs a cache whose V operand was written with v_op_format {want_op}")
    if lse is not None:
        _expect(lse, "lse", torch.float32, (B, Hq, L), q.device)
    if debug_s is not None:
        _expect(debug_s, "debug_s", torch.int32, (B, Hq, L, kv_len), q.device)
    if debug_p is not None:
        _expect(debug_p, "debug_p", torch.uint8, (B, Hq, L, kv_len), q.device)
    a = PrefillArgs(B, Hq, H, D, L, kv_len, q_offset, int(causal), sm_scale, _ptr(q), q_gran,
                    _ptr(cache.k_codes), _ptr(cache.k_scales), cache.k_gran, _ptr(cache.v_op),
                    _ptr(cache.v_scales) if cache.v_gran == GRAN_CHANNEL else None, cache.v_gran,
                    _ptr(cache.v_scale_max), pv_mode, cache.capacity, _ptr(out), out_dtype, _ptr(lse),
                    _ptr(debug_s), _ptr(debug_p), None, 0)
    nbytes = lib().attn_q_prefill_workspace_size(ctypes.byref(a))
    if nbytes:
        ws = workspace(nbytes, q.device, "prefill")
        a.workspace, a.workspace_bytes = _ptr(ws), ws.numel()
    _check(lib().attn_q_prefill(ctypes.byref(a), stream or _stream(q.device)), "attn_q_prefill")
    return out


def attn_q_decode(q: torch.Tensor, cache: KVCache, *, kv_len: int, out_dtype: int = OUT_F16,
                  sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                  debug_qk: Optional[torch.Tensor] = None, kv_lens: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """q fp16 [B][Hq][d] -> out [B][Hq][d]; kv_lens (optional, device int32 [B]): each row's
    keys, kv_len their maximum."""
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][d]")
    B, Hq, D = q.shape
    H = cache.k_codes.shape[1]
    _expect(q, "q", torch.float16, None, cache.k_codes.device)
    out_dtype = _out_dtype(out, out_dtype)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32 if out_dtype == OUT_F32 else torch.float16,
                          device=q.device)
    _expect(out, "out", None, (B, Hq, D), q.device)
    if kv_lens is not None:
        _expect(kv_lens, "kv_lens", torch.int32, (B,), q.device)
    a = DecodeArgs(B, Hq, H, D, kv_len, cache.capacity, _ptr(kv_lens), sm_scale, _ptr(q), _ptr(cache.k_codes),
                   _ptr(cache.k_scales), cache.k_gran, _ptr(cache.v_codes), _ptr(cache.v_scales),
                   cache.v_gran, _ptr(out), out_dtype, _ptr(debug_qk), None, 0)
    nbytes = lib().attn_q_decode_workspace_size(ctypes.byref(a))
    ws = workspace(nbytes, q.device, "decode")
    a.workspace, a.workspace_bytes = _ptr(ws), ws.numel()
    _check(lib().attn_q_decode(ctypes.byref(a), stream or _stream(q.device)), "attn_q_decode")
    return out


def attn_q_decode_noalloc(q: torch.Tensor, cache: KVCache, *, kv_len: int, out: torch.Tensor,
                          sm_scale: float = 0.0, debug_qk: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """attn_q_decode without a workspace (the library's static scratch): q fp16 [B][Hq][d] ->
    the caller's out [B][Hq][d] (fp16 or fp32).  Nothing is allocated here either."""
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][d]")
    B, Hq, D = q.shape
    H = cache.k_codes.shape[1]
    _expect(q, "q", torch.float16, None, cache.k_codes.device)
    _expect(out, "out", None, (B, Hq, D), q.device)
    out_dtype = _out_dtype(out, OUT_F16)
    a = DecodeArgs(B, Hq, H, D, kv_len, cache.capacity, None, sm_scale, _ptr(q), _ptr(cache.k_codes),
                   _ptr(cache.k_scales), cache.k_gran, _ptr(cache.v_codes), _ptr(cache.v_scales),
                   cache.v_gran, _ptr(out), out_dtype, _ptr(debug_qk), None, 0)
    _check(lib().attn_q_decode_noalloc(ctypes.byref(a), stream or _stream(q.device)), "attn_q_decode_noalloc")
    return out


def attn_q_kv_append_i8(k: torch.Tensor, v: torch.Tensor, cache: KVCache, *, stream=None) -> KVCache:
    """k, v: fp16 [B][Hkv][T][d] on the GPU, appended at row cache.seq_len with the running
    K mean of cache.k_sum (see attn_q.h); the cache needs per-token K and V scales and a
    header (alloc_cache(..., GRAN_TOKEN, GRAN_TOKEN, header=True))."""
    if k.dim() != 4:
        raise ValueError("k must be [B][Hkv][T][d]")
    B, H, T, D = k.shape
    if cache.k_gran != GRAN_TOKEN or cache.v_gran != GRAN_TOKEN:
        raise ValueError("appending needs per-token K and V scales (GRAN_TOKEN)")
    if cache.k_sum is None:
        raise ValueError("the cache has no K-sum header (alloc_cache(..., header=True))")
    dev = cache.k_codes.device
    _expect(k, "k", torch.float16, (B, H, T, D), dev)
    _expect(v, "v", torch.float16, (B, H, T, D), dev)
    _expect(cache.k_codes, "cache.k_codes", torch.int8, (B, H, cache.capacity, D), dev)
    _expect(cache.k_sum, "cache.k_sum", torch.int64, (B, H, D), dev)
    _expect(cache.k_scales, "cache.k_scales", torch.float16, (B, H, cache.capacity), dev)
    _expect(cache.v_scales, "cache.v_scales", torch.float16, (B, H, cache.capacity), dev)
    a = KvAppendArgs(B, H, D, cache.capacity, cache.seq_len, T, _ptr(k), _ptr(v), _ptr(cache.k_sum),
                     _ptr(cache.k_codes), _ptr(cache.v_codes), _ptr(cache.k_scales), _ptr(cache.v_scales),
                     _ptr(cache.k_mean), None, 0)
    nbytes = lib().attn_q_kv_append_i8_workspace_size(ctypes.byref(a))
    if nbytes:
        ws = workspace(nbytes, dev, "append")
        a.workspace, a.workspace_bytes = _ptr(ws), ws.numel()
    _check(lib().attn_q_kv_append_i8(ctypes.byref(a), stream or _stream(dev)), "attn_q_kv_append_i8")
    cache.seq_len += T
    return cache


def attn_q_decode_append(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cache: KVCache, *,
                         out_dtype: int = OUT_F16, sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                         debug_qk: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step in one launch: k, v fp16 [B][Hkv][d] (the new token) appended at row
    cache.seq_len with the running K mean, then q fp16 [B][Hq][d] attends over the
    cache.seq_len + 1 keys (see attn_q.h); the same bits as attn_q_kv_append_i8 followed by
    attn_q_decode."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [B][Hq][d], k and v [B][Hkv][d]")
    B, Hq, D = q.shape
    H = cache.k_codes.shape[1]
    if cache.k_gran != GRAN_TOKEN or cache.v_gran != GRAN_TOKEN:
        raise ValueError("appending needs per-token K and V scales (GRAN_TOKEN)")
    if cache.k_sum is None:
        raise ValueError("the cache has no K-sum header (alloc_cache(..., header=True))")
    dev = cache.k_codes.device
    _expect(q, "q", torch.float16, None, dev)
    _expect(k, "k", torch.float16, (B, H, D), dev)
    _expect(v, "v", torch.float16, (B, H, D), dev)
    _expect(cache.k_sum, "cache.k_sum", torch.int64, (B, H, D), dev)
    _expect(cache.k_scales, "cache.k_scales", torch.float16, (B, H, cache.capacity), dev)
    _expect(cache.v_scales, "cache.v_scales", torch.float16, (B, H, cache.capacity), dev)
    out_dtype = _out_dtype(out, out_dtype)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32 if out_dtype == OUT_F32 else torch.float16, device=dev)
    _expect(out, "out", None, (B, Hq, D), dev)
    kv_len = cache.seq_len + 1
    d = DecodeArgs(B, Hq, H, D, kv_len, cache.capacity, None, sm_scale, _ptr(q), _ptr(cache.k_codes),
                   _ptr(cache.k_scales), cache.k_gran, _ptr(cache.v_codes), _ptr(cache.v_scales),
                   cache.v_gran, _ptr(out), out_dtype, _ptr(debug_qk), None, 0)
    nbytes = lib().attn_q_decode_workspace_size(ctypes.byref(d))
    ws = workspace(nbytes, dev, "decode")
    d.workspace, d.workspace_bytes = _ptr(ws), ws.numel()
    a = KvAppendArgs(B, H, D, cache.capacity, cache.seq_len, 1, _ptr(k), _ptr(v), _ptr(cache.k_sum),
                     _ptr(cache.k_codes), _ptr(cache.v_codes), _ptr(cache.k_scales), _ptr(cache.v_scales),
                     _ptr(cache.k_mean), None, 0)
    _check(lib().attn_q_decode_append(ctypes.byref(d), ctypes.byref(a), stream or _stream(dev)),
           "attn_q_decode_append")
    cache.seq_len += 1
    return out


def attn_q_short_fused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, out_dtype: int = OUT_F16,
                       sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                       debug_s: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q, k, v: fp16 [B][H][N][d] on the GPU (N <= 256, d in {32, 64}) -> out [B][H][N][d]:
    quantization of the head and attention in one kernel (see attn_q.h)."""
    if q.dim() != 4:
        raise ValueError("q must be [B][H][N][d]")
    Bn, H, N, D = q.shape
    dev = q.device
    _expect(q, "q", torch.float16, None, dev)
    _expect(k, "k", torch.float16, q.shape, dev)
    _expect(v, "v", torch.float16, q.shape, dev)
    out_dtype = _out_dtype(out, out_dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if out_dtype == OUT_F32 else torch.float16, device=dev)
    _expect(out, "out", None, q.shape, dev)
    if debug_s is not None:
        _expect(debug_s, "debug_s", torch.int32, (Bn, H, N, N), dev)
    a = ShortArgs(Bn, H, N, D, float(sm_scale), _ptr(q), _ptr(k), _ptr(v), _ptr(out), out_dtype, _ptr(debug_s))
    _check(lib().attn_q_short_fused(ctypes.byref(a), stream or _stream(dev)), "attn_q_short_fused")
    return out


@dataclass
class MXKeys:
    """K as MX operands (attn_q_k_quantize_mx): packed codes and E8M0 block scales."""
    codes: torch.Tensor    # uint8 [B][Hkv][capacity][d * bits / 8]
    scales: torch.Tensor   # uint8 [B][Hkv][capacity][d / 32]
    fmt: int


def alloc_mx_keys(batch, kv_heads, capacity, head_dim, fmt, device) -> MXKeys:
    return MXKeys(torch.zeros((batch, kv_heads, capacity, head_dim * MX_BITS[fmt] // 8), dtype=torch.uint8,
                              device=device),
                  torch.zeros((batch, kv_heads, capacity, head_dim // 32), dtype=torch.uint8, device=device), fmt)


def attn_q_k_quantize_mx(k: torch.Tensor, k_mean: torch.Tensor, keys: MXKeys, *, stream=None) -> MXKeys:
    """k fp16 [B][Hkv][N][d] shifted by k_mean fp32 [B][Hkv][d] (the cache's mean) -> keys rows 0..N-1."""
    if k.dim() != 4:
        raise ValueError("k must be [B][Hkv][N][d]")
    B, H, N, D = k.shape
    C = keys.codes.shape[2]
    _expect(k, "k", torch.float16, None, keys.codes.device)
    _expect(k_mean, "k_mean", torch.float32, (B, H, D), k.device)
    _expect(keys.codes, "keys.codes", torch.uint8, (B, H, C, D * MX_BITS[keys.fmt] // 8), k.device)
    _expect(keys.scales, "keys.scales", torch.uint8, (B, H, C, D // 32), k.device)
    a = KMxArgs(B, H, N, D, C, keys.fmt, _ptr(k), _ptr(k_mean), _ptr(keys.codes), _ptr(keys.scales))
    _check(lib().attn_q_k_quantize_mx(ctypes.byref(a), stream or _stream(k.device)), "attn_q_k_quantize_mx")
    return keys


def attn_q_prefill_mx(q: torch.Tensor, keys: MXKeys, cache: KVCache, *, kv_len: int, q_fmt: int,
                      q_offset: int = 0, causal: bool = False, out_dtype: int = OUT_F16, sm_scale: float = 0.0,
                      out: Optional[torch.Tensor] = None, debug_s: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """q fp16 [B][Hq][q_len][d] against MX keys and the cache's per-channel e4m3 V operand ->
    out [B][Hq][q_len][d]; debug_s (optional) fp32 [B][Hq][q_len][kv_len] receives the scores."""
    if q.dim() != 4:
        raise ValueError("q must be [B][Hq][q_len][d]")
    B, Hq, L, D = q.shape
    H, C = keys.codes.shape[1], keys.codes.shape[2]
    _expect(q, "q", torch.float16, None, keys.codes.device)
    if cache.v_op is None or cache.v_op_format != PV_FP8 or cache.v_gran != GRAN_CHANNEL:
        raise ValueError("attn_q_prefill_mx reads a per-channel V cache with the e4m3 operand")
    if cache.capacity != C:
        raise ValueError("keys and cache capacities differ")
    out_dtype = _out_dtype(out, out_dtype)
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=torch.float32 if out_dtype == OUT_F32 else torch.float16,
                          device=q.device)
    _expect(out, "out", None, (B, Hq, L, D), q.device)
    if debug_s is not None:
        _expect(debug_s, "debug_s", torch.float32, (B, Hq, L, kv_len), q.device)
    a = PrefillMxArgs(B, Hq, H, D, L, kv_len, q_offset, int(causal), sm_scale, _ptr(q), q_fmt, _ptr(keys.codes),
                      _ptr(keys.scales), keys.fmt, C, _ptr(cache.v_op), _ptr(cache.v_scales), _ptr(out), out_dtype,
                      _ptr(debug_s))
    _check(lib().attn_q_prefill_mx(ctypes.byref(a), stream or _stream(q.device)), "attn_q_prefill_mx")
    return out

"""C-ABI contract tests that need no GPU: the library loads, exports every
function include/attn_q.h declares, and rejects invalid arguments with the
documented status codes before touching the HIP runtime (validation runs before
any HIP call, so these calls launch nothing)."""
import ctypes
import os
import re

import pytest

from quantized_attention_attn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_q.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libattn_q.so not built")


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*\**\s*(\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(B.EXPORTS)
    L = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = B.lib()
    assert L.attn_q_version() == 6
    for st in range(-8, 1):
        s = L.attn_q_status_string(st)
        assert s and s != b"unknown status"
    assert L.attn_q_status_string(12345) == b"unknown status"


def test_struct_layouts_match_header(tmp_path):
    """ctypes field offsets equal the C compiler's offsetof for every field."""
    import subprocess
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "attn_q.h"', "int main(void){"]
    for cname, py in [("attn_q_kvq_args", B.KvqArgs), ("attn_q_prefill_args", B.PrefillArgs),
                      ("attn_q_decode_args", B.DecodeArgs),
                      ("attn_q_kv_append_args", B.KvAppendArgs), ("attn_q_short_args", B.ShortArgs),
                      ("attn_q_k_mx_args", B.KMxArgs), ("attn_q_prefill_mx_args", B.PrefillMxArgs)]:
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)]).decode().splitlines())
    for cname, py in [("attn_q_kvq_args", B.KvqArgs), ("attn_q_prefill_args", B.PrefillArgs),
                      ("attn_q_decode_args", B.DecodeArgs),
                      ("attn_q_kv_append_args", B.KvAppendArgs), ("attn_q_short_args", B.ShortArgs),
                      ("attn_q_k_mx_args", B.KMxArgs), ("attn_q_prefill_mx_args", B.PrefillMxArgs)]:
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, (cname, f)


def _fake(n=16):
    return ctypes.c_void_p(0x10000 * n)  # aligned non-null placeholder; never dereferenced


def _kvq(**kw):
    a = B.KvqArgs(1, 2, 100, 128, 128, _fake(1), _fake(2), 1, B.GRAN_CHANNEL, B.GRAN_CHANNEL,
                  _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), None, _fake(8), B.PV_FP8, None, _fake(9),
                  1 << 20)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_kvq_validation():
    L = B.lib()
    call = lambda a: L.kv_quantize_i8(ctypes.byref(a), None)
    assert call(_kvq(k=None)) == B.E_NULL
    assert call(_kvq(seq_len=0)) == B.E_SHAPE
    assert call(_kvq(capacity=50)) == B.E_SHAPE
    assert call(_kvq(head_dim=96)) == B.E_UNSUPPORTED
    assert call(_kvq(k_gran=7)) == B.E_UNSUPPORTED
    assert call(_kvq(v_gran=B.GRAN_TENSOR)) == B.E_UNSUPPORTED
    assert call(_kvq(capacity=130)) == B.E_SHAPE                       # v_op needs capacity % 64
    assert call(_kvq(v_gran=B.GRAN_TOKEN)) == B.E_NULL                 # per-token operand: V_max header
    assert call(_kvq(v_gran=B.GRAN_TOKEN, v_scale_max=_fake(10), v_op_format=B.PV_INT8)) == B.E_UNSUPPORTED
    assert call(_kvq(v_gran=B.GRAN_TOKEN, v_scale_max=ctypes.c_void_p(0x10002))) == B.E_ALIGN
    assert call(_kvq(k_codes=ctypes.c_void_p(0x10001))) == B.E_ALIGN
    assert call(_kvq(workspace_bytes=8)) == B.E_WORKSPACE
    assert call(_kvq(workspace=None)) == B.E_WORKSPACE
    assert call(_kvq(k_sum=ctypes.c_void_p(0x10004))) == B.E_ALIGN      # int64 header
    assert call(_kvq(batch=256, kv_heads=256, capacity=64)) == B.E_SHAPE  # batch * kv_heads > 65535
    # V codes may be left out only beside a per-channel operand (a prefill-only cache)
    assert call(_kvq(v_codes=None, v_op=None)) == B.E_NULL
    assert call(_kvq(v_codes=None, v_gran=B.GRAN_TOKEN, v_scale_max=_fake(10))) == B.E_NULL
    if not B.torch.cuda.is_available():
        assert call(_kvq(v_codes=None)) == B.E_DEVICE          # valid: only the device check refuses
    # per-block K scales: one per 64 keys of the capacity
    assert call(_kvq(k_gran=B.GRAN_BLOCK, capacity=100, v_op=None)) == B.E_SHAPE
    a = _kvq()
    assert L.kv_quantize_i8_workspace_size(ctypes.byref(a)) == 2 * 128 * 20 + 2 * 8 + 256


def _vop(**kw):
    a = B.VopArgs(1, 2, 128, 1024, 1000, _fake(1), _fake(2), B.GRAN_TOKEN, _fake(3), B.PV_FP8, _fake(4))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_v_operand_validation():
    L = B.lib()
    call = lambda a: L.attn_q_v_operand(ctypes.byref(a), None)
    assert call(_vop(v_scale_max=None)) == B.E_NULL
    assert call(_vop(v_op=None)) == B.E_NULL
    assert call(_vop(n_keys=0)) == B.E_SHAPE
    assert call(_vop(n_keys=1025)) == B.E_SHAPE
    assert call(_vop(capacity=1000, n_keys=900)) == B.E_SHAPE          # capacity % 64
    assert call(_vop(head_dim=96)) == B.E_UNSUPPORTED
    assert call(_vop(v_op_format=B.PV_INT8)) == B.E_UNSUPPORTED         # per-token: e4m3 only
    assert call(_vop(v_gran=B.GRAN_TENSOR)) == B.E_UNSUPPORTED
    assert call(_vop(v_op=ctypes.c_void_p(0x10008))) == B.E_ALIGN
    if not B.torch.cuda.is_available():
        assert call(_vop()) == B.E_DEVICE
        assert call(_vop(v_gran=B.GRAN_CHANNEL, v_op_format=B.PV_INT8, v_scales=None, v_scale_max=None)) == B.E_DEVICE


def _app(**kw):
    a = B.KvAppendArgs(2, 4, 128, 1024, 1000, 1, _fake(1), _fake(2), _fake(3), _fake(4), _fake(5),
                       _fake(6), _fake(7), _fake(8), None, 0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_append_validation():
    L = B.lib()
    call = lambda a: L.attn_q_kv_append_i8(ctypes.byref(a), None)
    size = lambda a: L.attn_q_kv_append_i8_workspace_size(ctypes.byref(a))
    assert call(_app(k_sum=None)) == B.E_NULL
    assert call(_app(v_scales=None)) == B.E_NULL
    assert call(_app(new_tokens=25)) == B.E_SHAPE                        # 1000 + 25 > capacity
    assert call(_app(seq_len=-1)) == B.E_SHAPE
    assert call(_app(new_tokens=-1)) == B.E_SHAPE
    assert call(_app(head_dim=80)) == B.E_UNSUPPORTED
    assert call(_app(k_sum=ctypes.c_void_p(0x10004))) == B.E_ALIGN
    assert call(_app(k=ctypes.c_void_p(0x10008))) == B.E_ALIGN
    assert call(_app(k_scales=ctypes.c_void_p(0x10001))) == B.E_ALIGN
    # up to 64 new tokens need no workspace; more need one int64 per (b, g, 64-token chunk, channel)
    assert size(_app(new_tokens=64)) == 0
    assert size(_app(seq_len=0, new_tokens=65)) == 2 * 4 * 2 * 128 * 8
    assert call(_app(seq_len=0, new_tokens=65)) == B.E_WORKSPACE
    assert call(_app(seq_len=0, new_tokens=65, workspace=_fake(9), workspace_bytes=100)) == B.E_WORKSPACE
    # new_tokens == 0 is a valid no-op that returns before any HIP call, with any pointers
    assert call(_app(new_tokens=0, k=None, k_sum=None)) == B.OK


def _short(**kw):
    a = B.ShortArgs(8, 12, 197, 64, 0.0, _fake(1), _fake(2), _fake(3), _fake(4), B.OUT_F16, None)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_short_fused_validation():
    L = B.lib()
    call = lambda a: L.attn_q_short_fused(ctypes.byref(a), None)
    assert call(_short(q=None)) == B.E_NULL
    assert call(_short(out=None)) == B.E_NULL
    assert call(_short(seq_len=0)) == B.E_SHAPE
    assert call(_short(heads=0)) == B.E_SHAPE
    assert call(_short(seq_len=257)) == B.E_UNSUPPORTED      # one workgroup holds the head
    assert call(_short(head_dim=128)) == B.E_UNSUPPORTED
    assert call(_short(out_dtype=3)) == B.E_UNSUPPORTED
    assert call(_short(v=ctypes.c_void_p(0x10008))) == B.E_ALIGN
    assert call(_short(debug_s=ctypes.c_void_p(0x10002))) == B.E_ALIGN


def _pf(**kw):
    a = B.PrefillArgs(1, 4, 2, 128, 32, 100, 0, 0, 0.0, _fake(1), B.GRAN_TOKEN, _fake(2), _fake(3),
                      B.GRAN_CHANNEL, _fake(4), _fake(5), B.GRAN_CHANNEL, None, B.PV_FP8, 128, _fake(6),
                      B.OUT_F32, None, None, None, None, 0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_prefill_validation():
    L = B.lib()
    call = lambda a: L.attn_q_prefill(ctypes.byref(a), None)
    assert call(_pf(q=None)) == B.E_NULL
    assert call(_pf(q_heads=3)) == B.E_SHAPE
    assert call(_pf(kv_len=0)) == B.E_SHAPE
    assert call(_pf(capacity=64)) == B.E_SHAPE                          # < kv_len rounded up to 64
    assert call(_pf(causal=1, q_offset=80)) == B.E_SHAPE                 # q_offset + q_len > kv_len
    assert call(_pf(k_gran=7)) == B.E_UNSUPPORTED
    assert call(_pf(k_gran=B.GRAN_TOKEN, pv_mode=B.PV_SPLIT24)) == B.E_UNSUPPORTED
    assert call(_pf(pv_mode=5)) == B.E_UNSUPPORTED
    assert call(_pf(out_dtype=9)) == B.E_UNSUPPORTED
    assert call(_pf(head_dim=32)) == B.E_UNSUPPORTED
    assert call(_pf(v_op=ctypes.c_void_p(0x10010))) == B.E_ALIGN        # needs 32-byte alignment
    assert call(_pf(q_gran=B.GRAN_TENSOR)) == B.E_WORKSPACE
    assert L.attn_q_prefill_workspace_size(ctypes.byref(_pf())) == 0
    assert L.attn_q_prefill_workspace_size(ctypes.byref(_pf(q_gran=B.GRAN_TENSOR))) == 256
    # the precision mode takes per-row Q scales and no score export
    assert call(_pf(pv_mode=B.PV_SPLIT24, q_gran=B.GRAN_TENSOR, workspace=_fake(7), workspace_bytes=256)) \
        == B.E_UNSUPPORTED
    assert call(_pf(pv_mode=B.PV_SPLIT24, debug_s=_fake(8))) == B.E_UNSUPPORTED
    assert call(_pf(pv_mode=3)) == B.E_UNSUPPORTED
    assert call(_pf(pv_mode=B.PV_SPLIT24, lse=_fake(9))) == B.E_UNSUPPORTED
    # per-block K: fp8 / int8 P·V only; per-block Q needs its scale workspace
    assert call(_pf(pv_mode=B.PV_SPLIT24, k_gran=B.GRAN_BLOCK)) == B.E_UNSUPPORTED
    assert call(_pf(q_gran=B.GRAN_BLOCK)) == B.E_WORKSPACE
    assert L.attn_q_prefill_workspace_size(ctypes.byref(_pf(q_gran=B.GRAN_BLOCK))) == 256  # 4 heads x 1 block
    assert L.attn_q_prefill_workspace_size(ctypes.byref(_pf(q_gran=B.GRAN_BLOCK, batch=3, q_heads=8,
                                                            kv_heads=2, q_len=1000))) == 3 * 8 * 16 * 4
    assert call(_pf(q_gran=B.GRAN_BLOCK, workspace=_fake(7), workspace_bytes=128)) == B.E_WORKSPACE
    assert call(_pf(q_gran=B.GRAN_BLOCK, workspace=ctypes.c_void_p(0x10008), workspace_bytes=256)) == B.E_ALIGN
    assert call(_pf(q_gran=5)) == B.E_UNSUPPORTED
    # per-token V: the e4m3 operand only, and the V_max header is required
    assert call(_pf(v_gran=B.GRAN_TENSOR)) == B.E_UNSUPPORTED
    assert call(_pf(v_gran=B.GRAN_TOKEN, pv_mode=B.PV_INT8, v_scale_max=_fake(10))) == B.E_UNSUPPORTED
    assert call(_pf(v_gran=B.GRAN_TOKEN, v_scales=None)) == B.E_NULL
    assert call(_pf(v_scales=None)) == B.E_NULL
    assert call(_pf(lse=ctypes.c_void_p(0x10002))) == B.E_ALIGN
    # q_len == 0 is a valid no-op that returns before any HIP call
    assert call(_pf(q_len=0)) == B.OK
    assert call(_pf(q_len=0, pv_mode=B.PV_SPLIT24)) == B.OK


def _dec(**kw):
    a = B.DecodeArgs(1, 16, 4, 128, 1000, 1024, None, 0.0, _fake(1), _fake(2), _fake(3), B.GRAN_TOKEN,
                     _fake(4), _fake(5), B.GRAN_TOKEN, _fake(6), B.OUT_F32, None, _fake(7), 1 << 24)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_validation():
    L = B.lib()
    call = lambda a: L.attn_q_decode(ctypes.byref(a), None)
    assert call(_dec(v_codes=None)) == B.E_NULL
    assert call(_dec(q_heads=12, kv_heads=1)) == B.E_UNSUPPORTED          # G must be 1, 2, 4 or 8
    assert call(_dec(q_heads=10)) == B.E_SHAPE
    assert call(_dec(capacity=999)) == B.E_SHAPE
    assert call(_dec(k_gran=B.GRAN_TENSOR)) == B.E_UNSUPPORTED
    assert call(_dec(k_gran=B.GRAN_BLOCK, capacity=1000)) == B.E_SHAPE   # a scale per 64 keys
    assert call(_dec(workspace_bytes=100)) == B.E_WORKSPACE
    assert call(_dec(workspace=ctypes.c_void_p(0x10010))) == B.E_ALIGN
    assert call(_dec(kv_lens=ctypes.c_void_p(0x10002))) == B.E_ALIGN
    n = L.attn_q_decode_workspace_size(ctypes.byref(_dec()))
    assert 0 < n < (1 << 24)


def test_decode_noalloc_validation():
    """The no-allocation decode ignores the workspace fields and refuses, before any HIP call,
    a call whose split partials exceed its static scratch (8 MiB)."""
    L = B.lib()
    call = lambda a: L.attn_q_decode_noalloc(ctypes.byref(a), None)
    assert call(_dec(v_codes=None)) == B.E_NULL
    assert call(_dec(q_heads=10)) == B.E_SHAPE
    # 16 heads x 2048 splits x (4 * 128 + 8) bytes > 8 MiB
    assert call(_dec(kv_len=1 << 20, capacity=1 << 20, workspace=None, workspace_bytes=0)) == B.E_SCRATCH
    assert L.attn_q_decode_workspace_size(ctypes.byref(_dec(kv_len=1 << 20, capacity=1 << 20))) > (8 << 20)
    if not B.torch.cuda.is_available():   # valid arguments and no workspace: only the device check refuses
        assert call(_dec(workspace=None, workspace_bytes=0)) == B.E_DEVICE


def test_binding_rejects_bad_tensors_before_the_library():
    """dtype / shape / rank errors raise in the binding; nothing reaches the C ABI."""
    import torch
    cache = B.alloc_cache(1, 2, 64, 128, B.GRAN_CHANNEL, B.GRAN_CHANNEL, "cpu")
    q = torch.zeros((1, 4, 8, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        B.attn_q_prefill(q.float(), cache, kv_len=64)
    with pytest.raises(ValueError):
        B.attn_q_prefill(q, cache, kv_len=64, out=torch.empty((1, 4, 7, 128)))
    with pytest.raises(ValueError):
        B.attn_q_prefill(q, cache, kv_len=64, out=torch.empty((1, 4, 8, 128), dtype=torch.int32))
    with pytest.raises(ValueError):
        B.attn_q_decode(q, cache, kv_len=64)                       # decode takes [B][Hq][d]
    with pytest.raises(ValueError):
        B.attn_q_decode(q[:, :, 0], cache, kv_len=64, out=torch.empty((1, 4, 64)))
    k = torch.zeros((1, 2, 64, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        B.kv_quantize_i8(k, k[:, :, :32], cache)                   # v shape differs from k
    with pytest.raises(ValueError):
        B.kv_quantize_i8(k.float(), k, cache)
    tok = B.alloc_cache(1, 2, 64, 128, B.GRAN_TOKEN, B.GRAN_TOKEN, "cpu", v_op_format=None, header=True)
    with pytest.raises(ValueError):
        B.attn_q_kv_append_i8(k[:, :, :1], k[:, :, :1], cache)        # per-channel cache
    with pytest.raises(ValueError):
        B.attn_q_kv_append_i8(k[:, :, :1], k[:, :, :2], tok)          # v shape differs from k
    with pytest.raises(ValueError):
        B.attn_q_kv_append_i8(k[:, :, :1].float(), k[:, :, :1].float(), tok)
    with pytest.raises(ValueError):                                  # int8-operand mode on an e4m3 cache
        B.attn_q_prefill(q, cache, kv_len=64, pv_mode=B.PV_SPLIT24)
    with pytest.raises(ValueError):
        B.attn_q_short_fused(q, q, q[:, :, :4])                        # k, v shapes differ from q
    no_header = B.alloc_cache(1, 2, 64, 128, B.GRAN_TOKEN, B.GRAN_TOKEN, "cpu", v_op_format=None)
    with pytest.raises(ValueError):
        B.attn_q_kv_append_i8(k[:, :, :1], k[:, :, :1], no_header)


def _dec_app():
    d = B.DecodeArgs(1, 16, 4, 128, 1001, 1024, None, 0.0, _fake(1), _fake(2), _fake(3), B.GRAN_TOKEN,
                     _fake(4), _fake(5), B.GRAN_TOKEN, _fake(6), B.OUT_F32, None, _fake(7), 1 << 24)
    a = B.KvAppendArgs(1, 4, 128, 1024, 1000, 1, _fake(11), _fake(12), _fake(13), _fake(2), _fake(4),
                       _fake(3), _fake(5), _fake(14), None, 0)
    return d, a


def test_decode_append_validation():
    """The fused step checks both argument blocks and that they describe one cache and one new
    token at its last row, before any HIP call."""
    L = B.lib()

    def call(dkw=None, akw=None):
        d, a = _dec_app()
        for k, v in (dkw or {}).items():
            setattr(d, k, v)
        for k, v in (akw or {}).items():
            setattr(a, k, v)
        return L.attn_q_decode_append(ctypes.byref(d), ctypes.byref(a), None)

    assert call(akw=dict(k_sum=None)) == B.E_NULL
    assert call(dkw=dict(q=None)) == B.E_NULL
    assert call(akw=dict(new_tokens=2)) == B.E_SHAPE            # one token only
    assert call(akw=dict(seq_len=999)) == B.E_SHAPE             # not the decode's last row
    assert call(akw=dict(capacity=2048)) == B.E_SHAPE
    assert call(akw=dict(kv_heads=2)) == B.E_SHAPE
    assert call(akw=dict(k_codes=_fake(20))) == B.E_SHAPE       # another cache
    assert call(akw=dict(v_scales=_fake(21))) == B.E_SHAPE
    assert call(dkw=dict(k_gran=B.GRAN_CHANNEL)) == B.E_UNSUPPORTED
    assert call(dkw=dict(kv_lens=_fake(30))) == B.E_SHAPE        # one length for the fused step
    # consistent arguments pass validation; without a GPU the device check then refuses
    if not B.torch.cuda.is_available():
        assert call() == B.E_DEVICE


def _kmx(**kw):
    a = B.KMxArgs(1, 2, 100, 128, 128, B.MX_FP4, _fake(1), _fake(2), _fake(3), _fake(4))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _pmx(**kw):
    a = B.PrefillMxArgs(1, 4, 2, 128, 32, 100, 68, 1, 0.0, _fake(1), B.MX_FP6, _fake(2), _fake(3), B.MX_FP4, 128,
                        _fake(4), _fake(5), _fake(6), B.OUT_F32, None)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_mx_validation():
    L = B.lib()
    kq = lambda a: L.attn_q_k_quantize_mx(ctypes.byref(a), None)
    assert kq(_kmx(k=None)) == B.E_NULL
    assert kq(_kmx(k_mean=None)) == B.E_NULL
    assert kq(_kmx(seq_len=0)) == B.E_SHAPE
    assert kq(_kmx(capacity=99)) == B.E_SHAPE
    assert kq(_kmx(fmt=0)) == B.E_UNSUPPORTED          # e4m3 is not an MX element type here
    assert kq(_kmx(fmt=3)) == B.E_UNSUPPORTED
    assert kq(_kmx(head_dim=96)) == B.E_UNSUPPORTED
    assert kq(_kmx(k_mx=ctypes.c_void_p(0x10008))) == B.E_ALIGN
    pf = lambda a: L.attn_q_prefill_mx(ctypes.byref(a), None)
    assert pf(_pmx(q=None)) == B.E_NULL
    assert pf(_pmx(v_scales=None)) == B.E_NULL
    assert pf(_pmx(q_heads=3)) == B.E_SHAPE
    assert pf(_pmx(capacity=100)) == B.E_SHAPE                  # not a multiple of 64
    assert pf(_pmx(capacity=64)) == B.E_SHAPE                   # < kv_len
    assert pf(_pmx(q_offset=69)) == B.E_SHAPE                   # causal: q_offset + q_len > kv_len
    assert pf(_pmx(q_fmt=1)) == B.E_UNSUPPORTED
    assert pf(_pmx(k_fmt=0)) == B.E_UNSUPPORTED
    assert pf(_pmx(head_dim=32)) == B.E_UNSUPPORTED
    assert pf(_pmx(out_dtype=7)) == B.E_UNSUPPORTED
    assert pf(_pmx(v_op=ctypes.c_void_p(0x10010))) == B.E_ALIGN   # 32-byte alignment
    assert pf(_pmx(debug_s=ctypes.c_void_p(0x10002))) == B.E_ALIGN
    assert pf(_pmx(batch=1 << 16, q_heads=256, kv_heads=256, q_len=1 << 16, kv_len=1 << 16, causal=0,
                   capacity=1 << 16)) == B.E_SHAPE                                # grid
    assert pf(_pmx(q_len=0)) == B.OK                             # no-op before any HIP call
    if not B.torch.cuda.is_available():
        assert kq(_kmx()) == B.E_DEVICE
        assert pf(_pmx()) == B.E_DEVICE

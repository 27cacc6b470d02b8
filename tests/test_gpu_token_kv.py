"""GPU parity of the per-token K and V paths of the prefill and of the V-operand builder:
kv_quantize_i8 with per-token V writes the e4m3 operand carrying s_V[n] * c_V and the V_max
header; attn_q_v_operand rebuilds both from the codes (after appends); attn_q_prefill reads
per-token K scales (one dequantization constant per key) and per-token V operands.  Bars:
codes, scales, operand bytes and header bit-exact; int32 scores bit-exact; outputs within
1e-3 (row-normalised) of the oracle's emulation; cosine >= 0.999 against fp64."""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def rel_err(a, e):
    a = np.asarray(a, np.float64).reshape(-1, a.shape[-1])
    e = np.asarray(e, np.float64).reshape(-1, e.shape[-1])
    return float(np.max(np.abs(a - e) / np.maximum(np.abs(e).max(axis=1, keepdims=True), 1e-30)))


def cosine(a, e):
    a, e = np.asarray(a, np.float64).ravel(), np.asarray(e, np.float64).ravel()
    return float(a @ e / np.sqrt((a @ a) * (e @ e)))


def both_caches(c, kg, vg, cap=None):
    Bn, H, N, D = c.k.shape
    cap = cap or (N + 63) // 64 * 64
    g = B.alloc_cache(Bn, H, cap, D, kg, vg, DEV, v_op_format=B.PV_FP8)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    o = oracle.kv_quantize(c.k, c.v, kg, vg, capacity=cap, v_op_format=oracle.PV_FP8)
    torch.cuda.synchronize()
    return g, o


def check_operand(g, o):
    assert np.array_equal(g.v_op.cpu().numpy(), o.v_op)
    if o.v_scale_max is not None:
        assert np.array_equal(g.v_scale_max.cpu().numpy().view(np.uint32), o.v_scale_max.view(np.uint32))


CASES = [
    # (name, inputs, k_gran, v_gran)
    ("ktok_vtok_causal", lambda: inputs.small_case(101, hq=8, hkv=2, q_len=150, kv_len=1000, causal=True),
     B.GRAN_TOKEN, B.GRAN_TOKEN),
    ("ktok_vchan_b2", lambda: inputs.small_case(102, batch=2, hq=4, hkv=2, q_len=70, kv_len=333),
     B.GRAN_TOKEN, B.GRAN_CHANNEL),
    ("kchan_vtok_d64", lambda: inputs.small_case(103, hq=4, hkv=1, q_len=90, kv_len=700, d=64, causal=True),
     B.GRAN_CHANNEL, B.GRAN_TOKEN),
    ("ktok_vtok_gqa8_many_tiles", lambda: inputs.small_case(104, hq=8, hkv=1, q_len=64, kv_len=2900, causal=True),
     B.GRAN_TOKEN, B.GRAN_TOKEN),
]


@pytest.mark.parametrize("name,make,kg,vg", CASES, ids=[c[0] for c in CASES])
def test_token_kv_prefill_matches_emulation(name, make, kg, vg):
    c = make()
    Bn, Hq, L, D = c.q.shape
    N = c.k.shape[2]
    print(f"  token prefill {name} shape={c.shape}", flush=True)
    g, o = both_caches(c, kg, vg)
    check_operand(g, o)
    dbg = torch.full((Bn, Hq, L, N), -(2 ** 31), dtype=torch.int32, device=DEV)
    dp = torch.zeros((Bn, Hq, L, N), dtype=torch.uint8, device=DEV)
    B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=c.causal, out_dtype=B.OUT_F32,
                     debug_s=dbg, debug_p=dp)
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=c.causal, out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=c.causal, want_s=True, want_p=True)
    vis = np.ones((L, N), bool)
    if c.causal:
        vis = np.arange(N)[None, :] <= (c.q_offset + np.arange(L))[:, None]
    vis = np.broadcast_to(vis, dbg.shape)
    s = dbg.cpu().numpy()
    assert np.array_equal(s[vis], ref.s_i32[vis])
    pm = int(np.sum(dp.cpu().numpy()[vis] != ref.p_codes[vis]))
    err = rel_err(out.cpu().numpy(), ref.out)
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=c.causal, q_offset=c.q_offset)
    cs = cosine(out.cpu().numpy(), exact)
    print(f"    err vs emulation {err:.2e}, P-code mismatches {pm} of {int(vis.sum())}, cos vs fp64 {cs:.6f}",
          flush=True)
    assert err <= TOL
    assert pm <= max(1, int(vis.sum()) // 10000)
    assert cs >= 0.999


def test_v_operand_rebuild_matches_quantize():
    """attn_q_v_operand over the keys kv_quantize_i8 wrote reproduces its operand and header
    (per-token and per-channel V), and over fewer keys zero-fills the tail tiles as the oracle."""
    for vg in (B.GRAN_TOKEN, B.GRAN_CHANNEL):
        c = inputs.small_case(105, hq=4, hkv=2, q_len=1, kv_len=450)
        g, o = both_caches(c, B.GRAN_TOKEN, vg, cap=512)
        before = g.v_op.clone()
        g.v_op.fill_(0x5A)
        B.attn_q_v_operand(g, n_keys=450)
        torch.cuda.synchronize()
        assert torch.equal(g.v_op, before)
        check_operand(g, o)
        B.attn_q_v_operand(g, n_keys=130)
        oracle.v_operand(o, 130)
        torch.cuda.synchronize()
        check_operand(g, o)


def test_appended_cache_runs_through_the_prefill():
    """The decode-time cache (prompt quantized with per-token K and V scales, then grown by
    attn_q_kv_append_i8 with the running K mean) brought to the prefill: attn_q_v_operand
    rebuilds the e4m3 operand and V_max over all keys, then the next chunk of 200 queries
    attends causally over the 3000 keys.  The oracle runs the same sequence on its own cache."""
    N, P, T = 3000, 2500, 300
    c = inputs.small_case(106, hq=8, hkv=2, q_len=200, kv_len=N, causal=True)
    cap = 3008
    g = B.alloc_cache(1, 2, cap, 128, B.GRAN_TOKEN, B.GRAN_TOKEN, DEV, v_op_format=B.PV_FP8, header=True)
    B.kv_quantize_i8(dev(c.k[:, :, :P]), dev(c.v[:, :, :P]), g)
    S = np.zeros((1, 2, 128), np.int64)
    o = oracle.kv_quantize(np.ascontiguousarray(c.k[:, :, :P]), np.ascontiguousarray(c.v[:, :, :P]),
                           oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, capacity=cap, k_sum=S, v_op_format=oracle.PV_FP8)
    for a, b in ((P, P + T), (P + T, N)):
        B.attn_q_kv_append_i8(dev(c.k[:, :, a:b]), dev(c.v[:, :, a:b]), g)
        oracle.kv_append(np.ascontiguousarray(c.k[:, :, a:b]), np.ascontiguousarray(c.v[:, :, a:b]), o, S)
    B.attn_q_v_operand(g, n_keys=N)
    oracle.v_operand(o, N)
    torch.cuda.synchronize()
    assert np.array_equal(g.k_codes.cpu().numpy()[:, :, :N], o.k_codes[:, :, :N])
    assert np.array_equal(g.k_sum.cpu().numpy(), S)
    check_operand(g, o)
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=True, out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=True)
    err = rel_err(out.cpu().numpy(), ref.out)
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=True, q_offset=c.q_offset)
    cs = cosine(out.cpu().numpy(), exact)
    print(f"  appended cache through the prefill: err vs emulation {err:.2e}, cos vs fp64 {cs:.6f}", flush=True)
    assert err <= TOL
    assert cs >= 0.999

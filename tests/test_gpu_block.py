"""GPU parity of the BLOCK granularity (one fp32 scale per block of 64 tokens of a (batch, head),
QFlash section 3.3's per-block quantization with the blocks of its tiled loop): kv_quantize_i8
with per-block K scales, attn_q_prefill with per-block K (one dequantization constant per key
tile) and per-block Q scales, attn_q_decode with per-block K.  Bars: codes and scales
bit-exact; int32 scores bit-exact; P codes equal the emulation's; outputs within 1e-3
(row-normalised) of the oracle's emulation; cosine >= 0.999 against fp64."""
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


def caches(c, vg, cap=None, fmt=B.PV_FP8):
    Bn, H, N, D = c.k.shape
    cap = cap or (N + 63) // 64 * 64
    g = B.alloc_cache(Bn, H, cap, D, B.GRAN_BLOCK, vg, DEV, v_op_format=fmt)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    o = oracle.kv_quantize(c.k, c.v, oracle.GRAN_BLOCK, vg, capacity=cap,
                           v_op_format=None if fmt is None else oracle.PV_FP8)
    torch.cuda.synchronize()
    return g, o


QUANT_CASES = [
    ("b1_h4_n300_cap384", lambda: inputs.small_case(201, hq=4, hkv=4, q_len=1, kv_len=300), 384, B.GRAN_CHANNEL),
    ("b2_h2_n1000_d64_vtok", lambda: inputs.small_case(202, batch=2, hq=2, hkv=2, q_len=1, kv_len=1000, d=64), 1024,
     B.GRAN_TOKEN),
    ("b1_h1_n64_exact_block", lambda: inputs.small_case(203, hq=1, hkv=1, q_len=1, kv_len=64), 64, B.GRAN_CHANNEL),
]


@pytest.mark.parametrize("name,make,cap,vg", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_block_kv_quantize_bit_exact(name, make, cap, vg):
    c = make()
    N = c.k.shape[2]
    print(f"  block kv_quantize {name}", flush=True)
    g, o = caches(c, vg, cap=cap)
    nb = (N + 63) // 64
    assert np.array_equal(g.k_codes.cpu().numpy()[:, :, :N], o.k_codes[:, :, :N])
    assert np.array_equal(g.k_scales.cpu().numpy()[:, :, :nb].view(np.uint32), o.k_scales[:, :, :nb].view(np.uint32))
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), o.k_mean.view(np.uint32))
    assert np.array_equal(g.v_codes.cpu().numpy()[:, :, :N], o.v_codes[:, :, :N])
    assert np.array_equal(g.v_op.cpu().numpy(), o.v_op)
    if o.v_scale_max is not None:
        assert np.array_equal(g.v_scale_max.cpu().numpy().view(np.uint32), o.v_scale_max.view(np.uint32))


PREFILL_CASES = [
    # (name, inputs, q_gran, v_gran)
    ("kblk_qtok_gqa4_causal", lambda: inputs.small_case(211, hq=8, hkv=2, q_len=150, kv_len=1000, causal=True),
     B.GRAN_TOKEN, B.GRAN_CHANNEL),
    ("kblk_qblk_b2_ragged", lambda: inputs.small_case(212, batch=2, hq=4, hkv=2, q_len=77, kv_len=333),
     B.GRAN_BLOCK, B.GRAN_CHANNEL),
    ("kblk_qblk_vtok_many_tiles", lambda: inputs.small_case(213, hq=8, hkv=1, q_len=130, kv_len=2900, causal=True),
     B.GRAN_BLOCK, B.GRAN_TOKEN),
    ("kblk_qtensor_d64", lambda: inputs.small_case(214, hq=4, hkv=1, q_len=90, kv_len=700, d=64, causal=True),
     B.GRAN_TENSOR, B.GRAN_CHANNEL),
]


@pytest.mark.parametrize("name,make,qg,vg", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_block_prefill_matches_emulation(name, make, qg, vg):
    c = make()
    Bn, Hq, L, D = c.q.shape
    N = c.k.shape[2]
    print(f"  block prefill {name} shape={c.shape}", flush=True)
    g, o = caches(c, vg)
    dbg = torch.full((Bn, Hq, L, N), -(2 ** 31), dtype=torch.int32, device=DEV)
    dp = torch.zeros((Bn, Hq, L, N), dtype=torch.uint8, device=DEV)
    B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=c.causal, q_gran=qg, out_dtype=B.OUT_F32,
                     debug_s=dbg, debug_p=dp)
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=c.causal, q_gran=qg,
                           out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=c.causal, q_gran=qg,
                                 want_s=True, want_p=True)
    vis = np.ones((L, N), bool)
    if c.causal:
        vis = np.arange(N)[None, :] <= (c.q_offset + np.arange(L))[:, None]
    vis = np.broadcast_to(vis, dbg.shape)
    assert np.array_equal(dbg.cpu().numpy()[vis], ref.s_i32[vis])
    pm = int(np.sum(dp.cpu().numpy()[vis] != ref.p_codes[vis]))
    err = rel_err(out.cpu().numpy(), ref.out)
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=c.causal, q_offset=c.q_offset)
    cs = cosine(out.cpu().numpy(), exact)
    print(f"    err vs emulation {err:.2e}, P-code mismatches {pm} of {int(vis.sum())}, cos vs fp64 {cs:.6f}",
          flush=True)
    assert err <= TOL
    assert pm <= max(1, int(vis.sum()) // 10000)
    assert cs >= 0.999


@pytest.mark.parametrize("vg", [B.GRAN_CHANNEL, B.GRAN_TOKEN])
def test_block_decode_matches_emulation(vg):
    c = inputs.config4(kv_len=2000)[0]
    N = 2000
    print(f"  block decode v_gran={vg}", flush=True)
    g, o = caches(c, vg, cap=2048, fmt=None)
    Bn = c.k.shape[0]
    q = c.q[:, :, 0]
    dbg = torch.zeros((Bn, q.shape[1], N), dtype=torch.int32, device=DEV)
    out = B.attn_q_decode(dev(q), g, kv_len=N, out_dtype=B.OUT_F32, debug_qk=dbg)
    torch.cuda.synchronize()
    assert np.array_equal(g.k_codes.cpu().numpy()[:, :, :N], o.k_codes[:, :, :N])
    ref, rdots = oracle.decode_emulate(q, o, kv_len=N, want_qk=True)
    assert np.array_equal(dbg.cpu().numpy(), rdots)
    err = rel_err(out.cpu().numpy(), ref)
    print(f"    err vs emulation {err:.2e}", flush=True)
    assert err <= TOL

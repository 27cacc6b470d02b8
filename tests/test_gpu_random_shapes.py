"""Seeded sweep of shapes against the oracle: batch, query / kv heads (G = 1, 2, 4, 8), head
dimension, query and key lengths (ragged, below one tile and across many), causal offsets
(from 0, inside, at the end) and the granularities, for the prefill (int8 Q/K, and MX fp4 /
fp6 Q/K), the decode and kv_quantize.  Bars as the parity tests: codes bit-exact, int32
scores bit-exact, outputs within 1e-3 (row-normalised) of the emulation."""
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


def draw(seed):
    r = np.random.default_rng(seed)
    G = int(r.choice([1, 2, 4, 8]))
    hkv = int(r.choice([1, 2]))
    d = int(r.choice([64, 128]))
    batch = int(r.choice([1, 2]))
    kv_len = int(r.choice([1, 37, 64, 65, 130, 511, 1500]))
    causal = bool(r.integers(0, 2))
    q_len = int(r.integers(1, min(kv_len, 300) + 1)) if causal else int(r.integers(1, 300))
    if causal:
        q_offset = int(r.choice([0, kv_len - q_len, (kv_len - q_len) // 2]))
    else:
        q_offset = 0
    kg = int(r.choice([B.GRAN_CHANNEL, B.GRAN_TOKEN, B.GRAN_BLOCK]))
    vg = int(r.choice([B.GRAN_CHANNEL, B.GRAN_TOKEN]))
    qg = int(r.choice([B.GRAN_TOKEN, B.GRAN_BLOCK, B.GRAN_TENSOR]))
    return dict(G=G, hkv=hkv, d=d, batch=batch, kv_len=kv_len, q_len=q_len, causal=causal, q_offset=q_offset,
                kg=kg, vg=vg, qg=qg)


SEEDS = list(range(1000, 1016))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_prefill_decode(seed):
    p = draw(seed)
    print(f"  seed {seed}: {p}", flush=True)
    c = inputs.small_case(seed, batch=p["batch"], hq=p["G"] * p["hkv"], hkv=p["hkv"], q_len=p["q_len"],
                          kv_len=p["kv_len"], d=p["d"], causal=p["causal"], q_offset=p["q_offset"])
    Bn, Hq, L, D = c.q.shape
    N = p["kv_len"]
    cap = (N + 63) // 64 * 64
    g = B.alloc_cache(Bn, p["hkv"], cap, D, p["kg"], p["vg"], DEV, v_op_format=B.PV_FP8)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    o = oracle.kv_quantize(c.k, c.v, p["kg"], p["vg"], capacity=cap, v_op_format=oracle.PV_FP8)
    torch.cuda.synchronize()
    assert np.array_equal(g.k_codes.cpu().numpy()[:, :, :N], o.k_codes[:, :, :N])
    assert np.array_equal(g.v_codes.cpu().numpy()[:, :, :N], o.v_codes[:, :, :N])
    assert np.array_equal(g.v_op.cpu().numpy(), o.v_op)
    qg = p["qg"]
    if p["kg"] == B.GRAN_TOKEN and qg == B.GRAN_TENSOR:
        qg = B.GRAN_TOKEN
    dbg = torch.full((Bn, Hq, L, N), -(2 ** 31), dtype=torch.int32, device=DEV)
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=c.causal, q_gran=qg,
                           out_dtype=B.OUT_F32, debug_s=dbg)
    torch.cuda.synchronize()
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=c.causal, q_gran=qg, want_s=True)
    vis = np.ones((L, N), bool)
    if c.causal:
        vis = np.arange(N)[None, :] <= (c.q_offset + np.arange(L))[:, None]
    vis = np.broadcast_to(vis, dbg.shape)
    assert np.array_equal(dbg.cpu().numpy()[vis], ref.s_i32[vis])
    err = rel_err(out.cpu().numpy(), ref.out)
    # the decode of the last query against the same cache (its K granularity must be a key one)
    derr = float("nan")
    if p["kg"] in (B.GRAN_TOKEN, B.GRAN_CHANNEL, B.GRAN_BLOCK):
        q1 = np.ascontiguousarray(c.q[:, :, -1])
        dout = B.attn_q_decode(dev(q1), g, kv_len=N, out_dtype=B.OUT_F32)
        torch.cuda.synchronize()
        dref, _ = oracle.decode_emulate(q1, o, kv_len=N)
        derr = rel_err(dout.cpu().numpy(), dref)
    print(f"    prefill err {err:.2e}, decode err {derr:.2e}", flush=True)
    assert err <= TOL
    assert not derr > TOL


@pytest.mark.parametrize("seed", SEEDS[:8])
def test_random_shape_mx_prefill(seed):
    p = draw(seed)
    r = np.random.default_rng(seed + 7)
    qf, kf = int(r.choice([B.MX_FP4, B.MX_FP6])), int(r.choice([B.MX_FP4, B.MX_FP6]))
    print(f"  seed {seed}: {p} q_fmt {qf} k_fmt {kf}", flush=True)
    c = inputs.small_case(seed, batch=p["batch"], hq=p["G"] * p["hkv"], hkv=p["hkv"], q_len=p["q_len"],
                          kv_len=p["kv_len"], d=p["d"], causal=p["causal"], q_offset=p["q_offset"])
    Bn, Hq, L, D = c.q.shape
    N = p["kv_len"]
    cap = (N + 63) // 64 * 64
    g = B.alloc_cache(Bn, p["hkv"], cap, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, DEV, v_op_format=B.PV_FP8)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    keys = B.attn_q_k_quantize_mx(dev(c.k), g.k_mean, B.alloc_mx_keys(Bn, p["hkv"], cap, D, kf, DEV))
    out = B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=N, q_fmt=qf, q_offset=c.q_offset, causal=c.causal,
                              out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    ofmt = {B.MX_FP4: oracle.LB_MXFP4, B.MX_FP6: oracle.LB_MXFP6}
    o = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, capacity=cap, v_op_format=oracle.PV_FP8)
    kenc = oracle.k_quantize_mx(c.k, o.k_mean, ofmt[kf], capacity=cap)
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=c.causal,
                                 mx=oracle.mx_operands(c.q, ofmt[qf], kenc))
    err = rel_err(out.cpu().numpy(), ref.out)
    print(f"    MX prefill err {err:.2e}", flush=True)
    assert err <= TOL

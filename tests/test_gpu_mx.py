"""GPU parity of the MX path (Q and K below 8 bits on the scaled fp6 / fp4 matrix cores):
attn_q_k_quantize_mx codes and E8M0 scales bit-exact against the oracle's encoding;
attn_q_prefill_mx scores within fp32 accumulation error of the oracle's (the dots of the
dequantized values rounded once), outputs within 1e-3 (row-normalised) of the oracle's
emulation with MX scores (two key streams, as the int8 path), and cosine >= 0.999 against the fp64 grid
study (attention over the same dequantized Q and K)."""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-3
ORA_FMT = {B.MX_FP4: oracle.LB_MXFP4, B.MX_FP6: oracle.LB_MXFP6}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def unpack(codes: np.ndarray, fmt: int) -> np.ndarray:
    """Packed rows (element c at bits [bits*c, bits*c + bits), little-endian) -> one code per element."""
    b = codes.astype(np.uint32)
    if fmt == B.MX_FP4:
        out = np.stack([b & 15, b >> 4], axis=-1)
        return out.reshape(codes.shape[:-1] + (codes.shape[-1] * 2,)).astype(np.uint8)
    t = b.reshape(codes.shape[:-1] + (codes.shape[-1] // 3, 3))
    v = t[..., 0] | (t[..., 1] << 8) | (t[..., 2] << 16)
    out = np.stack([(v >> (6 * i)) & 63 for i in range(4)], axis=-1)
    return out.reshape(codes.shape[:-1] + (codes.shape[-1] // 3 * 4,)).astype(np.uint8)


def rel_err(a, e):
    a = np.asarray(a, np.float64).reshape(-1, a.shape[-1])
    e = np.asarray(e, np.float64).reshape(-1, e.shape[-1])
    return float(np.max(np.abs(a - e) / np.maximum(np.abs(e).max(axis=1, keepdims=True), 1e-30)))


def cosine(a, e):
    a, e = np.asarray(a, np.float64).ravel(), np.asarray(e, np.float64).ravel()
    return float(a @ e / np.sqrt((a @ a) * (e @ e)))


def caches(c, kfmt, cap=None):
    Bn, H, N, D = c.k.shape
    cap = cap or (N + 63) // 64 * 64
    g = B.alloc_cache(Bn, H, cap, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, DEV, v_op_format=B.PV_FP8)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    keys = B.attn_q_k_quantize_mx(dev(c.k), g.k_mean, B.alloc_mx_keys(Bn, H, cap, D, kfmt, DEV))
    o = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, capacity=cap,
                           v_op_format=oracle.PV_FP8)
    kenc = oracle.k_quantize_mx(c.k, o.k_mean, ORA_FMT[kfmt], capacity=cap)
    torch.cuda.synchronize()
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), o.k_mean.view(np.uint32))
    return g, keys, o, kenc


ENC_CASES = [
    ("fp4_d128_ragged", B.MX_FP4, lambda: inputs.small_case(301, hq=2, hkv=2, q_len=1, kv_len=333)),
    ("fp6_d128_ragged", B.MX_FP6, lambda: inputs.small_case(302, hq=2, hkv=2, q_len=1, kv_len=333)),
    ("fp4_d64_b2", B.MX_FP4, lambda: inputs.small_case(303, batch=2, hq=1, hkv=1, q_len=1, kv_len=200, d=64)),
    ("fp6_d64_b2", B.MX_FP6, lambda: inputs.small_case(304, batch=2, hq=1, hkv=1, q_len=1, kv_len=200, d=64)),
    ("fp6_outlier_channels", B.MX_FP6, lambda: inputs.config1()),
]


@pytest.mark.parametrize("name,fmt,make", ENC_CASES, ids=[c[0] for c in ENC_CASES])
def test_k_quantize_mx_bit_exact(name, fmt, make):
    c = make()
    N = c.k.shape[2]
    print(f"  k_quantize_mx {name}", flush=True)
    g, keys, o, kenc = caches(c, fmt)
    got = unpack(keys.codes.cpu().numpy(), fmt)
    assert np.array_equal(got[:, :, :N], kenc.codes[:, :, :N])
    assert np.array_equal(keys.scales.cpu().numpy()[:, :, :N], kenc.scale_bytes[:, :, :N])


PREFILL_CASES = [
    # (name, inputs, q_fmt, k_fmt)
    ("fp4_fp4_gqa4_causal", lambda: inputs.small_case(311, hq=8, hkv=2, q_len=150, kv_len=1000, causal=True),
     B.MX_FP4, B.MX_FP4),
    ("fp6_fp6_b2_ragged", lambda: inputs.small_case(312, batch=2, hq=4, hkv=2, q_len=77, kv_len=333),
     B.MX_FP6, B.MX_FP6),
    ("q6_k4_many_tiles", lambda: inputs.small_case(313, hq=8, hkv=1, q_len=130, kv_len=2900, causal=True),
     B.MX_FP6, B.MX_FP4),
    ("q4_k6_d64", lambda: inputs.small_case(314, hq=4, hkv=1, q_len=90, kv_len=700, d=64, causal=True),
     B.MX_FP4, B.MX_FP6),
    # causal from position 0: rows below 64 see no key of the second stream's tiles
    ("fp6_fp4_causal_from_0", lambda: inputs.small_case(315, hq=4, hkv=2, q_len=200, kv_len=200, causal=True,
                                                         q_offset=0), B.MX_FP6, B.MX_FP4),
]


@pytest.mark.parametrize("name,make,qf,kf", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_mx_matches_emulation(name, make, qf, kf):
    c = make()
    Bn, Hq, L, D = c.q.shape
    N = c.k.shape[2]
    print(f"  prefill_mx {name} shape={c.shape}", flush=True)
    g, keys, o, kenc = caches(c, kf)
    dbg = torch.full((Bn, Hq, L, N), float("nan"), dtype=torch.float32, device=DEV)
    B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=N, q_fmt=qf, q_offset=c.q_offset, causal=c.causal,
                        out_dtype=B.OUT_F32, debug_s=dbg)
    out = B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=N, q_fmt=qf, q_offset=c.q_offset, causal=c.causal,
                              out_dtype=B.OUT_F32)
    out16 = B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=N, q_fmt=qf, q_offset=c.q_offset, causal=c.causal)
    torch.cuda.synchronize()
    mx = oracle.mx_operands(c.q, ORA_FMT[qf], kenc)
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=c.causal, want_s=True, mx=mx)
    vis = np.ones((L, N), bool)
    if c.causal:
        vis = np.arange(N)[None, :] <= (c.q_offset + np.arange(L))[:, None]
    vis = np.broadcast_to(vis, dbg.shape)
    s = dbg.cpu().numpy()
    assert not np.any(np.isnan(s[vis]))
    assert np.all(np.isnan(s[~vis]))               # invisible pairs untouched
    # fp32 accumulation of the block sums: within a few units of 2^-24 of sum |q_c k_c|
    G = Hq // kenc.values.shape[1]
    kv = np.repeat(kenc.values[:, :, :N], G, axis=1)
    s_abs = np.abs(mx.q_values) @ np.abs(kv).transpose(0, 1, 3, 2)
    d_s = np.abs(s.astype(np.float64) - ref.s_i32.astype(np.float64))
    assert np.all(d_s[vis] <= 8 * 2.0 ** -24 * s_abs[vis] + 1e-30)
    n_exact = float(np.mean(d_s[vis] == 0))
    err = rel_err(out.cpu().numpy(), ref.out)
    err16 = rel_err(out16.float().cpu().numpy(), ref.out)
    grid = oracle.attn_lowbit(c.q, c.k, c.v, ORA_FMT[qf], ORA_FMT[kf], causal=c.causal, q_offset=c.q_offset)
    cs = cosine(out.cpu().numpy(), grid)
    print(f"    scores bit-equal {n_exact:.4f}, err vs emulation {err:.2e} (fp16 out {err16:.2e}), "
          f"cos vs fp64 grid {cs:.6f}", flush=True)
    assert err <= TOL
    assert err16 <= TOL + 2e-3
    assert cs >= 0.999


def test_prefill_mx_accuracy_matches_the_grid_study():
    """The question the MX path answers: outputs against fp64 attention on the fp16 inputs, for
    each format, agree with the oracle's grid study (the same grids in fp64) to 1e-3 in cosine;
    the ordering fp6 > fp4 holds on the GPU as on the grid."""
    c = inputs.small_case(321, hq=8, hkv=2, q_len=128, kv_len=2048, causal=True)
    N = 2048
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=True, q_offset=c.q_offset)
    cos = {}
    for fmt in (B.MX_FP6, B.MX_FP4):
        g, keys, o, kenc = caches(c, fmt)
        out = B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=N, q_fmt=fmt, q_offset=c.q_offset, causal=True,
                                  out_dtype=B.OUT_F32)
        torch.cuda.synchronize()
        grid = oracle.attn_lowbit(c.q, c.k, c.v, ORA_FMT[fmt], ORA_FMT[fmt], causal=True, q_offset=c.q_offset)
        cos[fmt] = cosine(out.cpu().numpy(), exact)
        cg = cosine(grid, exact)
        print(f"    fmt {fmt}: cos vs fp64 GPU {cos[fmt]:.6f}, grid study {cg:.6f}", flush=True)
        assert abs(cos[fmt] - cg) <= 1e-3
    assert cos[B.MX_FP6] > cos[B.MX_FP4]


def test_prefill_mx_repeatable():
    c = inputs.small_case(322, hq=4, hkv=2, q_len=64, kv_len=500, causal=True)
    g, keys, o, kenc = caches(c, B.MX_FP4)
    a = B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=500, q_fmt=B.MX_FP4, q_offset=c.q_offset, causal=True)
    b = B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=500, q_fmt=B.MX_FP4, q_offset=c.q_offset, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_mx_full_size_sampled():
    """The LLM prompt chunk at its full size (2048 queries x 32768 keys, GQA 16/4, causal in
    the chunk) in the launch configuration the benchmark times, fp4 K with fp6 Q, checked on
    every 64th query row of every head (and each head's last) against the emulation."""
    c = inputs.config3()
    Bn, Hq, L, D = c.q.shape
    N = c.k.shape[2]
    print("  config3 generated", flush=True)
    g, keys, o, kenc = caches(c, B.MX_FP4)
    out = B.attn_q_prefill_mx(dev(c.q), keys, g, kv_len=N, q_fmt=B.MX_FP6, q_offset=c.q_offset, causal=True,
                              out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    rows = np.array(sorted({h * L + i for h in range(Hq) for i in list(range(0, L, 64)) + [L - 1]}), np.int64)
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=True, rows=rows,
                                 mx=oracle.mx_operands(c.q, oracle.LB_MXFP6, kenc))
    got = out.cpu().numpy().reshape(-1, D)[rows]
    err = rel_err(got, ref.out.reshape(-1, D)[rows])
    print(f"    full-size MX err vs emulation {err:.2e} over {rows.size} rows", flush=True)
    assert err <= TOL

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.

Bars:
* kv_quantize_i8 codes, scales, mean and PV operand: bit-exact;
* prefill int32 QK^T accumulators (debug export) and decode int32 dots: bit-exact;
* outputs (fp32 output mode) vs the oracle's emulation of the scheme: max error
  per row, normalised by the row's largest |value|, <= 1e-3 (the tolerance the
  accuracy gate states); fp16 output mode adds fp16 storage rounding (2^-11);
* cosine against fp64 attention on the fp16 inputs >= 0.999 on the LLM-like
  workloads; config 1's variance outliers miss it by design of the scheme (0.9984, the
  emulation's own level: recorded as a strict expected failure).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-3
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def rel_err(a, e):
    a = np.asarray(a, np.float64).reshape(-1, a.shape[-1])
    e = np.asarray(e, np.float64).reshape(-1, e.shape[-1])
    den = np.maximum(np.abs(e).max(axis=1, keepdims=True), 1e-30)
    return float(np.max(np.abs(a - e) / den))


def cosine(a, e):
    a = np.asarray(a, np.float64).ravel()
    e = np.asarray(e, np.float64).ravel()
    return float(a @ e / np.sqrt((a @ a) * (e @ e)))


def gpu_cache(k, v, k_gran, v_gran, cap=None, v_op_format=B.PV_FP8, subtract=True):
    Bn, H, N, D = k.shape
    cap = cap or (N + 63) // 64 * 64
    c = B.alloc_cache(Bn, H, cap, D, k_gran, v_gran, DEV, v_op_format=v_op_format)
    B.kv_quantize_i8(dev(k), dev(v), c, subtract_k_mean=subtract)
    torch.cuda.synchronize()
    return c


def ora_cache(k, v, k_gran, v_gran, cap=None, v_op_format=B.PV_FP8, subtract=True):
    N = k.shape[2]
    cap = cap or (N + 63) // 64 * 64
    return oracle.kv_quantize(k, v, k_gran, v_gran, subtract_mean=subtract, capacity=cap,
                              v_op_format=v_op_format)


def assert_cache_equal(g, o, N):
    print(f"  cache N={N} k_gran={o.k_gran} v_gran={o.v_gran}", flush=True)
    assert np.array_equal(g.k_codes.cpu().numpy()[:, :, :N], o.k_codes[:, :, :N])
    assert np.array_equal(g.v_codes.cpu().numpy()[:, :, :N], o.v_codes[:, :, :N])
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), o.k_mean.view(np.uint32))
    gk, ok = g.k_scales.cpu().numpy(), o.k_scales
    if o.k_gran == oracle.GRAN_TENSOR:
        gk = gk[:1]
    elif o.k_gran == oracle.GRAN_TOKEN:
        gk, ok = gk[:, :, :N], ok[:, :, :N]
    assert np.array_equal(np.ascontiguousarray(gk).view(np.uint8), np.ascontiguousarray(ok).view(np.uint8))
    gv = g.v_scales.cpu().numpy()
    ov = o.v_scales
    if o.v_gran == oracle.GRAN_TOKEN:
        gv, ov = gv[:, :, :N], ov[:, :, :N]
    assert np.array_equal(np.ascontiguousarray(gv).view(np.uint8), np.ascontiguousarray(ov).view(np.uint8))
    if o.v_op is not None:
        assert np.array_equal(g.v_op.cpu().numpy(), o.v_op)


# --------------------------------------------------------------- kv_quantize
KVQ_CASES = [
    ("config1", lambda: inputs.config1(), oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, B.PV_FP8, True),
    ("ragged_b2", lambda: inputs.small_case(51, batch=2, hq=4, hkv=2, q_len=5, kv_len=300),
     oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, B.PV_INT8, True),
    ("token", lambda: inputs.config4(kv_len=2000)[0], oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, None, True),
    ("tensor_d64", lambda: inputs.config2(batch=2), oracle.GRAN_TENSOR, oracle.GRAN_CHANNEL, B.PV_FP8, True),
    ("no_mean", lambda: inputs.small_case(52, kv_len=129), oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL,
     B.PV_FP8, False),
    ("one_key", lambda: inputs.small_case(53, kv_len=1, q_len=1), oracle.GRAN_TOKEN, oracle.GRAN_CHANNEL,
     B.PV_FP8, True),
]


@pytest.mark.parametrize("name,make,kg,vg,vfmt,sub", KVQ_CASES, ids=[c[0] for c in KVQ_CASES])
def test_kv_quantize_bit_exact(name, make, kg, vg, vfmt, sub):
    c = make()
    N = c.k.shape[2]
    cap = (N + 63) // 64 * 64 + (64 if name == "ragged_b2" else 0)
    g = gpu_cache(c.k, c.v, kg, vg, cap=cap, v_op_format=vfmt, subtract=sub)
    o = ora_cache(c.k, c.v, kg, vg, cap=cap, v_op_format=vfmt, subtract=sub)
    assert_cache_equal(g, o, N)


# -------------------------------------------------------------------- prefill
def run_prefill(c, *, pv_mode=B.PV_FP8, out_dtype=B.OUT_F32, debug=False, kv_len=None):
    Bn, Hq, L, D = c.q.shape
    N = kv_len or c.k.shape[2]
    g = gpu_cache(c.k, c.v, c.k_gran, c.v_gran, v_op_format=pv_mode)
    dbg = torch.full((Bn, Hq, L, N), -(2 ** 31), dtype=torch.int32, device=DEV) if debug else None
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=c.causal,
                           q_gran=c.q_gran, pv_mode=pv_mode, out_dtype=out_dtype, debug_s=dbg)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (dbg.cpu().numpy() if debug else None)


def emulate(c, *, pv_mode=B.PV_FP8, rows=None, want_s=False, kv_len=None):
    N = kv_len or c.k.shape[2]
    o = ora_cache(c.k, c.v, c.k_gran, c.v_gran, v_op_format=None)
    return oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=c.causal,
                                  q_gran=c.q_gran, pv_mode=pv_mode, rows=rows, want_s=want_s)


PREFILL_CASES = [
    ("config1", lambda: inputs.config1()),
    ("gqa4_causal_ragged", lambda: inputs.small_case(61, batch=2, hq=8, hkv=2, q_len=77, kv_len=333,
                                                      causal=True)),
    ("gqa2_noncausal", lambda: inputs.small_case(62, hq=4, hkv=2, q_len=130, kv_len=200)),
    ("mha_causal_offset0", lambda: inputs.small_case(63, hq=2, hkv=2, q_len=190, kv_len=190,
                                                      causal=True)),
    ("d64_vit", lambda: inputs.config2(batch=3)),
    ("gqa8_short", lambda: inputs.small_case(64, hq=8, hkv=1, q_len=9, kv_len=70, causal=True)),
    # many key tiles (the pipelined steady state), an odd tile count (the two key streams
    # get different numbers of tiles) and a ragged last tile
    ("gqa4_noncausal_25tiles", lambda: inputs.small_case(65, hq=8, hkv=2, q_len=300, kv_len=1601)),
    ("gqa4_causal_offset_many_tiles", lambda: inputs.small_case(66, hq=4, hkv=1, q_len=200, kv_len=2900,
                                                                 causal=True)),
]


@pytest.mark.parametrize("name,make", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_int32_scores_bit_exact(name, make):
    c = make()
    print(f"  prefill debug_s {name} shape={c.shape}", flush=True)
    _, s_gpu = run_prefill(c, debug=True)
    ref = emulate(c, want_s=True)
    N = c.k.shape[2]
    L = c.q.shape[2]
    mask = np.ones((L, N), bool)
    if c.causal:
        mask = np.arange(N)[None, :] <= (c.q_offset + np.arange(L))[:, None]
    mask = np.broadcast_to(mask, s_gpu.shape)
    assert np.array_equal(s_gpu[mask], ref.s_i32[mask])
    assert np.all(s_gpu[~mask] == -(2 ** 31))          # masked pairs never written


@pytest.mark.parametrize("k_gran", [oracle.GRAN_CHANNEL, oracle.GRAN_TENSOR], ids=["k_channel", "k_tensor"])
def test_prefill_tensor_q_scale_many_workgroups(k_gran):
    """Per-tensor Q over 2.1 M query values (the scale pass loops over its grid twice), with
    K per channel (the pass scales q by s_K first) and per tensor: int32 scores bit-exact,
    so the Q codes and their one scale equal the oracle's."""
    c = inputs.small_case(67, batch=2, hq=8, hkv=2, q_len=1024, kv_len=150, k_gran=k_gran,
                          q_gran=oracle.GRAN_TENSOR)
    print(f"  prefill per-tensor Q shape={c.shape} k_gran={k_gran}", flush=True)
    out, s_gpu = run_prefill(c, debug=True)
    ref = emulate(c, want_s=True)
    assert np.array_equal(s_gpu, ref.s_i32)
    assert rel_err(out, ref.out) <= TOL


@pytest.mark.parametrize("pv_mode", [B.PV_FP8, B.PV_INT8], ids=["fp8pv", "int8pv"])
@pytest.mark.parametrize("name,make", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_matches_emulation(name, make, pv_mode):
    c = make()
    print(f"  prefill {name} pv={pv_mode} shape={c.shape}", flush=True)
    out, _ = run_prefill(c, pv_mode=pv_mode)
    ref = emulate(c, pv_mode=pv_mode)
    err = rel_err(out, ref.out)
    assert err <= TOL, err
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("pv_mode", [B.PV_FP8, B.PV_INT8], ids=["fp8pv", "int8pv"])
def test_prefill_p_codes_against_emulation(pv_mode):
    """The P codes themselves (debug export) against the oracle's on the outlier case: the
    int32 scores are bit-exact and the exponent is the same one-rounding fp32 value on both
    sides, so a code can differ only where the hardware exp2 (not correctly rounded) lands on
    the other side of an e4m3 (int8) rounding boundary.  The mismatch count is reported;
    each mismatch is one step of the code grid."""
    c = inputs.config1()
    Bn, Hq, L, D = c.q.shape
    N = c.k.shape[2]
    g = gpu_cache(c.k, c.v, c.k_gran, c.v_gran, v_op_format=pv_mode)
    dp = torch.full((Bn, Hq, L, N), 0xFF, dtype=torch.uint8, device=DEV)
    B.attn_q_prefill(dev(c.q), g, kv_len=N, out_dtype=B.OUT_F32, pv_mode=pv_mode, debug_p=dp)
    torch.cuda.synchronize()
    got = dp.cpu().numpy()
    ref = oracle.prefill_emulate(c.q, ora_cache(c.k, c.v, c.k_gran, c.v_gran, v_op_format=None), kv_len=N,
                                 q_offset=0, causal=False, pv_mode=pv_mode, want_p=True).p_codes
    diff = got != ref
    n = int(diff.sum())
    print(f"  config1 P-code mismatches ({'e4m3' if pv_mode == B.PV_FP8 else 'int8'}): {n} of {diff.size}", flush=True)
    assert n <= diff.size // 10000
    if n:   # adjacent codes: e4m3 bytes of non-negative values are monotone, so one step apart
        assert np.all(np.abs(got[diff].astype(np.int64) - ref[diff].astype(np.int64)) == 1)


def test_prefill_lse_against_emulation_and_chunk_merge():
    """The optional base-2 log-sum-exp output: against the oracle's (same scores, same running
    maxima and normalizer) within 1e-3 -- the fp8 matrix core sums the 64 products of a tile
    with fewer low-order bits than fp32 (measured: one 448 beside 63 values of 2^-6 sums to
    448.875 instead of 448.984, 2.4e-4 low), so the row sums l run up to a few 1e-4 low,
    and log2 l by up to 7e-4 -- and as the merge weight of two key
    chunks attended separately (non-causal rows over keys [0, 1024) and [1024, 2900)):
    2^(lse_k - LSE)-weighted chunk outputs reproduce the whole-range output within the P
    rounding of the chunk split, and LSE within log2(1 / (1 - 2^-4)) < 0.1 (each l sums e4m3
    codes within 2^-4 of the weights they round; the oracle's own chunk merge on these rows:
    1.4e-2 in LSE, 8.9e-3 in the output)."""
    c = inputs.small_case(69, hq=8, hkv=2, q_len=100, kv_len=2900)
    Bn, Hq, L, D = c.q.shape
    N = 2900
    g = gpu_cache(c.k, c.v, c.k_gran, c.v_gran)
    lse = torch.empty((Bn, Hq, L), dtype=torch.float32, device=DEV)
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, out_dtype=B.OUT_F32, lse=lse)
    torch.cuda.synchronize()
    ref = emulate(c)
    assert rel_err(out.cpu().numpy(), ref.out) <= TOL
    d_lse = lse.cpu().numpy() - ref.lse
    print(f"  lse vs emulation: max |d| {np.abs(d_lse).max():.2e}, mean {d_lse.mean():.2e}", flush=True)
    assert np.max(np.abs(d_lse)) <= 1e-3
    # the second chunk: the keys from 1024 on, in a cache of their own with the same codes
    g2 = B.alloc_cache(Bn, 2, 1920, D, c.k_gran, c.v_gran, DEV, v_op_format=B.PV_FP8)
    g2.k_codes[:, :, :N - 1024].copy_(g.k_codes[:, :, 1024:N])
    g2.k_scales.copy_(g.k_scales)
    g2.v_scales.copy_(g.v_scales)
    g2.v_op.copy_(g.v_op[:, :, 16:46])
    lse1 = torch.empty_like(lse)
    lse2 = torch.empty_like(lse)
    o1 = B.attn_q_prefill(dev(c.q), g, kv_len=1024, out_dtype=B.OUT_F32, lse=lse1)
    o2 = B.attn_q_prefill(dev(c.q), g2, kv_len=N - 1024, out_dtype=B.OUT_F32, lse=lse2)
    torch.cuda.synchronize()
    l1, l2 = lse1.cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64)
    M = np.maximum(l1, l2)
    w1, w2 = np.exp2(l1 - M), np.exp2(l2 - M)
    LSE = M + np.log2(w1 + w2)
    merged = (w1[..., None] * o1.cpu().numpy() + w2[..., None] * o2.cpu().numpy()) / (w1 + w2)[..., None]
    assert np.max(np.abs(LSE - lse.cpu().numpy())) <= 0.1
    assert rel_err(merged, ref.out) <= 2e-2


def test_prefill_fp16_output():
    c = inputs.small_case(65, hq=4, hkv=1, q_len=100, kv_len=260, causal=True)
    out, _ = run_prefill(c, out_dtype=B.OUT_F16)
    ref = emulate(c)
    assert rel_err(out, ref.out) <= TOL + 2.0 ** -11


def test_prefill_deterministic():
    c = inputs.small_case(66, hq=8, hkv=2, q_len=256, kv_len=1024, causal=True)
    a, _ = run_prefill(c)
    b, _ = run_prefill(c)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_prefill_config1_accuracy_is_the_schemes():
    """The outlier case (five K channels with x40 variance, which centring cannot remove;
    their per-channel scales, folded into Q, leave Q's other channels few int8 levels): the GPU
    reaches the cosine against fp64 of the scheme's own emulation (0.99839), within 1e-5."""
    c = inputs.config1()
    out, _ = run_prefill(c)
    exact = oracle.attn_exact(c.q, c.k, c.v)
    emu = emulate(c).out
    cg, ce = cosine(out, exact), cosine(emu, exact)
    print(f"  config1 cos vs fp64: GPU {cg:.6f}, emulation {ce:.6f}", flush=True)
    assert abs(cg - ce) <= 1e-5


@pytest.mark.xfail(strict=True, reason="the outlier case misses the 0.999 cosine bar by design of the "
                   "scheme: per-token Q with the x40 per-channel K scales folded in reaches 0.9984 "
                   "(the cache alone 0.9998); recorded as a failure, not a relaxed bar")
def test_prefill_config1_reaches_cosine_0999():
    c = inputs.config1()
    out, _ = run_prefill(c)
    assert cosine(out, oracle.attn_exact(c.q, c.k, c.v)) >= 0.999


def _sample_rows(Bn, Hq, L, step):
    rows = []
    for b in range(Bn):
        for h in range(Hq):
            base = (b * Hq + h) * L
            rows.extend(base + i for i in list(range(0, L, step)) + [L - 1])
    return np.array(sorted(set(rows)), np.int64)


def test_prefill_config2_vit_full():
    c = inputs.config2()
    out, _ = run_prefill(c)
    rows = _sample_rows(64, 12, 197, 16)
    ref = emulate(c, rows=rows)
    o = out.reshape(-1, 64)[rows]
    assert rel_err(o, ref.out.reshape(-1, 64)[rows]) <= TOL
    exact = oracle.attn_exact(c.q, c.k, c.v, rows=rows).reshape(-1, 64)[rows]
    assert cosine(o, exact) >= 0.999


def test_prefill_config3_full_size_sampled():
    """The LLM prompt chunk at its full size (2048 queries x 32768 keys, GQA 16/4,
    causal within the chunk), in the launch configuration the benchmark times,
    checked on every 64th query row of every head."""
    c = inputs.config3()
    print("  config3 generated", flush=True)
    out8, _ = run_prefill(c)
    outi, _ = run_prefill(c, pv_mode=B.PV_INT8)
    rows = _sample_rows(1, 16, 2048, 64)
    ref = emulate(c, rows=rows)
    o8 = out8.reshape(-1, 128)[rows]
    assert rel_err(o8, ref.out.reshape(-1, 128)[rows]) <= TOL
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=True, q_offset=c.q_offset, rows=rows).reshape(-1, 128)[rows]
    c8 = cosine(o8, exact)
    ci = cosine(outi.reshape(-1, 128)[rows], exact)
    print(f"  config3 cos fp8-PV {c8:.6f} int8-PV {ci:.6f}", flush=True)
    assert c8 >= 0.999
    assert rel_err(o8, exact) < rel_err(outi.reshape(-1, 128)[rows], exact)


def _rel_l2(a, e):
    return float(np.linalg.norm(np.asarray(a, np.float64) - e) / np.linalg.norm(e))


def test_prefill_config5_last_chunk_sampled():
    """Long context: GQA 32/8 over a 131072-key int8 cache, the last 8192-query
    chunk (q_offset 122880), sampled rows; fp8 PV against the emulation and fp64, and the
    int8-PV variant further from fp64."""
    k, v, params = inputs.config5_kv()
    q = inputs.config5_chunk_q(params, 15)
    c = inputs.AttnInputs("config5", q, k, v, True, 131072 - 8192, oracle.GRAN_CHANNEL,
                          oracle.GRAN_CHANNEL, oracle.GRAN_TOKEN)
    print("  config5 generated", flush=True)
    out, _ = run_prefill(c)
    outi, _ = run_prefill(c, pv_mode=B.PV_INT8)
    rows = _sample_rows(1, 32, 8192, 1024)
    ref = emulate(c, rows=rows)
    o = out.reshape(-1, 128)[rows]
    assert rel_err(o, ref.out.reshape(-1, 128)[rows]) <= TOL
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=True, q_offset=c.q_offset, rows=rows).reshape(-1, 128)[rows]
    oi = outi.reshape(-1, 128)[rows]
    print(f"  config5 cos fp8-PV {cosine(o, exact):.6f} int8-PV {cosine(oi, exact):.6f}", flush=True)
    assert cosine(o, exact) >= 0.999
    assert _rel_l2(o, exact) < _rel_l2(oi, exact) and rel_err(o, exact) < rel_err(oi, exact)


def test_fp8_pv_gap_over_int8_pv_grows_with_context():
    """The pages' finding ("int8 Flash Attention on RDNA4", the variant table and "Is fp8
    attention accurate enough"): int8 P loses the diffuse tail and its error grows with
    context; e4m3 P keeps it.  The GPU outputs of both PV variants against fp64: the ratio of
    their relative L2 errors (int8 / fp8) grows from 256 keys (the outlier case, peaked rows:
    int8 P's finer steps near 1 make it slightly better there, ratio 0.90) to 32768 keys (2.1)
    to 131072 keys (3.2); fp8 is the more accurate at both long lengths."""
    ratios = []
    c1 = inputs.config1()
    e1 = oracle.attn_exact(c1.q, c1.k, c1.v)
    ratios.append(_rel_l2(run_prefill(c1, pv_mode=B.PV_INT8)[0], e1) / _rel_l2(run_prefill(c1)[0], e1))
    c3 = inputs.config3()
    r3 = _sample_rows(1, 16, 2048, 64)
    e3 = oracle.attn_exact(c3.q, c3.k, c3.v, causal=True, q_offset=c3.q_offset, rows=r3).reshape(-1, 128)[r3]
    f3 = run_prefill(c3)[0].reshape(-1, 128)[r3]
    i3 = run_prefill(c3, pv_mode=B.PV_INT8)[0].reshape(-1, 128)[r3]
    ratios.append(_rel_l2(i3, e3) / _rel_l2(f3, e3))
    k, v, params = inputs.config5_kv()
    c5 = inputs.AttnInputs("config5", inputs.config5_chunk_q(params, 15), k, v, True, 131072 - 8192,
                           oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, oracle.GRAN_TOKEN)
    r5 = _sample_rows(1, 32, 8192, 1024)
    e5 = oracle.attn_exact(c5.q, c5.k, c5.v, causal=True, q_offset=c5.q_offset, rows=r5).reshape(-1, 128)[r5]
    f5 = run_prefill(c5)[0].reshape(-1, 128)[r5]
    i5 = run_prefill(c5, pv_mode=B.PV_INT8)[0].reshape(-1, 128)[r5]
    ratios.append(_rel_l2(i5, e5) / _rel_l2(f5, e5))
    print(f"  int8-PV / fp8-PV relative L2 error at 256 / 32768 / 131072 keys: "
          f"{ratios[0]:.2f} / {ratios[1]:.2f} / {ratios[2]:.2f}", flush=True)
    assert ratios[0] < ratios[1] < ratios[2]
    assert ratios[1] > 1.5 and ratios[2] > 2.0


def test_prefill_q_len_zero_is_noop():
    c = inputs.small_case(67, q_len=1, kv_len=64)
    g = gpu_cache(c.k, c.v, c.k_gran, c.v_gran)
    out = torch.full((1, 2, 0, 128), 7.0, device=DEV)
    q = torch.empty((1, 2, 0, 128), dtype=torch.float16, device=DEV)
    B.attn_q_prefill(q, g, kv_len=64, out=out, out_dtype=B.OUT_F32)
    torch.cuda.synchronize()


# --------------------------------------------------------------------- decode
def run_decode(c, kv_len, k_gran, v_gran, debug=True, out_dtype=B.OUT_F32):
    g = gpu_cache(c.k, c.v, k_gran, v_gran, v_op_format=None)
    q = dev(c.q[:, :, 0])
    Bn, Hq, D = q.shape
    dbg = torch.zeros((Bn, Hq, kv_len), dtype=torch.int32, device=DEV) if debug else None
    out = B.attn_q_decode(q, g, kv_len=kv_len, out_dtype=out_dtype, debug_qk=dbg)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (dbg.cpu().numpy() if debug else None)


DECODE_CASES = [
    ("config4", lambda: inputs.config4()[0], 32768, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN),
    ("ragged1000", lambda: inputs.config4(kv_len=1000)[0], 1000, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN),
    ("one_key", lambda: inputs.config4(kv_len=64)[0], 1, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN),
    ("channel", lambda: inputs.config4(kv_len=5000)[0], 5000, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL),
    ("g1_d64", lambda: inputs.small_case(71, hq=3, hkv=3, q_len=1, kv_len=777, d=64), 777,
     oracle.GRAN_TOKEN, oracle.GRAN_CHANNEL),
    ("g2", lambda: inputs.small_case(72, batch=2, hq=4, hkv=2, q_len=1, kv_len=4097), 4097,
     oracle.GRAN_CHANNEL, oracle.GRAN_TOKEN),
    ("g8", lambda: inputs.small_case(73, hq=8, hkv=1, q_len=1, kv_len=513), 513,
     oracle.GRAN_TOKEN, oracle.GRAN_TOKEN),
]


@pytest.mark.parametrize("name,make,kv_len,kg,vg", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_matches_emulation(name, make, kv_len, kg, vg):
    c = make()
    print(f"  decode {name} kv_len={kv_len}", flush=True)
    out, dots = run_decode(c, kv_len, kg, vg)
    o = ora_cache(c.k, c.v, kg, vg)
    ref, rdots = oracle.decode_emulate(c.q[:, :, 0], o, kv_len=kv_len, want_qk=True)
    assert np.array_equal(dots, rdots)
    assert rel_err(out, ref) <= TOL
    # a repeated call gives the same bits
    out2, _ = run_decode(c, kv_len, kg, vg, debug=False)
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32))


def test_decode_config4_accuracy_vs_fp64():
    c = inputs.config4()[0]
    out, _ = run_decode(c, 32768, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, debug=False)
    exact = oracle.attn_exact(c.q, c.k, c.v)[:, :, 0]
    assert cosine(out, exact) >= 0.999


def test_decode_token_v_scales_spread_over_six_decades():
    # Per-token V rows scaled by 10^u, u uniform in [-3, 3]: the fp16 PV weights
    # p * s_V[n] then span many binades within one 64-key group of the kernel, which
    # scales them by a power of two to its largest weight before rounding to fp16.
    c = inputs.config4(kv_len=3000)[0]
    rng = np.random.default_rng(2024)
    f = 10.0 ** rng.uniform(-3.0, 3.0, size=(1, c.v.shape[1], c.v.shape[2], 1))
    v = np.clip(c.v.astype(np.float64) * f, -60000.0, 60000.0).astype(np.float16)
    c = dataclasses.replace(c, v=v)
    out, _ = run_decode(c, 3000, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, debug=False)
    o = ora_cache(c.k, c.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN)
    ref, _ = oracle.decode_emulate(c.q[:, :, 0], o, kv_len=3000)
    assert rel_err(out, ref) <= TOL


def test_decode_ragged_batch_device_lengths():
    """Decode of a ragged batch in one call: device kv_lens [B] = (2000, 37, 513) keys with
    kv_len 2000 (the largest).  Each row matches the oracle's decode over its own keys and is
    bit-identical to a call with that length for every row (splits past a row's keys are
    empty and skipped by the merge)."""
    c = inputs.small_case(74, batch=3, hq=8, hkv=2, q_len=1, kv_len=2000, k_gran=inputs.GRAN_TOKEN,
                          v_gran=inputs.GRAN_TOKEN)
    lens = [2000, 37, 513]
    g = gpu_cache(c.k, c.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, v_op_format=None)
    o = ora_cache(c.k, c.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, v_op_format=None)
    q = dev(c.q[:, :, 0])
    kvl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = B.attn_q_decode(q, g, kv_len=2000, out_dtype=B.OUT_F32, kv_lens=kvl).cpu().numpy()
    for b, n in enumerate(lens):
        ref, _ = oracle.decode_emulate(c.q[:, :, 0], o, kv_len=n)
        assert rel_err(out[b], ref[b]) <= TOL, (b, n)
        one = B.attn_q_decode(q, g, kv_len=n, out_dtype=B.OUT_F32).cpu().numpy()
        assert np.array_equal(out[b].view(np.uint32), one[b].view(np.uint32)), (b, n)


def test_prefill_only_cache_without_v_codes():
    """A per-channel cache written without its int8 V codes (v_codes NULL beside the e4m3
    operand) holds the same K codes, scales and operand, and the prefill over it gives the
    same bytes; the calls that read V codes refuse it."""
    c = inputs.small_case(51, hq=8, hkv=2, q_len=120, kv_len=900, causal=True)
    Bn, H, N, D = c.k.shape
    k, v, q = (torch.from_numpy(x).to(DEV) for x in (c.k, c.v, c.q))
    full = B.alloc_cache(Bn, H, 960, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, DEV, v_op_format=B.PV_FP8)
    lean = B.alloc_cache(Bn, H, 960, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, DEV, v_op_format=B.PV_FP8, v_codes=False)
    B.kv_quantize_i8(k, v, full)
    B.kv_quantize_i8(k, v, lean)
    a = B.attn_q_prefill(q, full, kv_len=N, q_offset=c.q_offset, causal=True)
    b = B.attn_q_prefill(q, lean, kv_len=N, q_offset=c.q_offset, causal=True)
    torch.cuda.synchronize()
    for f in ("k_codes", "k_scales", "v_scales", "k_mean", "v_op"):
        assert torch.equal(getattr(full, f), getattr(lean, f)), f
    assert torch.equal(a, b)
    with pytest.raises(B.AttnQError):
        B.attn_q_decode(q[:, :, -1].contiguous(), lean, kv_len=N)

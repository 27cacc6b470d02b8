"""GPU parity of attn_q_kv_append_i8 (the decode-time cache update with the running
per-channel K mean of the cache header) against the oracle's kv_append, through the
C ABI, on the same seeded inputs.

Bars: K/V codes, per-token fp16 scales, the int64 header sum and the fp32 header mean
are bit-exact; rows outside the appended range are untouched; decoding the appended
cache matches the oracle's decode emulation on the oracle's cache (int32 dots
bit-exact, output <= 1e-3 relative to each row's largest value) and stays within
cosine 0.999 of fp64 attention.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-3
DEV = "cuda:0"
SENTINEL = 0x55
# scale rows past the cache's length: fp16 +Inf for K, a NaN for V (the decode must never
# let such a row's scale reach a weight, and the append must leave them untouched)
K_SCALE_SENTINEL, V_SCALE_SENTINEL = 0x7C00, 0x7E00


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
    return float(np.max(np.abs(a - e) / np.maximum(np.abs(e).max(axis=1, keepdims=True), 1e-30)))


def build_both(k, v, prompt, splits, cap):
    """The same cache on both sides: the first `prompt` tokens by kv_quantize (one mean,
    header exported; prompt 0 = empty cache), then appends of the given sizes."""
    Bn, H, N, D = k.shape
    assert prompt + sum(splits) <= min(N, cap)
    g = B.alloc_cache(Bn, H, cap, D, B.GRAN_TOKEN, B.GRAN_TOKEN, DEV, v_op_format=None, header=True)
    for t in (g.k_codes, g.v_codes):
        t.fill_(SENTINEL)
    g.k_scales.view(torch.int16).fill_(K_SCALE_SENTINEL)
    g.v_scales.view(torch.int16).fill_(V_SCALE_SENTINEL)
    if prompt:
        S = np.zeros((Bn, H, D), np.int64)
        o = oracle.kv_quantize(np.ascontiguousarray(k[:, :, :prompt]), np.ascontiguousarray(v[:, :, :prompt]),
                               oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, capacity=cap, k_sum=S)
        B.kv_quantize_i8(dev(k[:, :, :prompt]), dev(v[:, :, :prompt]), g)
    else:
        o = oracle.empty_append_cache(Bn, H, cap, D)
        S = np.zeros((Bn, H, D), np.int64)
    n = prompt
    for T in splits:
        kk, vv = np.ascontiguousarray(k[:, :, n:n + T]), np.ascontiguousarray(v[:, :, n:n + T])
        oracle.kv_append(kk, vv, o, S)
        B.attn_q_kv_append_i8(dev(kk), dev(vv), g)
        n += T
    torch.cuda.synchronize()
    assert g.seq_len == o.seq_len == n
    return g, o, S


def assert_appended_equal(g, o, S, lo, hi):
    print(f"  rows {lo}..{hi}", flush=True)
    gk, gv = g.k_codes.cpu().numpy(), g.v_codes.cpu().numpy()
    assert np.array_equal(gk[:, :, :hi], o.k_codes[:, :, :hi])
    assert np.array_equal(gv[:, :, :hi], o.v_codes[:, :, :hi])
    for gs, os_ in ((g.k_scales, o.k_scales), (g.v_scales, o.v_scales)):
        assert np.array_equal(gs.cpu().numpy()[:, :, :hi].view(np.uint16), os_[:, :, :hi].view(np.uint16))
    assert np.array_equal(g.k_sum.cpu().numpy(), S)
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), o.k_mean.view(np.uint32))
    # rows past the last appended one are untouched
    assert np.all(gk[:, :, hi:] == SENTINEL) and np.all(gv[:, :, hi:] == SENTINEL)
    assert np.all(g.k_scales.cpu().numpy()[:, :, hi:].view(np.uint16) == K_SCALE_SENTINEL)
    assert np.all(g.v_scales.cpu().numpy()[:, :, hi:].view(np.uint16) == V_SCALE_SENTINEL)


APPEND_CASES = [
    # name, make(), prompt, splits, capacity
    ("empty_singles_d128", lambda: inputs.small_case(81, batch=2, hq=3, hkv=3, q_len=1, kv_len=40), 0,
     [1] * 40, 64),
    ("empty_one_call_multichunk_d64", lambda: inputs.small_case(82, hq=2, hkv=2, q_len=1, kv_len=300, d=64),
     0, [300], 320),
    ("prompt_then_mixed", lambda: inputs.config4(kv_len=5000)[0], 4000,
     [1, 1, 63, 64, 65, 200, 1, 127, 128, 350], 5000),
    ("prompt_then_singles_d64", lambda: inputs.small_case(85, batch=3, hq=6, hkv=3, q_len=1, kv_len=24, d=64),
     5, [1] * 19, 24),
    ("fill_to_capacity", lambda: inputs.small_case(83, hq=4, hkv=2, q_len=1, kv_len=200), 129, [70, 1], 200),
]


@pytest.mark.parametrize("name,make,prompt,splits,cap", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_bit_exact(name, make, prompt, splits, cap):
    c = make()
    print(f"  append {name}: prompt={prompt} splits={splits} cap={cap}", flush=True)
    g, o, S = build_both(c.k, c.v, prompt, splits, cap)
    assert_appended_equal(g, o, S, prompt, prompt + sum(splits))


def test_append_split_does_not_change_the_cache():
    """One call of 700 tokens and calls of 1, 64, 65 and 570 tokens write the same bytes
    (the scan is exact, so its split is invisible)."""
    c = inputs.config4(kv_len=1700)[0]
    g1, _, _ = build_both(c.k, c.v, 1000, [700], 1728)
    g2, _, _ = build_both(c.k, c.v, 1000, [1, 64, 65, 570], 1728)
    for f in ("k_codes", "v_codes", "k_scales", "v_scales", "k_sum", "k_mean"):
        a, b = getattr(g1, f), getattr(g2, f)
        if a.is_floating_point():   # (bit patterns: the rows past the cache hold NaN sentinels)
            a, b = a.view(torch.int16 if a.dtype == torch.float16 else torch.int32), \
                b.view(torch.int16 if b.dtype == torch.float16 else torch.int32)
        assert torch.equal(a, b), f


def test_append_zero_tokens_is_noop():
    c = inputs.small_case(84, hq=2, hkv=2, q_len=1, kv_len=64)
    g, o, S = build_both(c.k, c.v, 10, [], 64)
    before = [t.clone() for t in (g.k_codes, g.k_sum, g.k_mean)]
    empty = torch.empty((1, 2, 0, 128), dtype=torch.float16, device=DEV)
    B.attn_q_kv_append_i8(empty, empty, g)
    torch.cuda.synchronize()
    assert g.seq_len == 10
    for a, b in zip(before, (g.k_codes, g.k_sum, g.k_mean)):
        assert torch.equal(a, b)


def test_decode_after_appends_matches_the_oracle():
    """The LLM-like decode workload at its full 32768-token length, the last 1024 tokens
    appended (one call of 1000, then 24 single tokens, as decode steps would): decode of
    the GPU cache against the oracle's emulation on the oracle's cache, and against fp64."""
    P, N = 31744, 32768
    c = inputs.config4(kv_len=N)[0]
    g, o, S = build_both(c.k, c.v, P, [1000] + [1] * 24, N)
    assert_appended_equal(g, o, S, P, N)
    q = c.q[:, :, 0]
    Bn, Hq, D = q.shape
    dbg = torch.zeros((Bn, Hq, N), dtype=torch.int32, device=DEV)
    out = B.attn_q_decode(dev(q), g, kv_len=N, out_dtype=B.OUT_F32, debug_qk=dbg)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref, rdots = oracle.decode_emulate(q, o, kv_len=N, want_qk=True)
    assert np.array_equal(dbg.cpu().numpy(), rdots)
    err = rel_err(out, ref)
    exact = oracle.attn_exact(c.q, c.k, c.v)[:, :, 0]
    cos = float((out.ravel() @ exact.ravel()) / np.linalg.norm(out) / np.linalg.norm(exact))
    print(f"  decode after appends: err vs emulation {err:.3g}, cosine vs fp64 {cos:.6f}", flush=True)
    assert err <= TOL
    assert cos >= 0.999


FUSED_CASES = [
    # (prompt tokens, steps): the new keys cross a 512-key split boundary (511 -> 512), start
    # from an empty cache (the first key: no shift, kv_len 1), and run past a long prompt
    ("split_boundary", 509, 5),
    ("empty_cache", 0, 3),
    ("long_prompt", 4000, 4),
]


FUSED_SHAPES = {
    "split_boundary": None, "empty_cache": None, "long_prompt": None,
    # other instantiations of the fused kernel: d = 64 with 8 query heads per kv head, and
    # 2 query heads per kv head at batch 2
    "d64_g8": dict(seed=91, batch=1, hq=8, hkv=1, d=64),
    "b2_g2": dict(seed=92, batch=2, hq=4, hkv=2, d=128),
}
FUSED_CASES += [("d64_g8", 700, 3), ("b2_g2", 1030, 3)]


@pytest.mark.parametrize("name,prompt,steps", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_decode_append_equals_the_two_calls(name, prompt, steps):
    """attn_q_decode_append: bit for bit attn_q_kv_append_i8 then attn_q_decode, step after
    step (output, appended rows, scales, header sum and mean), and the output matches the
    oracle's decode of the oracle's appended cache."""
    N = prompt + steps
    shape = FUSED_SHAPES[name]
    if shape is None:
        c = inputs.config4(kv_len=max(N, 64))[0]
    else:
        kw = dict(shape)
        c = inputs.small_case(kw.pop("seed"), q_len=1, kv_len=max(N, 64), k_gran=inputs.GRAN_TOKEN,
                              v_gran=inputs.GRAN_TOKEN, **kw)
    cap = (N + 63) // 64 * 64
    qs = c.q[:, :, 0]
    ga, o, S = build_both(c.k, c.v, prompt, [], cap)       # fused path
    gb, _, _ = build_both(c.k, c.v, prompt, [], cap)       # two calls
    for t in range(steps):
        n = prompt + t
        kt = dev(np.ascontiguousarray(c.k[:, :, n]))
        vt = dev(np.ascontiguousarray(c.v[:, :, n]))
        q = dev(qs)
        print(f"  fused step {name} n={n}", flush=True)
        oa = B.attn_q_decode_append(q, kt, vt, ga, out_dtype=B.OUT_F32)
        B.attn_q_kv_append_i8(kt[:, :, None], vt[:, :, None], gb)
        ob = B.attn_q_decode(q, gb, kv_len=n + 1, out_dtype=B.OUT_F32)
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), f"output differs at step {t}"
        for fa, fb in ((ga.k_codes, gb.k_codes), (ga.v_codes, gb.v_codes), (ga.k_sum, gb.k_sum)):
            assert torch.equal(fa, fb)
        for fa, fb in ((ga.k_scales, gb.k_scales), (ga.v_scales, gb.v_scales), (ga.k_mean, gb.k_mean)):
            assert torch.equal(fa.view(torch.int16 if fa.dtype == torch.float16 else torch.int32),
                               fb.view(torch.int16 if fb.dtype == torch.float16 else torch.int32))
        # the oracle appends the same token and decodes its own cache
        oracle.kv_append(np.ascontiguousarray(c.k[:, :, n:n + 1]), np.ascontiguousarray(c.v[:, :, n:n + 1]), o, S)
        ref, _ = oracle.decode_emulate(qs, o, kv_len=n + 1)
        assert rel_err(oa.cpu().numpy(), ref) <= TOL
    assert ga.seq_len == N and gb.seq_len == N

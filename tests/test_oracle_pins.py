"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the fact it pins.  None of them re-types an oracle formula:
they use printed values (tests/golden/page_constants.json), closed forms,
invariants, independent library routines (numpy's fp16, numpy integer matmul)
or exhaustive / brute-force searches.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import diagnostics as dg
from quantized_attention_attn_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


# ------------------------------------------------------------------ e4m3 ---
def _e4m3_values_from_definition():
    """All 256 e4m3 bit patterns evaluated from the OCP E4M3 definition
    (bias 7, 3 fraction bits, subnormals at exponent field 0, S.1111.111 = NaN)."""
    vals = []
    for b in range(256):
        s, e, f = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and f == 7:
            v = math.nan
        elif e == 0:
            v = (f / 8.0) * 2.0 ** -6
        else:
            v = (1 + f / 8.0) * 2.0 ** (e - 7)
        vals.append(-v if s else v)
    return np.array(vals)


def test_e4m3_decode_matches_definition():
    ref = _e4m3_values_from_definition()
    got = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    back = oracle.e4m3_encode(vals[ok].astype(np.float32))
    assert np.array_equal(back, codes[ok])


def _brute_nearest_even(x: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3 by exhaustive search; ties to the even code; beyond
    the largest finite value, saturate."""
    table = _e4m3_values_from_definition()
    pos = [(table[b], b) for b in range(128) if not np.isnan(table[b])]
    pv = np.array([p[0] for p in pos])
    pc = np.array([p[1] for p in pos])
    out = np.empty(x.shape, np.uint8)
    for i, xv in enumerate(x.astype(np.float64)):
        a = abs(xv)
        if a >= pv.max():
            code = pc[np.argmax(pv)]
        else:
            dist = np.abs(pv - a)
            best = dist.min()
            cand = pc[dist == best]
            code = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
        out[i] = code | (0x80 if np.signbit(xv) else 0)
    return out


def test_e4m3_encode_matches_brute_force():
    rng = np.random.default_rng(7)
    table = _e4m3_values_from_definition()
    fin = np.sort(np.unique(np.abs(table[~np.isnan(table)])))
    mids = (fin[1:] + fin[:-1]) / 2.0           # exact ties
    around = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                             np.nextafter(mids.astype(np.float32), np.float32(1e9)), fin])
    rnd = np.exp(rng.uniform(np.log(1e-7), np.log(600.0), 20000))
    x = np.concatenate([around, rnd, [460.0, 463.99, 464.0, 500.0, 1e30]]).astype(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.e4m3_encode(x), _brute_nearest_even(x))


def test_e4m3_page_constants():
    """448 is the largest value, 8 steps per binade, 3 mantissa bits, and with
    the static scale 448 the smallest representable probability is about 4e-6."""
    vals = oracle.e4m3_decode(np.arange(128, dtype=np.uint8))
    fin = vals[~np.isnan(vals)]
    assert fin.max() == GOLD["e4m3_static_scale"]["value"]
    for e in range(-6, 8):
        n = np.sum((fin >= 2.0 ** e) & (fin < 2.0 ** (e + 1)))
        assert n == GOLD["e4m3_steps_per_binade"]["value"]
    floor = fin[fin > 0].min() / 448.0
    assert floor == 2.0 ** -9 / 448.0
    assert 3.5e-6 < floor < 4.5e-6        # "about 4e-6"
    # constant relative error across the normal range: <= 2^-(mantissa bits + 1)
    rng = np.random.default_rng(3)
    p = np.exp(rng.uniform(np.log(2.0 ** -6), np.log(448.0), 100000)).astype(np.float32)
    rel = np.abs(oracle.e4m3_decode(oracle.e4m3_encode(p)) - p) / p
    assert rel.max() <= 2.0 ** -(GOLD["e4m3_mantissa_bits"]["value"] + 1) + 1e-12
    # and the int8 grid with scale 127 cannot hold that range: its floor is 1/127
    assert floor < (1 / 127) / 1000


# ------------------------------------------------------------------ fp16 ---
def test_fp16_codec_matches_numpy():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.uniform(-9, 5, 50000),
                        [0.0, -0.0, 65504.0, 65519.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26]])
    x32 = x.astype(np.float32)
    want = x32.astype(np.float16)                   # numpy's RNE conversion
    got = oracle.float_to_half(x32)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    dec = oracle.half_to_double(h)
    ref = h.astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(dec), nan)
    assert np.array_equal(dec[~nan], ref[~nan])


# ------------------------------------------------------------------ int8 ---
def test_int8_page_step_and_threshold():
    """Static scale 127: step 1/127 ~ 0.0079, round-to-zero threshold 0.5/127 ~ 0.0039."""
    s = np.float32(1.0) / np.float32(127.0)
    assert round(float(s), GOLD["int8_step"]["digits"]) == GOLD["int8_step"]["value"]
    assert round(0.5 / 127, GOLD["int8_zero_threshold"]["digits"]) == GOLD["int8_zero_threshold"]["value"]
    assert oracle.quant_i8([0.0039], s)[0] == 0
    assert oracle.quant_i8([0.0040], s)[0] == 1
    assert oracle.quant_i8([1.0], s)[0] == 127


def test_int8_quantizer_properties():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    amax = np.float32(np.abs(x).max())
    s = amax / np.float32(127.0)
    q = oracle.quant_i8(x, s).astype(np.int64)
    assert q.max() <= 127 and q.min() >= -127
    assert abs(q[np.argmax(np.abs(x))]) == 127                  # amax -> +-127
    err = np.abs(x.astype(np.float64) - q * np.float64(s))
    assert err.max() <= 0.5 * float(s) * (1 + 1e-6)
    # exact ties go to even
    ties = (np.arange(-126, 126) + 0.5).astype(np.float32)
    tq = oracle.quant_i8(ties, 1.0).astype(np.int64)
    assert np.all(tq % 2 == 0)
    assert np.all(np.abs(tq - ties) == 0.5)
    # beyond the clamp and zero scale
    assert oracle.quant_i8([1000.0, -1000.0], 1.0).tolist() == [127, -127]
    assert oracle.quant_i8([3.0], 0.0).tolist() == [0]


def test_int_dots_brute_force():
    rng = np.random.default_rng(9)
    a = rng.integers(-127, 128, (37, 128), dtype=np.int64).astype(np.int8)
    b = rng.integers(-127, 128, (53, 128), dtype=np.int64).astype(np.int8)
    acc, ov = oracle.int_dots(a, b)
    assert not ov
    assert np.array_equal(acc, a.astype(np.int64) @ b.astype(np.int64).T)
    # worst case |acc| <= 127^2 * d fits int32 exactly
    full = np.full((1, 128), 127, np.int8)
    acc, ov = oracle.int_dots(full, -full)
    assert acc[0, 0] == -127 * 127 * 128 and not ov


# ----------------------------------------------------------- exact fp64 ---
def _rows_sum(q, k, v, **kw):
    ones = np.ones_like(v)
    return oracle.attn_exact(q, k, ones, **kw)


def test_exact_attention_is_softmax():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 9, 16)).astype(np.float16)
    k = rng.standard_normal((1, 1, 13, 16)).astype(np.float16)
    v = rng.standard_normal((1, 1, 13, 16)).astype(np.float16)
    out = oracle.attn_exact(q, k, v)
    qd, kd, vd = (x.astype(np.float64) for x in (q, k, v))
    s = np.einsum("bhid,bjd->bhij", qd, kd[:, 0]) / 4.0
    w = dg.softmax_rows(s)
    ref = np.einsum("bhij,bjd->bhid", w, vd[:, 0])
    assert np.allclose(out, ref, rtol=0, atol=1e-13)
    assert np.allclose(_rows_sum(q, k, v), 1.0, atol=1e-14)      # weights sum to 1
    # causal: query i sees keys j <= q_offset + i
    outc = oracle.attn_exact(q, k, v, causal=True, q_offset=4)
    mask = np.arange(13)[None, :] <= (4 + np.arange(9))[:, None]
    w = dg.softmax_rows(np.where(mask, s, -np.inf))
    assert np.allclose(outc, np.einsum("bhij,bjd->bhid", w, vd[:, 0]), atol=1e-13)


def test_k_mean_shift_invariance():
    """Subtracting any per-channel vector from K leaves attention unchanged:
    every score of a row moves by the same constant q.mu."""
    c = inputs.config1()
    rng = np.random.default_rng(4)
    mu = rng.standard_normal((1, 1, 128)) * 20
    a = oracle.attn_exact(c.q, c.k, c.v)
    b = oracle.attn_exact(c.q, c.k, c.v, kmu=mu)
    assert np.max(np.abs(a - b)) < 1e-12


# --------------------------------------------------------- KV quantizer ---
def test_kv_quantize_mean_and_ranges():
    c = inputs.small_case(21, hq=4, hkv=2, q_len=8, kv_len=300, batch=2)
    cache = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, capacity=320,
                               v_op_format=oracle.PV_FP8)
    mean = c.k.astype(np.float64).mean(axis=2)                  # numpy's own mean
    assert np.allclose(cache.k_mean, mean.astype(np.float32), rtol=2 ** -23, atol=0)
    kc = cache.k_codes[:, :, :300].astype(np.int64)
    assert np.all(np.abs(kc).max(axis=2) == 127)                 # each channel reaches 127
    x = c.k.astype(np.float32) - cache.k_mean[:, :, None, :]
    err = np.abs(x - kc * cache.k_scales[:, :, None, :])
    assert np.all(err <= 0.5 * cache.k_scales[:, :, None, :] * (1 + 1e-5))
    # rows beyond seq_len untouched
    assert np.all(cache.k_codes[:, :, 300:] == 0)
    # v operand: the documented permutation of e4m3(code); padding keys are zero
    T, p = 2, np.arange(64)
    perm = 32 * ((p % 32) // 16) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4
    assert sorted(perm.tolist()) == list(range(64))
    keys = 64 * T + perm
    want = oracle.e4m3_encode(cache.v_codes[1, 0, keys, 5].astype(np.float32))
    assert np.array_equal(cache.v_op[1, 0, T, 5], want)
    assert np.all(cache.v_op[:, :, 4, :, :][..., keys[keys >= 300] - 256] == 0) or True
    last = cache.v_op[:, :, 4]                                    # keys 256..319
    pad = (256 + perm) >= 300
    assert np.all(last[..., pad] == 0)


def test_kv_quantize_token_scales_fp16():
    c = inputs.config4(kv_len=512)[0]
    cache = oracle.kv_quantize(c.k, c.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN)
    assert cache.k_scales.dtype == np.float16
    kc = cache.k_codes.astype(np.int64)
    x = c.k.astype(np.float32) - cache.k_mean[:, :, None, :]
    amax = np.abs(x).max(axis=3)
    s32 = amax / np.float32(127)
    assert np.array_equal(cache.k_scales, s32.astype(np.float16))   # numpy RNE to fp16
    assert np.all(np.abs(kc).max(axis=3) >= 126)                      # fp16 rounding of s
    vc = cache.v_codes.astype(np.int64)
    assert np.all(np.abs(vc).max(axis=3) >= 126)


def test_k_levels_match_page():
    """On the LLM-like generator the typical channel gets ~3 levels from a
    per-tensor scale before centring and ~31 after (printed 3 -> 31)."""
    k, _, params = inputs.llm_kv(np.random.default_rng(1003), 1, 32768, 128)
    raw = dg.typical_channel_levels(k[0, 0], centred=False)
    cen = dg.typical_channel_levels(k[0, 0], centred=True)
    assert 2.0 <= raw <= 4.5, raw
    assert 25 <= cen <= 40, cen
    r_raw = dg.channel_absmax_ratios(k[0, 0], centred=False)
    r_cen = dg.channel_absmax_ratios(k[0, 0], centred=True)
    top = np.sort(r_raw)[-5:]
    assert np.allclose(top, GOLD["k_outlier_channel_ratios"]["value"], rtol=0.25), top
    assert r_cen.max() <= 4.6


def test_mass_by_decade_matches_figure():
    """Gaussian logits of std 3.4 over 32k keys put the row mass where the
    figure's 32k histogram does (within a few points); the int8 threshold
    flushes far more mass at 32k than at 4k."""
    rng = np.random.default_rng(17)
    p32 = dg.gaussian_logit_rows(rng, 48, 32768, inputs.LOGIT_STD)
    h = dg.mass_by_decade(p32)
    g = GOLD["row_mass_by_decade_32k"]
    assert abs(h[0] - g["below_1e-4"]) < 0.03
    assert abs(h[1] - g["1e-4_1e-3"]) < 0.03
    assert abs(h[2] - g["1e-3_1e-2"]) < 0.04
    assert abs(h[4] - g["above_0.1"]) < 0.04
    p4 = dg.gaussian_logit_rows(rng, 64, 4096, inputs.LOGIT_STD)
    b32, b4 = dg.mass_below(p32), dg.mass_below(p4)
    assert b32 > 1.5 * b4
    assert abs(b32 - GOLD["row_mass_below_int8_threshold"]["32k"]) < 0.08


# ---------------------------------------------------- prefill emulation ---
def _exact_from_codes(q, cache, kv_len, q_offset, causal, pv_mode, q_gran=oracle.GRAN_TOKEN):
    """fp64 attention over the *quantized* scores c*acc (real arithmetic, no
    tiling, no P quantization) with the PV operand's V values: the result the
    emulation must reach up to its P rounding."""
    B, Hq, L, d = q.shape
    H = cache.k_codes.shape[1]
    G = Hq // H
    ksc = cache.k_scales if cache.k_gran == oracle.GRAN_CHANNEL else None
    qc, qs = oracle.quantize_q(q, H, q_gran, ksc)
    kc = oracle.kconst(0.0, d)
    out = np.zeros((B, Hq, L, d))
    vtab = (oracle.e4m3_decode(oracle.e4m3_encode(np.arange(-128, 128).astype(np.float32)))
            if pv_mode == oracle.PV_FP8 else np.arange(-128, 128).astype(np.float64))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            acc = qc[b, h].astype(np.int64) @ cache.k_codes[b, g, :kv_len].astype(np.int64).T
            c = np.float64(np.float32(qs[b, h] * np.float32(kc)))[..., None] * np.ones(1)
            if cache.k_gran == oracle.GRAN_TENSOR:
                c = np.float64(np.float32(np.float32(qs[b, h] * np.float32(kc)) * cache.k_scales[0]))[..., None]
            s = c * acc
            if causal:
                mask = np.arange(kv_len)[None, :] <= (q_offset + np.arange(L))[:, None]
                s = np.where(mask, s, -np.inf)
            w = np.exp2(s - s.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            vv = vtab[cache.v_codes[b, g, :kv_len].astype(np.int64) + 128]
            out[b, h] = (w @ vv) * cache.v_scales[b, g][None, :]
    return out


@pytest.mark.parametrize("pv_mode", [oracle.PV_FP8, oracle.PV_INT8])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_emulation_within_p_rounding_bound(pv_mode, causal):
    """The emulated output differs from exact softmax over the same quantized
    scores only by P's rounding: relative error <= 2^-4 per weight for e4m3
    normal values (plus the subnormal floor), absolute <= 0.5/127 for int8; the
    weights are renormalized by their own (rounded) sum, which at most doubles
    the bound."""
    c = inputs.small_case(31, hq=4, hkv=2, q_len=70, kv_len=333, causal=causal)
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran, capacity=384)
    res = oracle.prefill_emulate(c.q, cache, kv_len=333, q_offset=c.q_offset, causal=causal,
                                 pv_mode=pv_mode)
    ref = _exact_from_codes(c.q, cache, 333, c.q_offset, causal, pv_mode)
    vmax = np.max(np.abs(cache.v_codes).astype(np.float64)) * cache.v_scales.max()
    err = np.abs(res.out - ref).max()
    if pv_mode == oracle.PV_FP8:
        bound = 2 * (2.0 ** -4 + 333 * 2.0 ** -10 / 448) * vmax
    else:
        bound = 2 * 333 * 0.5 / 127 * vmax
    assert err <= bound, (err, bound)
    assert err > 0          # P really was quantized
    # and the fp8 path is markedly closer than the bound
    if pv_mode == oracle.PV_FP8:
        assert err < 0.3 * bound


def test_prefill_emulation_p_codes_bounded_and_max_is_448():
    c = inputs.small_case(41, hq=2, hkv=1, q_len=40, kv_len=200)
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran, capacity=256)
    res = oracle.prefill_emulate(c.q, cache, kv_len=200, q_offset=0, causal=False, want_p=True,
                                 want_s=True)
    p = res.p_codes
    assert p.max() <= 0x7E and not np.any((p & 0x7F) == 0x7F)     # P <= 448, no NaN
    assert np.all(p < 0x80)                                        # P >= 0
    # the row's arg-max key carries exactly 448
    qc, _ = oracle.quantize_q(c.q, 1, oracle.GRAN_TOKEN, cache.k_scales)
    for h in range(2):
        acc, _ = oracle.int_dots(qc[0, h], cache.k_codes[0, 0, :200])
        assert np.array_equal(acc, res.s_i32[0, h])                # int32 dots: brute force
        am = np.argmax(acc, axis=1)
        assert np.all(p[0, h, np.arange(40), am] == 0x7E)


def test_prefill_special_cases():
    d = 128
    rng = np.random.default_rng(8)
    # (a) every key identical -> uniform weights -> mean of the V operand values
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), 100, axis=2).astype(np.float16)
    v = rng.standard_normal((1, 1, 100, d)).astype(np.float16)
    q = rng.standard_normal((1, 1, 5, d)).astype(np.float16)
    cache = oracle.kv_quantize(k, v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, capacity=128)
    assert np.all(cache.k_codes[:, :, :100] == 0)             # amax 0 -> scale 0 -> codes 0
    res = oracle.prefill_emulate(q, cache, kv_len=100, q_offset=0, causal=False)
    vv = oracle.e4m3_decode(oracle.e4m3_encode(cache.v_codes[0, 0, :100].astype(np.float32)))
    want = vv.mean(axis=0) * cache.v_scales[0, 0]
    assert np.allclose(res.out[0, 0], want[None, :], rtol=1e-12, atol=1e-15)
    # (b) one key -> its V operand value exactly
    res1 = oracle.prefill_emulate(q, cache, kv_len=1, q_offset=0, causal=False)
    assert np.allclose(res1.out[0, 0], (vv[0] * cache.v_scales[0, 0])[None, :], rtol=1e-12, atol=0)
    # (c) Q = 0 -> uniform weights even for distinct keys
    k2 = rng.standard_normal((1, 1, 100, d)).astype(np.float16)
    cache2 = oracle.kv_quantize(k2, v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, capacity=128)
    res0 = oracle.prefill_emulate(np.zeros_like(q), cache2, kv_len=100, q_offset=0, causal=False)
    assert np.allclose(res0.out[0, 0], want[None, :], rtol=1e-12, atol=1e-15)
    # (d) one dominant key (+50 logits) -> that key's value within e4m3 error
    q3 = np.zeros((1, 1, 1, d), np.float16)
    q3[..., 0] = 8.0
    k3 = np.zeros((1, 1, 100, d), np.float16)
    k3[0, 0, 37, 0] = 50.0 * np.sqrt(d) / 8.0
    cache3 = oracle.kv_quantize(k3, v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL,
                                subtract_mean=False, capacity=128)
    res3 = oracle.prefill_emulate(q3, cache3, kv_len=100, q_offset=0, causal=False)
    target = vv[37] * cache3.v_scales[0, 0]
    # every other key is 2^-72 below it: flushed in its own stream, and the second
    # stream (keys 64..99, all equal) enters the merge with weight 2^-72
    assert np.allclose(res3.out[0, 0, 0], target, rtol=1e-12, atol=1e-15 * np.abs(target).max())


def _rel_err(a, e):
    """row-infinity-normalised max error"""
    den = np.abs(e).max(axis=-1, keepdims=True)
    return float(np.max(np.abs(a - e) / den))


def _cos(a, b):
    a, b = a.ravel(), b.ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def test_prefill_cosine_vs_fp64_config1():
    """Config 1 is the stress case: five K channels carry x40 *variance*
    outliers, which the mean subtraction cannot remove, and its rows are very
    peaked (logit std ~8).  Per-channel K scales folded into Q keep the scheme
    at cosine ~0.998 against fp64 (Q's own int8 rounding is the largest term),
    and the page's ordering holds: the naive per-tensor int8 QK with no K
    smoothing is several times worse."""
    c = inputs.config1()
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran)
    exact = oracle.attn_exact(c.q, c.k, c.v)
    fp8 = oracle.prefill_emulate(c.q, cache, kv_len=256, q_offset=0, causal=False)
    # the scheme's level here, which misses the 0.999 bar of the LLM-like workloads (the GPU
    # reaches the same value; its 0.999 test is a strict expected failure)
    assert 0.998 <= _cos(fp8.out, exact) < 0.999
    naive = oracle.kv_quantize(c.k, c.v, oracle.GRAN_TENSOR, c.v_gran, subtract_mean=False)
    nv = oracle.prefill_emulate(c.q, naive, kv_len=256, q_offset=0, causal=False)
    assert (1 - _cos(nv.out, exact)) > 3 * (1 - _cos(fp8.out, exact))


def test_fp8_pv_beats_int8_pv_at_long_context():
    """The page's finding: int8 P flushes the diffuse tail and its error grows
    with context; e4m3 P keeps it.  Checked on sampled rows of a 32k-key,
    Gaussian-logit (std 3.4) workload."""
    c = inputs.config3(q_len=64, kv_len=8192, hq=4, hkv=1)
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran)
    rows = np.arange(0, 4 * 64, 7)
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=True, q_offset=c.q_offset, rows=rows)
    kw = dict(kv_len=8192, q_offset=c.q_offset, causal=True, rows=rows)
    f8 = oracle.prefill_emulate(c.q, cache, pv_mode=oracle.PV_FP8, **kw)
    i8 = oracle.prefill_emulate(c.q, cache, pv_mode=oracle.PV_INT8, **kw)
    e = exact.reshape(-1, 128)[rows]
    a8 = f8.out.reshape(-1, 128)[rows]
    ai = i8.out.reshape(-1, 128)[rows]
    assert _cos(a8, e) >= 0.999
    assert _rel_err(a8, e) < _rel_err(ai, e)
    assert f8.n_flushed < i8.n_flushed


# ----------------------------------------------------- decode emulation ---
def test_decode_emulation_pins():
    c = inputs.config4(kv_len=700)[0]
    cache = oracle.kv_quantize(c.k, c.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN)
    q = c.q[:, :, 0]
    out, dots = oracle.decode_emulate(q, cache, kv_len=700, want_qk=True)
    # int32 dots equal a brute-force product of the same codes
    qs = np.abs(q.astype(np.float32)).max(axis=-1) / np.float32(127)
    for h in range(16):
        qc = oracle.quant_i8(q[0, h].astype(np.float32), qs[0, h])
        assert np.array_equal(dots[0, h], cache.k_codes[0, h // 4, :700].astype(np.int64) @ qc.astype(np.int64))
    # close to fp64 attention on the fp16 inputs
    exact = oracle.attn_exact(c.q, c.k, c.v)[:, :, 0]
    assert _cos(out, exact) >= 0.999
    # one key -> its dequantized value; Q = 0 -> mean of dequantized V
    o1, _ = oracle.decode_emulate(q, cache, kv_len=1)
    vdq = cache.v_codes[0, :, :700].astype(np.float64) * cache.v_scales[0, :, :700, None].astype(np.float64)
    assert np.allclose(o1[0], np.repeat(vdq[:, 0], 4, axis=0), rtol=1e-12, atol=0)
    o0, _ = oracle.decode_emulate(np.zeros_like(q), cache, kv_len=700)
    assert np.allclose(o0[0], np.repeat(vdq.mean(axis=1), 4, axis=0), rtol=1e-10, atol=1e-12)


# ------------------------------------------- readings of the online softmax ---
def _p_rounding_bound(n_keys, vmax, fp32_norm):
    """Bound on |out - exact| for an online softmax whose numerator weights are e4m3 codes
    of w_j = 448 * 2^(s_j - max): each code is within 2^-4 * w_j (normal range) or 2^-10
    (subnormal half step) of w_j, the largest weight is 448 exactly, so with numerator
    weights w'_j and normalizer l',
      out - e = sum_j (w'_j - w_j)(v_j - e) / l'          (l' = sum w'_j, quantized P)
      out - e = [sum_j (w'_j - w_j) v_j + e (sum w_j - l')] / l'   (l' = sum of fp32 p)
    and |v_j - e| <= 2 vmax."""
    rel = 2.0 ** -4 + n_keys * 2.0 ** -10 / 448.0
    if fp32_norm:
        return 2.0 * rel * vmax / (1.0 - 2.0 ** -20)
    return 2.0 * rel / (1.0 - rel) * vmax


def test_stream_split_and_normalizer_readings_are_bounded():
    """The built readings -- key tiles dealt to two interleaved online softmaxes merged at
    the end, normalizer l = sum of the quantized weights -- against the plain reading (one
    stream over all tiles, l = sum of the unquantized fp32 p).  All four combinations stay
    within the P-rounding bound of exact softmax over the same quantized scores, so any two
    differ by at most the sum of their bounds; the measured distances on the 8192-key
    LLM-like rows are recorded here (the tile grouping decides which p's round up or down,
    nothing else)."""
    c = inputs.config3(q_len=64, kv_len=8192, hq=4, hkv=1)
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran)
    rows = np.arange(0, 4 * 64, 5)
    kw = dict(kv_len=8192, q_offset=c.q_offset, causal=True, rows=rows)
    ref = _exact_from_codes(c.q, cache, 8192, c.q_offset, True, oracle.PV_FP8).reshape(-1, 128)[rows]
    vmax = float(np.max(np.abs(cache.v_codes).astype(np.float64)) * cache.v_scales.max())
    outs = {}
    for ns in (2, 1):
        for nf in (False, True):
            o = oracle.prefill_emulate(c.q, cache, n_streams=ns, norm_fp32=nf, **kw).out.reshape(-1, 128)[rows]
            assert np.abs(o - ref).max() <= _p_rounding_bound(8192, vmax, nf)
            outs[(ns, nf)] = o
    built, plain = outs[(2, False)], outs[(1, True)]
    d_stream = _rel_err(outs[(1, False)], built)
    d_norm = _rel_err(outs[(2, True)], built)
    d_both = _rel_err(plain, built)
    print(f"reading distances (row-normalised): stream split {d_stream:.2e}, normalizer {d_norm:.2e}, "
          f"both {d_both:.2e}")
    b = _p_rounding_bound(8192, vmax, False) + _p_rounding_bound(8192, vmax, True)
    assert np.abs(plain - built).max() <= b
    # the readings really differ (P is quantized against different running maxima) but by
    # P rounding only: well below the bound, and each is as close to fp64 as the others
    assert 0 < d_stream < 0.02 and 0 < d_norm < 0.02 and 0 < d_both < 0.03
    exact = oracle.attn_exact(c.q, c.k, c.v, causal=True, q_offset=c.q_offset, rows=rows).reshape(-1, 128)[rows]
    cs = [_cos(o, exact) for o in outs.values()]
    assert min(cs) >= 0.999 and max(cs) - min(cs) < 1e-5


def test_one_tile_rows_do_not_depend_on_the_stream_split():
    """With every visible key in one tile, stream 1 holds nothing: the two-stream and
    one-stream emulations are the same computation, bit for bit."""
    c = inputs.small_case(44, hq=4, hkv=2, q_len=30, kv_len=64)
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran, capacity=64)
    a = oracle.prefill_emulate(c.q, cache, kv_len=64, q_offset=0, causal=False, n_streams=2).out
    b = oracle.prefill_emulate(c.q, cache, kv_len=64, q_offset=0, causal=False, n_streams=1).out
    assert np.array_equal(a, b)


def test_exponent_is_one_rounding_of_c_acc_minus_mL():
    """The exponent of p is fp32(c*acc - mL) rounded once: in a one-key row, p = 448 exactly
    (acc = acc_max, so c*acc - mL = log2 448 exactly when rounded once); and every P code of
    a small case equals e4m3 of 2^x with x = c*acc - mL computed here in fp64 (the product
    of the fp32 c and the integer acc < 2^22 is exact; the difference is rounded to 53 bits
    before its rounding to fp32, which can differ from a single rounding only for an exact
    fp32 tie after the first, about 2^-29 per element)."""
    c = inputs.small_case(45, hq=2, hkv=1, q_len=20, kv_len=150)
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran, capacity=192)
    res = oracle.prefill_emulate(c.q, cache, kv_len=150, q_offset=0, causal=False, want_p=True, want_s=True,
                                 n_streams=1, block_c=256)
    qc, qs = oracle.quantize_q(c.q, 1, oracle.GRAN_TOKEN, cache.k_scales)
    kc = np.float32(oracle.kconst(0.0, 128))
    L = np.float32(np.log2(448.0))
    for h in range(2):
        acc = res.s_i32[0, h].astype(np.int64)
        cc = (qs[0, h] * kc).astype(np.float32)[:, None]
        s2 = (cc.astype(np.float64) * acc).astype(np.float32)          # fp32(c * acc)
        m = s2.max(axis=1, keepdims=True)
        mL = (m.astype(np.float64) - np.float64(L)).astype(np.float32)
        x = (cc.astype(np.float64) * acc - mL.astype(np.float64)).astype(np.float32)   # exact, rounded once
        p = np.exp2(x.astype(np.float64)).astype(np.float32)
        assert np.array_equal(oracle.e4m3_encode(p), res.p_codes[0, h])



# ------------------------------------------------------------ Q quantizer ---
def test_quantize_q_independent_of_the_oracle():
    """q' = fp32(q) * s_K[b, h // G, c] (per-channel K folded in, G = Hq / Hkv query heads per
    kv head), s_Q = fp32(amax / 127) per row (TOKEN) or over the whole call (TENSOR), codes
    rint(q' / s_Q) clamped to +-127 -- computed with numpy float32 arithmetic (IEEE, one
    rounding per operation) on a batch of 2 with 3 kv heads of 2 query heads each, so a
    wrong kv-head or batch index for the folded scales, or an amax taken over the wrong set,
    changes codes."""
    rng = np.random.default_rng(77)
    Bn, Hq, Hkv, L, d = 2, 6, 3, 11, 64
    q = (rng.standard_normal((Bn, Hq, L, d)) * np.exp(rng.uniform(-1, 1, (Bn, Hq, 1, 1)))).astype(np.float16)
    ks = np.exp(rng.uniform(-3, 1, (Bn, Hkv, d))).astype(np.float32)   # distinct per (b, g, c)
    G = Hq // Hkv
    qp = q.astype(np.float32) * ks[:, np.repeat(np.arange(Hkv), G)][:, :, None, :]
    for gran in (oracle.GRAN_TOKEN, oracle.GRAN_TENSOR):
        codes, scales = oracle.quantize_q(q, Hkv, gran, ks)
        amax = np.abs(qp).max(axis=-1) if gran == oracle.GRAN_TOKEN else np.full((Bn, Hq, L), np.abs(qp).max())
        s = (amax / np.float32(127)).astype(np.float32)
        want = np.clip(np.rint(qp / s[..., None]), -127, 127).astype(np.int8)
        assert np.array_equal(scales.view(np.uint32), s.view(np.uint32))
        assert np.array_equal(codes, want)
        # TOKEN: every row reaches +-127; TENSOR: exactly the rows holding the global amax do
        peak = np.abs(codes.astype(np.int64)).max(axis=-1)
        assert np.all(peak == 127) if gran == oracle.GRAN_TOKEN else peak.max() == 127 and peak.min() < 127
    # without per-channel K scales nothing is folded
    codes, scales = oracle.quantize_q(q, Hkv, oracle.GRAN_TOKEN, None)
    s = (np.abs(q.astype(np.float32)).max(axis=-1) / np.float32(127)).astype(np.float32)
    assert np.array_equal(codes, np.clip(np.rint(q.astype(np.float32) / s[..., None]), -127, 127).astype(np.int8))


def test_flushed_mass_diagnostic():
    """The flushed-mass diagnostic against a direct computation: the softmax of the row's
    quantized scores c*acc in fp64 (numpy), summed over the keys whose P code the emulation
    reports as zero; and int8 P flushes far more mass than e4m3 P (the first figure's
    point: 0.5/127 is a coarse floor, 2^-10 / 448 is not)."""
    c = inputs.config3(q_len=16, kv_len=4096, hq=2, hkv=1)
    cache = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran)
    kw = dict(kv_len=4096, q_offset=c.q_offset, causal=True, want_p=True, want_s=True, n_streams=1,
              block_c=8192)
    r8 = oracle.prefill_emulate(c.q, cache, **kw)
    ri = oracle.prefill_emulate(c.q, cache, pv_mode=oracle.PV_INT8, **kw)
    _, qs = oracle.quantize_q(c.q, 1, oracle.GRAN_TOKEN, cache.k_scales)
    cc = (qs * np.float32(oracle.kconst(0.0, 128))).astype(np.float32).astype(np.float64)
    s = cc[..., None] * r8.s_i32.astype(np.float64)
    vis = np.arange(4096)[None, :] <= (c.q_offset + np.arange(16))[:, None]
    s = np.where(vis[None, None], s, -np.inf)
    w = np.exp2(s - s.max(axis=-1, keepdims=True))
    w /= w.sum(axis=-1, keepdims=True)
    for r in (r8, ri):
        want = np.sum(np.where((r.p_codes == 0) & vis[None, None], w, 0.0), axis=-1)
        assert np.allclose(r.flushed_mass, want, rtol=1e-9, atol=1e-15)
    assert np.mean(ri.flushed_mass) > 5 * np.mean(r8.flushed_mass)


# ------------------------------------------------------- per-token K and V ---
def _token_cache(seed=47, N=300, cap=320, hkv=2, hq=4, q_len=40):
    c = inputs.small_case(seed, hq=hq, hkv=hkv, q_len=q_len, kv_len=N)
    cache = oracle.kv_quantize(c.k, c.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, capacity=cap,
                               v_op_format=oracle.PV_FP8)
    return c, cache


def test_token_v_operand_bytes():
    """Per-token V operand: f_n = fp32(s_V[n] * c_V), c_V = fp32(448 / fp32(127 * V_max)) with
    V_max the largest per-token scale of the head (the header), byte = e4m3(fp32(code * f_n))
    in the permuted tile order -- recomputed here with numpy float32 arithmetic; every value
    stays within the static bound 448, and the token holding V_max reaches it."""
    c, cache = _token_cache()
    N = 300
    vs = cache.v_scales[:, :, :N].astype(np.float32)
    vmax = vs.max(axis=2)
    assert np.array_equal(cache.v_scale_max.view(np.uint32), vmax.view(np.uint32))
    cv = (np.float32(448) / (np.float32(127) * vmax)).astype(np.float32)
    f = (vs * cv[:, :, None]).astype(np.float32)
    x = (cache.v_codes[:, :, :N].astype(np.float32) * f[..., None]).astype(np.float32)
    want = oracle.e4m3_encode(x)                                        # [B][H][N][d]
    p = np.arange(64)
    perm = 32 * ((p % 32) // 16) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4
    for T in range(5):
        keys = 64 * T + perm
        ok = keys < N
        got = cache.v_op[:, :, T][..., ok]                               # [B][H][d][valid]
        assert np.array_equal(got, np.transpose(want[:, :, keys[ok]], (0, 1, 3, 2)))
        assert np.all(cache.v_op[:, :, T][..., ~ok] == 0)
    dec = oracle.e4m3_decode(cache.v_op)
    assert np.abs(dec).max() <= 448.0
    for g in range(2):   # the largest-scale token's largest code lands on the bound (or next to it)
        n = int(np.argmax(vs[0, g]))
        assert np.abs(dec[0, g, n // 64]).max() >= 416.0


def test_token_kv_emulation_within_p_rounding_bound():
    """Per-token K scales (c_j = fp32(c * s_K[j]) per key: no integer row max) and per-token V
    (operand carrying s_V[n] * c_V, output times 1 / c_V): the emulation differs from exact
    softmax over the same quantized scores c_j * acc_j with the operand's V values only by P's
    rounding (the bound of test_prefill_emulation_within_p_rounding_bound)."""
    c, cache = _token_cache()
    N, d = 300, 128
    res = oracle.prefill_emulate(c.q, cache, kv_len=N, q_offset=0, causal=False, want_s=True)
    qc, qs = oracle.quantize_q(c.q, 2, oracle.GRAN_TOKEN, None)          # nothing folded into Q
    kc = np.float32(oracle.kconst(0.0, d))
    vmax = cache.v_scale_max
    cv = (np.float32(448) / (np.float32(127) * vmax)).astype(np.float32)
    p = np.arange(64)
    perm = 32 * ((p % 32) // 16) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4
    vop = np.zeros((1, 2, N, d))
    dec = oracle.e4m3_decode(cache.v_op)
    for T in range(5):
        keys = 64 * T + perm
        ok = keys < N
        vop[:, :, keys[ok]] = np.transpose(dec[:, :, T][..., ok], (0, 1, 3, 2))
    for h in range(4):
        g = h // 2
        acc = qc[0, h].astype(np.int64) @ cache.k_codes[0, g, :N].astype(np.int64).T
        assert np.array_equal(acc, res.s_i32[0, h])
        cj = ((qs[0, h] * kc).astype(np.float32)[:, None] * cache.k_scales[0, g, :N].astype(np.float32)[None, :])
        s = cj.astype(np.float32).astype(np.float64) * acc
        w = np.exp2(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        ref = (w @ vop[0, g]) / np.float64(cv[0, g])
        vmaxv = np.abs(vop[0, g]).max() / np.float64(cv[0, g])
        bound = 2 * (2.0 ** -4 + N * 2.0 ** -10 / 448) / (1 - 2.0 ** -4 - N * 2.0 ** -10 / 448) * vmaxv
        err = np.abs(res.out[0, h] - ref).max()
        assert 0 < err <= bound, (err, bound)


def test_token_kv_special_cases_and_accuracy():
    """One key: the output is that key's V operand value times 1 / c_V, within e4m3's 2^-4 of
    s_V * code; and on the decode workload's per-token cache the emulated prefill reaches
    cosine >= 0.999 against fp64 attention on the fp16 inputs."""
    c, cache = _token_cache()
    res1 = oracle.prefill_emulate(c.q, cache, kv_len=1, q_offset=0, causal=False)
    vdq = cache.v_codes[0, :, 0].astype(np.float64) * cache.v_scales[0, :, 0, None].astype(np.float64)
    for h in range(4):
        assert np.all(np.abs(res1.out[0, h] - vdq[h // 2]) <= 2.0 ** -4 * np.abs(vdq[h // 2]) + 1e-12)
    c4 = inputs.config3(q_len=64, kv_len=4096, hq=4, hkv=1)
    cache4 = oracle.kv_quantize(c4.k, c4.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, v_op_format=oracle.PV_FP8)
    rows = np.arange(0, 256, 3)
    out = oracle.prefill_emulate(c4.q, cache4, kv_len=4096, q_offset=c4.q_offset, causal=True, rows=rows)
    exact = oracle.attn_exact(c4.q, c4.k, c4.v, causal=True, q_offset=c4.q_offset, rows=rows)
    assert _cos(out.out.reshape(-1, 128)[rows], exact.reshape(-1, 128)[rows]) >= 0.999


def test_v_operand_rebuild_equals_quantize():
    """Rebuilding the operand from the cache's codes and scales (what follows an append)
    gives kv_quantize's bytes and header; built over fewer keys, the tail tiles are zero."""
    c, cache = _token_cache()
    op, vm = cache.v_op.copy(), cache.v_scale_max.copy()
    oracle.v_operand(cache, 300)
    assert np.array_equal(cache.v_op, op) and np.array_equal(cache.v_scale_max, vm)
    cc, ch = _token_cache(seed=48, N=300, cap=320)
    cc2 = oracle.kv_quantize(cc.k, cc.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, capacity=320,
                             v_op_format=oracle.PV_FP8)
    op2 = cc2.v_op.copy()
    oracle.v_operand(cc2, 300)
    assert np.array_equal(cc2.v_op, op2)
    oracle.v_operand(cc2, 100)
    assert np.all(cc2.v_op[:, :, 2:] == 0)

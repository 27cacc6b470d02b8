"""Pins of the oracle's MX path (Q and K below 8 bits on the matrix core's fp6 / fp4 operand
types; "int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8", closing section, asks
whether Q and K survive four bits).  The encoding follows the OCP Microscaling Formats v1.0
definition (E2M1 / E2M3 elements, one E8M0 scale per 32 elements, X = 2^(floor(log2 amax) -
2)); the emulation's MX scores are pinned to its integer-score path on inputs where both
compute the same dots."""
import dataclasses

import numpy as np
import pytest

import oracle

# the element grids written out from the format definitions (OCP MX v1.0: E2M1 = 1 sign,
# 2 exponent bits with bias 1, 1 mantissa bit; E2M3 = 2 exponent bits, 3 mantissa bits;
# exponent field 0 is subnormal with the exponent of field 1)
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
E2M3 = np.array([m / 8 for m in range(8)] + [(1 + m / 8) * 2.0 ** (e - 1) for e in (1, 2, 3) for m in range(8)])
FMTS = [(oracle.LB_MXFP4, E2M1, 8), (oracle.LB_MXFP6, E2M3, 32)]


def _decode(codes, grid, sign_bit):
    mag = grid[codes & (sign_bit - 1)]
    return np.where(codes & sign_bit, -mag, mag)


@pytest.mark.parametrize("fmt,grid,sign_bit", FMTS, ids=["mxfp4", "mxfp6"])
def test_mx_scale_is_the_block_exponent_and_elements_the_nearest_grid_point(fmt, grid, sign_bit):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-6, 6, (40, 1)))).astype(np.float32)
    x[3, 40:64] *= 300.0                       # one block with an outlier range
    e = oracle.mx_quantize(x, fmt)
    xb = x.reshape(40, 4, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    _, E = np.frexp(amax)                       # amax = m * 2^E, m in [0.5, 1)
    want_e = E - 1 - 2
    assert np.array_equal(e.scale_bytes.astype(int), 127 + want_e)
    X = np.ldexp(1.0, want_e)[:, :, None]
    y = xb / X
    assert np.all(np.abs(y) < 8)
    vals = e.values.reshape(40, 4, 32) / X
    # nearest grid point (no grid value strictly closer), sign restored
    d_best = np.abs(np.abs(y)[..., None] - grid).min(axis=-1)
    assert np.all(np.abs(np.abs(y) - np.abs(vals)) <= d_best + 0.0)
    assert np.all((vals == 0) | (np.sign(vals) == np.sign(y)))
    # codes decode to the values; a zero element carries no sign
    dec = _decode(e.codes.reshape(40, 4, 32).astype(int), grid, sign_bit) * X
    assert np.array_equal(dec, e.values.reshape(40, 4, 32))
    assert not np.any((e.codes & (sign_bit - 1) == 0) & (e.codes != 0))


@pytest.mark.parametrize("fmt,grid,sign_bit", FMTS, ids=["mxfp4", "mxfp6"])
def test_mx_ties_saturation_and_exact_values(fmt, grid, sign_bit):
    top = grid[-1]
    # a block whose amax is 4 (so X = 1): midpoints of neighbouring grid values go to the even code
    mids = (grid[:-1] + grid[1:]) / 2
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 4.0
    x[0, 1:1 + len(mids[:20])] = mids[:20]
    e = oracle.mx_quantize(x, fmt)
    assert e.scale_bytes[0, 0] == 127
    for i, m in enumerate(mids[:20]):
        lo, hi = np.searchsorted(grid, m) - 1, np.searchsorted(grid, m)
        want = grid[lo] if lo % 2 == 0 else grid[hi]
        assert e.values[0, 1 + i] == want, (m, e.values[0, 1 + i], want)
    # saturation: x / X in (max, 8) gives the largest magnitude
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 7.99, -7.9, top + (8 - top) / 3
    e = oracle.mx_quantize(x, fmt)
    assert e.scale_bytes[0, 0] == 127 and np.all(np.abs(e.values[0, :3]) == top)
    # values already on the scaled grid are kept exactly; an all-zero block has X = 1
    rng = np.random.default_rng(3)
    g = rng.choice(np.concatenate([grid, -grid[1:]]), (8, 64))
    g[:, 0], g[:, 32] = top, -top
    x = (g * 2.0 ** rng.integers(-20, 20, (8, 1))).astype(np.float32)
    e = oracle.mx_quantize(x, fmt)
    assert np.array_equal(e.values, x.astype(np.float64))
    z = oracle.mx_quantize(np.zeros((2, 32), np.float32) - 0.0, fmt)
    assert np.all(z.scale_bytes == 127) and np.all(z.codes == 0) and np.all(z.values == 0)


def test_mx_values_match_the_grid_study_rows():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    for fmt in (oracle.LB_MXFP4, oracle.LB_MXFP6):
        e = oracle.mx_quantize(x, fmt)
        for r in range(6):
            assert np.array_equal(e.values[r], oracle.lowbit_row(x[r], fmt))


def test_mx_scores_reduce_to_the_integer_path():
    """With Q and K integers in [-7, 7] and a +-7 in every 32-channel block, both MX grids hold
    them exactly with X = 1, so the MX dots equal the int32 dots; with s_Q = 1 the row constant
    of both paths is kconst, and P, the outputs and the LSE agree bit for bit."""
    rng = np.random.default_rng(5)
    B, Hq, H, L, N, d = 1, 4, 2, 70, 300, 128
    qi = rng.integers(-7, 8, (B, Hq, L, d))
    ki = rng.integers(-7, 8, (B, H, N, d))
    qi[..., ::32] = 7
    ki[..., ::32] = -7
    v = rng.standard_normal((B, H, N, d)).astype(np.float16)
    cache = oracle.kv_quantize(ki.astype(np.float16), v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL,
                               subtract_mean=False, capacity=320, v_op_format=oracle.PV_FP8)
    kcodes = np.zeros_like(cache.k_codes)
    kcodes[:, :, :N] = ki
    icache = dataclasses.replace(cache, k_codes=kcodes)
    q16 = qi.astype(np.float16)
    ref = oracle.prefill_emulate(q16, icache, kv_len=N, q_offset=N - L, causal=True, want_p=True,
                                 q_quant=(qi.astype(np.int8), np.ones((B, Hq, L), np.float32)))
    for fmt in (oracle.LB_MXFP6,):   # (E2M1 lacks 5 and 7: the next test)
        kenc = oracle.k_quantize_mx(ki.astype(np.float16), np.zeros((B, H, d), np.float32), fmt, capacity=320)
        assert np.array_equal(kenc.values[:, :, :N], ki.astype(np.float64))
        mx = oracle.mx_operands(q16, fmt, kenc)
        assert np.array_equal(mx.q_values, qi.astype(np.float64))
        got = oracle.prefill_emulate(q16, cache, kv_len=N, q_offset=N - L, causal=True, want_p=True, want_s=True,
                                     mx=mx)
        assert np.array_equal(got.out, ref.out)
        assert np.array_equal(got.p_codes, ref.p_codes)
        assert np.array_equal(got.lse, ref.lse)
        vis = np.arange(N)[None, :] <= (N - L + np.arange(L))[:, None]
        dots = np.einsum("bhlc,bhnc->bhln", qi.astype(np.int64), np.repeat(ki, Hq // H, axis=1).astype(np.int64))
        assert np.array_equal(got.s_i32[..., vis], dots[..., vis].astype(np.float32))


def test_mx_fp4_integer_grid_reduces_to_the_integer_path():
    """The same reduction for E2M1, whose integers in [-6, 6] are 0, 1, 2, 3, 4, 6: Q and K
    drawn from them with a +-6 (amax in [4, 8), X = 1) in every block."""
    rng = np.random.default_rng(6)
    B, Hq, H, L, N, d = 1, 2, 1, 40, 200, 64
    vals = np.array([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6])
    qi = rng.choice(vals, (B, Hq, L, d))
    ki = rng.choice(vals, (B, H, N, d))
    qi[..., ::32] = 6
    ki[..., ::32] = -6
    v = rng.standard_normal((B, H, N, d)).astype(np.float16)
    cache = oracle.kv_quantize(ki.astype(np.float16), v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL,
                               subtract_mean=False, capacity=256, v_op_format=oracle.PV_FP8)
    kcodes = np.zeros_like(cache.k_codes)
    kcodes[:, :, :N] = ki
    ref = oracle.prefill_emulate(qi.astype(np.float16), dataclasses.replace(cache, k_codes=kcodes), kv_len=N,
                                 q_offset=0, causal=False, want_p=True,
                                 q_quant=(qi.astype(np.int8), np.ones((B, Hq, L), np.float32)))
    kenc = oracle.k_quantize_mx(ki.astype(np.float16), np.zeros((B, H, d), np.float32), oracle.LB_MXFP4,
                                capacity=256)
    got = oracle.prefill_emulate(qi.astype(np.float16), cache, kv_len=N, q_offset=0, causal=False, want_p=True,
                                 mx=oracle.mx_operands(qi.astype(np.float16), oracle.LB_MXFP4, kenc))
    assert np.array_equal(got.out, ref.out) and np.array_equal(got.p_codes, ref.p_codes)


def test_mx_emulation_tracks_the_fp64_grid_attention():
    """The emulated MX prefill (fp32 scores, e4m3 P, fp8 PV) against fp64 attention over the
    same dequantized Q and K (the grid study): the only differences are the P / V operand
    roundings and the score rounding, so the two are close."""
    from quantized_attention_attn_amd import inputs
    c = inputs.small_case(31, hq=4, hkv=2, q_len=64, kv_len=256, causal=True)
    N = 256
    cache = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, capacity=256,
                               v_op_format=oracle.PV_FP8)
    for fmt in (oracle.LB_MXFP6, oracle.LB_MXFP4):
        kenc = oracle.k_quantize_mx(c.k, cache.k_mean, fmt, capacity=256)
        got = oracle.prefill_emulate(c.q, cache, kv_len=N, q_offset=c.q_offset, causal=True,
                                     mx=oracle.mx_operands(c.q, fmt, kenc))
        grid = oracle.attn_lowbit(c.q, c.k, c.v, fmt, fmt, causal=True, q_offset=c.q_offset)
        a, e = got.out.ravel(), grid.ravel()
        cos = a @ e / np.sqrt((a @ a) * (e @ e))
        assert cos > 0.999, (fmt, cos)

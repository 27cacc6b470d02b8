"""Pins of the oracle's BLOCK granularity (one scale per block of 64 tokens of a (batch, head)):
K codes and scales, Q codes and scales, the prefill emulation's per-block dequantization
constant and the decode emulation's.  Per-block quantization follows "QFlash: Bridging
Quantization and Memory Efficiency in Vision Transformer Attention", section 3.3 (C3,
quantization granularity) with the blocks of its Algorithm 1; the symmetric amax/127
quantizer is its eq. (1)-(2).

Each pin checks the oracle against something other than itself: a single block reduces to
per-tensor scales (the oracle's TENSOR path, an independent branch), and tiny cases are
recomputed here with numpy from the definitions."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _fp16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def _mean_fp32(k16):
    # exact per-channel sum of fp16 values (multiples of 2^-24), mean rounded once to fp32
    s = np.round(k16.astype(np.float64) * 2.0 ** 24).astype(np.int64).sum(axis=2)
    n = k16.shape[2]
    return (s.astype(np.float64) / (n * 2.0 ** 24)).astype(np.float32)


def _quant(x32, s32):
    # code = clamp(RNE(fp32(x / s)), -127, 127); 0 for a zero scale
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x32 / s32).astype(np.float32)
    r = np.clip(np.rint(t), -127, 127)
    return np.where(s32 == 0, 0, r).astype(np.int8)


def test_single_key_block_equals_tensor_scale():
    rng = np.random.default_rng(11)
    k = _fp16(rng, (1, 1, 50, 32)); v = _fp16(rng, (1, 1, 50, 32))
    cb = oracle.kv_quantize(k, v, oracle.GRAN_BLOCK, oracle.GRAN_CHANNEL, capacity=64)
    ct = oracle.kv_quantize(k, v, oracle.GRAN_TENSOR, oracle.GRAN_CHANNEL, capacity=64)
    assert cb.k_scales.shape == (1, 1, 1)
    assert cb.k_scales[0, 0, 0] == ct.k_scales[0]
    assert np.array_equal(cb.k_codes, ct.k_codes)


def test_key_blocks_brute_force():
    rng = np.random.default_rng(12)
    B, H, N, d, cap = 1, 2, 150, 16, 192
    k = _fp16(rng, (B, H, N, d), 2.0); v = _fp16(rng, (B, H, N, d))
    k[0, 1, 70] = 40.0                      # one block with a large outlier row
    k[0, 0, 128:] = 0.0                     # a partial last block of zeros (after the mean shift: -mu)
    c = oracle.kv_quantize(k, v, oracle.GRAN_BLOCK, oracle.GRAN_TOKEN, capacity=cap)
    mu = _mean_fp32(k)
    x = (k.astype(np.float32) - mu[:, :, None, :]).astype(np.float32)
    for b in range(B):
        for h in range(H):
            for blk in range(cap // 64):
                n0, n1 = 64 * blk, min(N, 64 * blk + 64)
                if n0 >= N:
                    continue
                s = np.float32(np.abs(x[b, h, n0:n1]).max()) / np.float32(127.0)
                assert c.k_scales[b, h, blk] == np.float32(s), (h, blk)
                assert np.array_equal(c.k_codes[b, h, n0:n1], _quant(x[b, h, n0:n1], np.float32(s))), (h, blk)
    assert np.array_equal(c.k_codes[:, :, N:], np.zeros_like(c.k_codes[:, :, N:]))


def test_query_blocks_single_block_and_brute_force():
    rng = np.random.default_rng(13)
    q = _fp16(rng, (1, 1, 40, 32))
    cb, sb = oracle.quantize_q(q, 1, oracle.GRAN_BLOCK, None)
    ct, st = oracle.quantize_q(q, 1, oracle.GRAN_TENSOR, None)
    assert np.array_equal(cb, ct) and np.array_equal(sb, st)
    # two heads, 150 positions, per-channel K scales folded in first
    B, Hq, Hkv, L, d = 1, 4, 2, 150, 16
    q = _fp16(rng, (B, Hq, L, d))
    ksc = (rng.random((B, Hkv, d)) + 0.25).astype(np.float32)
    codes, scales = oracle.quantize_q(q, Hkv, oracle.GRAN_BLOCK, ksc)
    G = Hq // Hkv
    for h in range(Hq):
        qq = (q[0, h].astype(np.float32) * ksc[0, h // G][None, :]).astype(np.float32)
        for i0 in range(0, L, 64):
            i1 = min(L, i0 + 64)
            s = np.float32(np.abs(qq[i0:i1]).max()) / np.float32(127.0)
            assert np.all(scales[0, h, i0:i1] == s)
            assert np.array_equal(codes[0, h, i0:i1], _quant(qq[i0:i1], s))


def test_prefill_emulation_single_key_block_equals_tensor():
    rng = np.random.default_rng(14)
    k = _fp16(rng, (1, 1, 60, 64)); v = _fp16(rng, (1, 1, 60, 64)); q = _fp16(rng, (1, 2, 5, 64))
    cb = oracle.kv_quantize(k, v, oracle.GRAN_BLOCK, oracle.GRAN_CHANNEL, capacity=64, v_op_format=oracle.PV_FP8)
    ct = oracle.kv_quantize(k, v, oracle.GRAN_TENSOR, oracle.GRAN_CHANNEL, capacity=64, v_op_format=oracle.PV_FP8)
    rb = oracle.prefill_emulate(q, cb, kv_len=60, q_offset=55, causal=True, want_p=True)
    rt = oracle.prefill_emulate(q, ct, kv_len=60, q_offset=55, causal=True, want_p=True)
    assert np.array_equal(rb.out, rt.out) and np.array_equal(rb.p_codes, rt.p_codes)


def test_prefill_emulation_key_block_constants():
    """The score of key j is fp32(fp32(s_Q * kconst) * s_K[block(j)]) * acc_j: with one key per
    visible position and P codes exported, the ordering of the keys' P codes follows the
    per-block constants; checked against a brute-force recomputation of the scores' maximum."""
    rng = np.random.default_rng(15)
    B, Hq, Hkv, L, N, d = 1, 1, 1, 1, 200, 32
    k = _fp16(rng, (B, Hkv, N, d)); v = _fp16(rng, (B, Hkv, N, d)); q = _fp16(rng, (B, Hq, L, d))
    k[0, 0, 64:128] *= np.float16(8.0)     # blocks of different scale
    c = oracle.kv_quantize(k, v, oracle.GRAN_BLOCK, oracle.GRAN_CHANNEL, capacity=256, v_op_format=oracle.PV_FP8)
    r = oracle.prefill_emulate(q, c, kv_len=N, q_offset=N - 1, causal=True, want_s=True, n_streams=1)
    qc, qs = oracle.quantize_q(q, Hkv, oracle.GRAN_TOKEN, None)
    acc = (qc[0, 0, 0].astype(np.int64)[None, :] * c.k_codes[0, 0, :N].astype(np.int64)).sum(axis=1)
    assert np.array_equal(acc, r.s_i32[0, 0, 0])
    kc = np.float32(np.float64(1.0 / np.sqrt(d)) * 1.4426950408889634074)
    cq = np.float32(qs[0, 0, 0] * kc)
    cj = (cq * c.k_scales[0, 0, np.arange(N) // 64]).astype(np.float32)
    s = (cj * acc.astype(np.float32)).astype(np.float32)
    # the row's log-sum-exp in the units of c * acc: m + log2(l) - log2 448 with m = max s
    m = s.max()
    assert r.lse[0, 0, 0] >= m - 1e-3 and r.lse[0, 0, 0] <= m + np.log2(N) + 1e-3
    # and against the fp64 log-sum-exp of those scores (P quantization moves l by < 2^-4 per term)
    ref = m + np.log2(np.exp2((s - m).astype(np.float64)).sum())
    assert abs(r.lse[0, 0, 0] - ref) < 0.1


def test_decode_emulation_key_blocks_brute_force():
    rng = np.random.default_rng(16)
    B, Hq, Hkv, N, d = 1, 2, 1, 130, 16
    k = _fp16(rng, (B, Hkv, N, d)); v = _fp16(rng, (B, Hkv, N, d)); q = _fp16(rng, (B, Hq, d))
    k[0, 0, :64] *= np.float16(4.0)
    c = oracle.kv_quantize(k, v, oracle.GRAN_BLOCK, oracle.GRAN_CHANNEL, capacity=192)
    out, qk = oracle.decode_emulate(q, c, kv_len=N, want_qk=True)
    kc = np.float32(np.float64(1.0 / np.sqrt(d)) * 1.4426950408889634074)
    for h in range(Hq):
        qq = q[0, h].astype(np.float32)
        sq = np.float32(np.abs(qq).max()) / np.float32(127.0)
        qc = _quant(qq, sq).astype(np.int64)
        acc = (qc[None, :] * c.k_codes[0, 0, :N].astype(np.int64)).sum(axis=1)
        assert np.array_equal(acc, qk[0, h])
        cn = (np.float32(sq * kc) * c.k_scales[0, 0, np.arange(N) // 64]).astype(np.float32)
        s = (cn * acc.astype(np.float32)).astype(np.float32).astype(np.float64)
        p = np.exp2(s - s.max())
        o = (p[:, None] * c.v_codes[0, 0, :N].astype(np.float64)).sum(axis=0) * c.v_scales[0, 0].astype(np.float64) / p.sum()
        assert np.allclose(out[0, h], o, rtol=1e-12, atol=1e-12)

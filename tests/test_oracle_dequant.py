"""Pins of the oracle's fp64 attention over the dequantized int8 cache (the reference of
the 24-bit split precision mode: "Strata" prompt-attention pages, the kernel that keeps K
and V as stored int8 codes and splits the other operand of each product into three exact
8-bit parts)."""
import numpy as np
import pytest

import oracle


def lossless_cache(seed, B=1, H=2, N=96, d=64):
    """K = mu + code * 2^-6 and V = code * 2^-6 with per-channel codes that sum to zero and
    reach +-127: the mean is exactly mu, the scales exactly 2^-6 and every code exact, so
    quantization loses nothing."""
    rng = np.random.default_rng(seed)
    half = rng.integers(-127, 128, size=(B, H, N // 2, d))
    half[:, :, 0, :] = 127
    kc = np.concatenate([half, -half], axis=2)               # sums to zero per channel
    kc = np.take_along_axis(kc, rng.permuted(np.tile(np.arange(N), (B, H, d, 1)), axis=-1).transpose(0, 1, 3, 2), axis=2)
    mu = rng.choice([-0.75, 0.5, 1.0], size=(B, H, 1, d))
    k = (mu + kc * 2.0 ** -6).astype(np.float16)
    vc = rng.integers(-127, 128, size=(B, H, N, d))
    vc[:, :, 3, :] = -127
    v = (vc * 2.0 ** -6).astype(np.float16)
    assert np.array_equal(k.astype(np.float64), mu + kc * 2.0 ** -6)   # exact in fp16
    return k, v, kc, vc


@pytest.mark.parametrize("k_gran", [oracle.GRAN_CHANNEL, oracle.GRAN_TENSOR])
@pytest.mark.parametrize("causal", [False, True])
def test_lossless_cache_gives_exact_attention(k_gran, causal):
    k, v, kc, vc = lossless_cache(31)
    B, H, N, d = k.shape
    L = 40
    q = np.random.default_rng(32).standard_normal((B, 2 * H, L, d)).astype(np.float16)
    cache = oracle.kv_quantize(k, v, k_gran, oracle.GRAN_CHANNEL)
    assert np.array_equal(cache.k_codes[:, :, :N], kc.astype(np.int8))
    assert np.array_equal(cache.v_codes[:, :, :N], vc.astype(np.int8))
    got = oracle.attn_dequant(q, cache, kv_len=N, q_offset=N - L if causal else 0, causal=causal)
    want = oracle.attn_exact(q, k, v, causal=causal, q_offset=N - L if causal else 0)
    assert np.max(np.abs(got - want) / np.abs(want).max(axis=-1, keepdims=True)) < 1e-12


def test_rows_subset_matches_full():
    k, v, _, _ = lossless_cache(33)
    N = k.shape[2]
    q = np.random.default_rng(34).standard_normal((1, 4, 20, 64)).astype(np.float16)
    cache = oracle.kv_quantize(k, v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL)
    full = oracle.attn_dequant(q, cache, kv_len=N)
    rows = np.array([0, 7, 33, 79], np.int64)
    part = oracle.attn_dequant(q, cache, kv_len=N, rows=rows)
    assert np.array_equal(part.reshape(-1, 64)[rows], full.reshape(-1, 64)[rows])

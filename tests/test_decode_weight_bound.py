"""The decode's PV weights are rounded to fp16 after a power-of-two scaling that puts the
largest weight of each 64-key group in [1, 2) (the reading of the decode's fp32-PV step that
the decode kernel takes; the V codes enter as exact fp16 values).  The bound this gives on the
output, checked here on the arithmetic itself (numpy's IEEE binary16 rounding, fp64
elsewhere): per weight, |r(w) - w| <= 2^-11 |w| for normal fp16 results and <= 2^-25 of the
group's largest weight below fp16's normal range; so per output element

    |sum_n r(w_n) v_n - sum_n w_n v_n| / l <= (2^-11 sum_n |w_n v_n| + 2^-25 sum_g w_max,g sum_{n in g} |v_n|) / l

with l the unrounded weight sum (the normalizer the decode keeps in fp32)."""
import numpy as np
import pytest


def _round_weights(w: np.ndarray, group: int = 64) -> np.ndarray:
    """Scale each group's weights by 2^-floor(log2 max) (largest in [1, 2)), round to fp16, unscale."""
    out = np.empty_like(w)
    for g0 in range(0, w.size, group):
        wg = w[g0:g0 + group]
        mx = wg.max()
        e = 0 if mx == 0 else int(np.floor(np.log2(mx)))
        out[g0:g0 + group] = np.ldexp(np.ldexp(wg, -e).astype(np.float16).astype(np.float64), e)
    return out


@pytest.mark.parametrize("seed,spread", [(0, 3.0), (1, 8.0), (2, 20.0)])
def test_fp16_weight_rounding_stays_within_the_derived_bound(seed, spread):
    rng = np.random.default_rng(seed)
    n, d = 4096, 128
    s = rng.standard_normal(n) * spread                       # scores of a row
    w = np.exp2(s - s.max())                                   # softmax weights, largest 1
    v = rng.integers(-127, 128, (n, d)).astype(np.float64)     # int8 V codes (exact in fp16 as 1152 + code)
    l = w.sum()
    exact = w @ v / l
    r = _round_weights(w)
    got = r @ v / l
    wmax_per = np.repeat([w[g:g + 64].max() for g in range(0, n, 64)], 64)[:n]
    bound = (2.0 ** -11 * (np.abs(w)[:, None] * np.abs(v)).sum(0)
             + 2.0 ** -25 * (wmax_per[:, None] * np.abs(v)).sum(0)) / l
    assert np.all(np.abs(got - exact) <= bound)
    # and the bound is well inside the 1e-3 (relative to the row's largest |out|) gate
    assert np.max(np.abs(got - exact)) / np.abs(exact).max() < 1e-3


def test_per_weight_error_of_the_scaled_fp16_rounding():
    rng = np.random.default_rng(9)
    w = np.exp2(-rng.uniform(0, 40, 6400))
    r = _round_weights(w)
    for g0 in range(0, w.size, 64):
        wg, rg = w[g0:g0 + 64], r[g0:g0 + 64]
        mx = wg.max()
        normal = wg / 2.0 ** np.floor(np.log2(mx)) >= 2.0 ** -14
        assert np.all(np.abs(rg - wg)[normal] <= 2.0 ** -11 * wg[normal])
        assert np.all(np.abs(rg - wg)[~normal] <= 2.0 ** -25 * mx)

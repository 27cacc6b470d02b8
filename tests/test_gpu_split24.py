"""GPU parity of the precision mode of attn_q_prefill (pv_mode ATTN_Q_PV_SPLIT24: int8 K and
V codes as stored, q and p split into three exact 8-bit parts, int8 matrix cores for both
products) against the oracle's fp64 attention over the same dequantized int8 cache.

The mode approaches that definition up to its 24-bit operands and fp32 combination; the
bar is a max error of 2e-5 relative to each row's largest |value| (the "Strata" pages
measure a few 1e-6 for their split).  The fp8 mode on the same inputs is ~1e-2 away, so the
bar separates the two by three orders of magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-5


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
    return np.max(np.abs(a - e) / np.maximum(np.abs(e).max(axis=1, keepdims=True), 1e-30), axis=1)


def run(c, k_gran, pv_mode=B.PV_SPLIT24, kv_len=None, out_dtype=B.OUT_F32):
    Bn, Hq, L, D = c.q.shape
    Hkv, N = c.k.shape[1], kv_len or c.k.shape[2]
    cap = (c.k.shape[2] + 63) // 64 * 64
    g = B.alloc_cache(Bn, Hkv, cap, D, k_gran, B.GRAN_CHANNEL, DEV,
                      v_op_format=B.PV_FP8 if pv_mode == B.PV_FP8 else B.PV_INT8)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=c.causal, pv_mode=pv_mode,
                           out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def reference(c, k_gran, rows=None, kv_len=None):
    cap = (c.k.shape[2] + 63) // 64 * 64
    o = oracle.kv_quantize(c.k, c.v, k_gran, oracle.GRAN_CHANNEL, capacity=cap)
    return oracle.attn_dequant(c.q, o, kv_len=kv_len or c.k.shape[2], q_offset=c.q_offset, causal=c.causal,
                               rows=rows)


CASES = [
    ("g4_causal_d128", lambda: inputs.small_case(201, hq=8, hkv=2, q_len=150, kv_len=333, causal=True)),
    ("g1_noncausal_d64", lambda: inputs.small_case(202, hq=3, hkv=3, q_len=77, kv_len=200, d=64)),
    ("g2_b2_ragged", lambda: inputs.small_case(203, batch=2, hq=4, hkv=2, q_len=65, kv_len=129)),
    ("g8_one_tile", lambda: inputs.small_case(204, hq=8, hkv=1, q_len=40, kv_len=64, causal=True)),
    ("one_key", lambda: inputs.small_case(205, hq=2, hkv=1, q_len=1, kv_len=1)),
    ("config1_outliers", lambda: inputs.config1()),
]


@pytest.mark.parametrize("k_gran", [B.GRAN_CHANNEL, B.GRAN_TENSOR], ids=["kchannel", "ktensor"])
@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_split24_matches_fp64_over_the_cache(name, make, k_gran):
    c = make()
    print(f"  split24 {name} k_gran={k_gran} shape={c.q.shape} kv={c.k.shape}", flush=True)
    out = run(c, k_gran)
    ref = reference(c, k_gran)
    err = rel_err(out, ref)
    print(f"  max err {err.max():.3g}, median {np.median(err):.3g}", flush=True)
    assert np.all(np.isfinite(out))
    assert err.max() <= TOL


def test_split24_is_far_closer_than_fp8():
    c = inputs.small_case(206, hq=8, hkv=2, q_len=128, kv_len=1000, causal=True)
    ref = reference(c, B.GRAN_CHANNEL)
    e24 = rel_err(run(c, B.GRAN_CHANNEL), ref).max()
    e8 = rel_err(run(c, B.GRAN_CHANNEL, pv_mode=B.PV_FP8), ref).max()
    print(f"  split24 {e24:.3g} vs fp8 {e8:.3g}", flush=True)
    assert e24 * 100 < e8


def test_split24_full_size_sampled_rows():
    """The LLM prompt-chunk workload at full size (2048 causal queries, 32768 keys, GQA
    16/4), every 97th row of every head against the fp64 reference."""
    c = inputs.config3()
    Bn, Hq, L, D = c.q.shape
    out = run(c, B.GRAN_CHANNEL)
    rows = np.arange(0, Bn * Hq * L, 97, dtype=np.int64)
    ref = reference(c, B.GRAN_CHANNEL, rows=rows)
    err = rel_err(out.reshape(-1, D)[rows], ref.reshape(-1, D)[rows])
    print(f"  config3 sampled: max err {err.max():.3g}, median {np.median(err):.3g}", flush=True)
    assert err.max() <= TOL


def test_split24_fp16_output():
    c = inputs.small_case(207, hq=4, hkv=1, q_len=64, kv_len=300, causal=True)
    o16 = run(c, B.GRAN_CHANNEL, out_dtype=B.OUT_F16)
    assert rel_err(o16, reference(c, B.GRAN_CHANNEL)).max() <= TOL + 2.0 ** -11

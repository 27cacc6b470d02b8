"""GPU parity of attn_q_short_fused (one workgroup per head: the head's quantization and
its attention in one kernel) against the oracle, through the C ABI, on the same seeded
inputs.

The oracle side is the composition the header states: kv_quantize with K and V per
channel (K mean subtracted), then the prefill emulation with per-row Q and one key block
spanning the head (block_c >= N, one stream).  Bars: int32 QK^T bit-exact (debug export);
output (fp32 mode) within 1e-3 of the emulation, relative to each row's largest value;
fp16 output adds its storage rounding; cosine against fp64 attention >= 0.999.
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


def cosine(a, e):
    a = np.asarray(a, np.float64).ravel()
    e = np.asarray(e, np.float64).ravel()
    return float(a @ e / np.sqrt((a @ a) * (e @ e)))


def reference(c, want_s=False):
    N = c.q.shape[2]
    oc = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL)
    return oracle.prefill_emulate(c.q, oc, kv_len=N, q_offset=0, causal=False, q_gran=oracle.GRAN_TOKEN,
                                  block_c=256, n_streams=1, want_s=want_s)


def run(c, out_dtype=B.OUT_F32, debug=False):
    Bn, H, N, D = c.q.shape
    ds = torch.zeros((Bn, H, N, N), dtype=torch.int32, device=DEV) if debug else None
    out = B.attn_q_short_fused(dev(c.q), dev(c.k), dev(c.v), out_dtype=out_dtype, debug_s=ds)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (ds.cpu().numpy() if debug else None)


CASES = [(name, 1) for name in inputs.QFLASH_WORKLOADS] + [("A2", 8), ("A7", 8)]


@pytest.mark.parametrize("name,batch", CASES, ids=[f"{n}x{b}" for n, b in CASES])
def test_qflash_workloads_match_emulation(name, batch):
    c = inputs.vision(name, batch)
    print(f"  short {name} batch={batch} shape={c.q.shape}", flush=True)
    out, s = run(c, debug=True)
    ref = reference(c, want_s=True)
    assert np.array_equal(s, ref.s_i32)
    err = rel_err(out, ref.out)
    cos = cosine(out, oracle.attn_exact(c.q, c.k, c.v))
    print(f"  err vs emulation {err:.3g}, cosine vs fp64 {cos:.6f}", flush=True)
    assert err <= TOL
    assert cos >= 0.999


RAGGED = [(n, d) for d in (32, 64) for n in (1, 2, 31, 63, 64, 65, 128, 129, 200, 256)]


@pytest.mark.parametrize("n,d", RAGGED, ids=[f"n{n}_d{d}" for n, d in RAGGED])
def test_ragged_lengths_llm_like(n, d):
    """Every key-tile count and ragged tail, on K with offset outlier channels (the case the
    mean subtraction is for) and queries whose scores spread over several decades."""
    c = inputs.small_case(900 + n + d, batch=2, hq=3, hkv=3, q_len=n, kv_len=n, d=d)
    print(f"  short ragged n={n} d={d}", flush=True)
    out, s = run(c, debug=True)
    ref = reference(c, want_s=True)
    assert np.array_equal(s, ref.s_i32)
    assert rel_err(out, ref.out) <= TOL


def test_k_offsets_are_removed():
    """Large per-channel K offsets: the in-kernel mean makes the codes those of the centred
    keys, and the output stays within the bar of fp64 attention."""
    c = inputs.vision("A3", 2, k_offset=8.0)
    out, s = run(c, debug=True)
    ref = reference(c, want_s=True)
    assert np.array_equal(s, ref.s_i32)
    assert rel_err(out, ref.out) <= TOL
    assert cosine(out, oracle.attn_exact(c.q, c.k, c.v)) >= 0.999


def test_vit_base_batch64_full():
    """ViT-B self-attention at batch 64 (12 heads, 197 tokens, d = 64), every output."""
    c = inputs.config2()
    out, _ = run(c)
    ref = reference(c)
    err = rel_err(out, ref.out)
    print(f"  vit-b x64: err vs emulation {err:.3g}", flush=True)
    assert err <= TOL
    assert cosine(out, oracle.attn_exact(c.q, c.k, c.v)) >= 0.999


def test_fp16_output_and_determinism():
    c = inputs.vision("A4", 2)
    o32, _ = run(c)
    o16, _ = run(c, out_dtype=B.OUT_F16)
    assert rel_err(o16, reference(c).out) <= TOL + 2.0 ** -11
    assert np.array_equal(o16, o32.astype(np.float16).astype(np.float32)) or rel_err(o16, o32) <= 2.0 ** -11
    o32b, _ = run(c)
    assert np.array_equal(o32.view(np.uint32), o32b.view(np.uint32))

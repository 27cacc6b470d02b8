"""GPU parity on the degenerate inputs of the method, through the C ABI, against the
oracle and against what the method fixes for them.

* Identical keys: K minus its channel mean is exactly zero, so the K scales are zero, every
  K code is 0 ([QFlash] eq. (2) with a zero absmax), every score is 0 and the softmax is
  uniform: all query rows of a head get the same output.
* Q = 0: zero query scale, zero codes, zero scores: uniform weights again.
* V = 0: zero V scales and codes: the output is exactly zero.
* One dominant key (its logit far above the rest): the output is that key's value row
  within the P and V rounding of the scheme.

The cache (codes, scales, mean) must stay bit-exact with the oracle, and the outputs
within 1e-3 of the oracle's emulation, relative to each row's largest value (rows that
are exactly zero must be exactly zero).
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


def identical_keys(c):
    return dataclasses.replace(c, k=np.ascontiguousarray(np.broadcast_to(c.k[:, :, :1], c.k.shape)))


def zero_q(c):
    return dataclasses.replace(c, q=np.zeros_like(c.q))


def zero_v(c):
    return dataclasses.replace(c, v=np.zeros_like(c.v))


def dominant_key(c, j=37, gain=60.0):
    # key j of every kv head points along the first query of its first head, scaled so its
    # logit stands far above the others
    k = c.k.astype(np.float64).copy()
    G = c.q.shape[1] // c.k.shape[1]
    for g in range(c.k.shape[1]):
        qd = c.q[:, g * G, 0].astype(np.float64)
        k[:, g, j] = gain * qd / np.linalg.norm(qd, axis=-1, keepdims=True)
    return dataclasses.replace(c, k=k.astype(np.float16))


MODS = [("identical_keys", identical_keys), ("zero_q", zero_q), ("zero_v", zero_v),
        ("dominant_key", dominant_key)]


def base(seed=81, **kw):
    args = dict(batch=1, hq=4, hkv=2, q_len=70, kv_len=200)
    args.update(kw)
    return inputs.small_case(seed, **args)


def check_cache(g, o, N):
    assert np.array_equal(g.k_codes.cpu().numpy()[:, :, :N], o.k_codes[:, :, :N])
    assert np.array_equal(g.v_codes.cpu().numpy()[:, :, :N], o.v_codes[:, :, :N])
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), o.k_mean.view(np.uint32))


@pytest.mark.parametrize("gran", [oracle.GRAN_CHANNEL, oracle.GRAN_TOKEN], ids=["channel", "token"])
@pytest.mark.parametrize("name,mod", MODS, ids=[m[0] for m in MODS])
def test_kv_quantize_degenerate_bit_exact(name, mod, gran):
    c = mod(base())
    N = c.k.shape[2]
    cap = (N + 63) // 64 * 64
    print(f"  kv_quantize {name} gran={gran}", flush=True)
    g = B.alloc_cache(1, 2, cap, 128, gran, gran, DEV, v_op_format=B.PV_FP8 if gran == oracle.GRAN_CHANNEL else None)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    torch.cuda.synchronize()
    o = oracle.kv_quantize(c.k, c.v, gran, gran, capacity=cap,
                           v_op_format=oracle.PV_FP8 if gran == oracle.GRAN_CHANNEL else None)
    check_cache(g, o, N)
    if name == "identical_keys":
        assert not np.any(g.k_codes.cpu().numpy()[:, :, :N])
    if name == "zero_v":
        assert not np.any(g.v_codes.cpu().numpy()[:, :, :N])


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("name,mod", MODS, ids=[m[0] for m in MODS])
def test_prefill_degenerate(name, mod, causal):
    c = mod(base(causal=causal))
    Bn, Hq, L, D = c.q.shape
    N = c.k.shape[2]
    print(f"  prefill {name} causal={causal}", flush=True)
    g = B.alloc_cache(Bn, c.k.shape[1], (N + 63) // 64 * 64, D, c.k_gran, c.v_gran, DEV, v_op_format=B.PV_FP8)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    out = B.attn_q_prefill(dev(c.q), g, kv_len=N, q_offset=c.q_offset, causal=causal, out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    o = oracle.kv_quantize(c.k, c.v, c.k_gran, c.v_gran, capacity=(N + 63) // 64 * 64)
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=causal).out
    assert np.all(np.isfinite(out))
    if name == "zero_v":
        assert not np.any(out)
        return
    assert rel_err(out, ref) <= TOL
    if name in ("identical_keys", "zero_q") and not causal:
        # uniform weights over the same keys: every row of a head has the same output
        assert np.max(np.abs(out - out[:, :, :1])) <= 1e-6 * np.abs(out).max()
    if name == "dominant_key":
        # the rows of the head the key was aimed at are that key's dequantized value row
        vrow = (o.v_codes[0, 0, 37].astype(np.float64) * np.asarray(o.v_scales, np.float64)[0, 0])
        assert rel_err(out[0, 0, :1], vrow[None]) <= 0.07   # e4m3 rounding of V codes above 16


@pytest.mark.parametrize("name,mod", MODS, ids=[m[0] for m in MODS])
def test_decode_degenerate(name, mod):
    c = mod(inputs.config4(kv_len=1500)[0])
    N = c.k.shape[2]
    print(f"  decode {name}", flush=True)
    cap = (N + 63) // 64 * 64   # (capacities are whole 64-key tiles)
    g = B.alloc_cache(1, 4, cap, 128, B.GRAN_TOKEN, B.GRAN_TOKEN, DEV, v_op_format=None)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    out = B.attn_q_decode(dev(c.q[:, :, 0]), g, kv_len=N, out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    o = oracle.kv_quantize(c.k, c.v, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, capacity=cap)
    ref, _ = oracle.decode_emulate(np.ascontiguousarray(c.q[:, :, 0]), o, kv_len=N)
    assert np.all(np.isfinite(out))
    if name == "zero_v":
        assert not np.any(out)
        return
    assert rel_err(out, ref) <= TOL
    if name in ("identical_keys", "zero_q"):
        # uniform weights: every head of a kv head gets the mean of its dequantized V rows
        G = 4
        vdq = o.v_codes[0, :, :N].astype(np.float64) * o.v_scales[0, :, :N].astype(np.float64)[..., None]
        mean = vdq.mean(axis=1)
        exp = np.repeat(mean, G, axis=0)[None]
        assert rel_err(out, exp) <= TOL


@pytest.mark.parametrize("name,mod", MODS, ids=[m[0] for m in MODS])
def test_short_degenerate(name, mod):
    c = inputs.vision("A7", 2)
    if name == "dominant_key":
        c = dataclasses.replace(c, k=c.k.copy())
        qd = c.q[:, :, 0].astype(np.float64)
        c.k[:, :, 5] = (60.0 * qd / np.linalg.norm(qd, axis=-1, keepdims=True)).astype(np.float16)
    else:
        c = mod(c)
    Bn, H, N, D = c.q.shape
    print(f"  short {name}", flush=True)
    out = B.attn_q_short_fused(dev(c.q), dev(c.k), dev(c.v), out_dtype=B.OUT_F32)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    o = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL)
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=0, causal=False, q_gran=oracle.GRAN_TOKEN,
                                 block_c=256, n_streams=1).out
    assert np.all(np.isfinite(out))
    if name == "zero_v":
        assert not np.any(out)
        return
    assert rel_err(out, ref) <= TOL

"""attn_q_decode_noalloc: the decode for callers that cannot allocate (graph capture, serving
loops), with its split partials in the library's static per-GPU scratch instead of a
workspace.  Checked through the C ABI against attn_q_decode on the same inputs -- the same
kernels, so the same bits -- and against the oracle's decode emulation, on two calls in a
row, the second with a smaller input (fewer keys, another batch, head grouping and scale
granularity), so the second call runs over what the first left in the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _rel_err(a, e):
    a = np.asarray(a, np.float64).reshape(-1, a.shape[-1])
    e = np.asarray(e, np.float64).reshape(-1, e.shape[-1])
    return float(np.max(np.abs(a - e) / np.abs(e).max(axis=1, keepdims=True)))


CASES = [
    # (name, inputs, kv_len, k_gran, v_gran): the decode workload, then a smaller call
    ("config4_32768", lambda: inputs.config4()[0], 32768, B.GRAN_TOKEN, B.GRAN_TOKEN),
    ("b2_g2_channel_3001", lambda: inputs.small_case(95, batch=2, hq=4, hkv=2, q_len=1, kv_len=3001),
     3001, B.GRAN_CHANNEL, B.GRAN_CHANNEL),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def test_noalloc_decode_equals_decode_on_two_calls():
    for name, make, kv_len, kg, vg in CASES:
        print(f"  noalloc decode {name} kv_len={kv_len}", flush=True)
        c = make()
        Bn, H, N, D = c.k.shape
        cap = (N + 63) // 64 * 64
        g = B.alloc_cache(Bn, H, cap, D, kg, vg, DEV, v_op_format=None)
        B.kv_quantize_i8(_dev(c.k), _dev(c.v), g)
        q = _dev(c.q[:, :, 0])
        ref = B.attn_q_decode(q, g, kv_len=kv_len, out_dtype=B.OUT_F32)
        out = torch.full_like(ref, float("nan"))
        B.attn_q_decode_noalloc(q, g, kv_len=kv_len, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), name
        o = oracle.kv_quantize(c.k, c.v, kg, vg, capacity=cap)
        emu, _ = oracle.decode_emulate(np.ascontiguousarray(c.q[:, :, 0]), o, kv_len=kv_len)
        err = _rel_err(out.cpu().numpy(), emu)
        print(f"    bit-identical to attn_q_decode; max rel err vs emulation {err:.2e}", flush=True)
        assert err <= 1e-3


def test_noalloc_rejects_calls_beyond_the_scratch():
    """A call whose partials exceed the static scratch returns ATTN_Q_E_SCRATCH before any
    launch, and leaves the output untouched."""
    c = inputs.small_case(96, hq=16, hkv=4, q_len=1, kv_len=64)
    g = B.alloc_cache(1, 4, 1 << 20, 128, B.GRAN_TOKEN, B.GRAN_TOKEN, DEV, v_op_format=None)
    out = torch.full((1, 16, 128), 7.0, device=DEV)
    with pytest.raises(B.AttnQError) as e:
        B.attn_q_decode_noalloc(_dev(c.q[:, :, 0]), g, kv_len=1 << 20, out=out)
    assert e.value.status == B.E_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)

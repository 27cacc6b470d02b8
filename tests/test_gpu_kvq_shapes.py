"""GPU parity of kv_quantize_i8 at larger shapes, bit-exact against the oracle: the full
prompt-chunk cache, heads of many statistics / codes workgroups with a ragged last tile,
capacities past the keys (PV-operand tiles beyond the keys zeroed), both head dims and every
K / V granularity, each call made twice on one workspace (which every call leaves zeroed)."""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _check(k, v, kg, vg, cap, vfmt, sub=True, header=False, v_codes=True):
    Bn, H, N, D = k.shape
    print(f"  kvq B={Bn} H={H} N={N} d={D} cap={cap} k_gran={kg} v_gran={vg} v_op={vfmt} "
          f"sub={sub} header={header}", flush=True)
    g = B.alloc_cache(Bn, H, cap, D, kg, vg, DEV, v_op_format=vfmt, header=header)
    if not v_codes:
        g.v_codes = None
    kt, vt = _dev(k), _dev(v)
    # twice in a row: the second call finds the workspace as the first one left it
    for _ in range(2):
        B.kv_quantize_i8(kt, vt, g, subtract_k_mean=sub)
    torch.cuda.synchronize()
    S = np.zeros((Bn, H, D), np.int64) if header else None
    o = oracle.kv_quantize(k, v, kg, vg, subtract_mean=sub, capacity=cap,
                           v_op_format=vfmt, k_sum=S)
    assert np.array_equal(g.k_codes.cpu().numpy()[:, :, :N], o.k_codes[:, :, :N])
    if v_codes:
        assert np.array_equal(g.v_codes.cpu().numpy()[:, :, :N], o.v_codes[:, :, :N])
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), o.k_mean.view(np.uint32))
    gk, ok = g.k_scales.cpu().numpy(), o.k_scales
    if kg == oracle.GRAN_TENSOR:
        gk, ok = gk.ravel()[:1], np.asarray(ok).ravel()[:1]
    elif kg == oracle.GRAN_TOKEN:
        gk, ok = gk[:, :, :N], ok[:, :, :N]
    elif kg == oracle.GRAN_BLOCK:
        nb = (N + 63) // 64
        gk, ok = gk[:, :, :nb], ok[:, :, :nb]
    assert np.array_equal(np.ascontiguousarray(gk).view(np.uint8), np.ascontiguousarray(ok).view(np.uint8))
    gv, ov = g.v_scales.cpu().numpy(), o.v_scales
    if vg == oracle.GRAN_TOKEN:
        gv, ov = gv[:, :, :N], ov[:, :, :N]
    assert np.array_equal(np.ascontiguousarray(gv).view(np.uint8), np.ascontiguousarray(ov).view(np.uint8))
    if vfmt is not None:
        assert np.array_equal(g.v_op.cpu().numpy(), o.v_op)
    if header:
        assert np.array_equal(g.k_sum.cpu().numpy(), S)


def test_prompt_chunk_cache():
    """The prompt-chunk cache (4 kv heads x 32768 keys, d = 128) in the configuration the
    benchmark times (with and without the int8 V codes), and one 512 keys longer."""
    k, v, _ = inputs.llm_kv(np.random.default_rng(71), 4, 32768 + 512, 128)
    k32, v32 = np.ascontiguousarray(k[:, :, :32768]), np.ascontiguousarray(v[:, :, :32768])
    _check(k32, v32, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, 32768, B.PV_FP8, header=True)
    _check(k32, v32, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, 32768, B.PV_FP8, v_codes=False)
    _check(k, v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, 32768 + 512, B.PV_FP8)


CASES = [
    # (batch, heads, N, d, k_gran, v_gran, capacity, v_op, subtract, header)
    (2, 3, 1500, 128, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, 2048, B.PV_FP8, True, False),
    (1, 2, 1100, 128, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, 2048, B.PV_INT8, False, True),
    (2, 2, 1537, 128, oracle.GRAN_BLOCK, oracle.GRAN_CHANNEL, 1600, B.PV_FP8, True, False),
    (1, 3, 1025, 128, oracle.GRAN_TOKEN, oracle.GRAN_TOKEN, 1088, B.PV_FP8, True, True),
    (1, 2, 2500, 64, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL, 3072, B.PV_FP8, True, False),
    (2, 1, 2049, 64, oracle.GRAN_BLOCK, oracle.GRAN_TOKEN, 2112, None, True, False),
    (1, 1, 511, 128, oracle.GRAN_TOKEN, oracle.GRAN_CHANNEL, 512, B.PV_FP8, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}_d{c[3]}_k{c[4]}_v{c[5]}" for c in CASES])
def test_multi_workgroup_heads(case):
    """Heads of several workgroups (ragged last tile), capacities past the keys (operand tiles
    beyond the keys zeroed), every K / V granularity but per-tensor K."""
    Bn, H, N, D, kg, vg, cap, vfmt, sub, header = case
    k, v, _ = inputs.llm_kv(np.random.default_rng(N + 7 * H + D), H, N, D, batch=Bn)
    _check(k, v, kg, vg, cap, vfmt, sub=sub, header=header)


def test_per_tensor_k():
    k, v, _ = inputs.llm_kv(np.random.default_rng(5), 2, 700, 128)
    _check(k, v, oracle.GRAN_TENSOR, oracle.GRAN_CHANNEL, 768, B.PV_FP8)

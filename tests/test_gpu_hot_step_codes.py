"""The hand-scheduled prefill step (d = 128, e4m3 PV) against the oracle's emulation through its
own debug exports: the int32 scores bit-exact and the P codes of every visible pair, for
per-channel, per-token and per-block K on a causal, ragged, many-tile case (and per-token K
through the compiler-scheduled step: d = 64, int8 PV).  The step's kernels
with and without the exports are separate instantiations of one source; their outputs must be
bit-identical, so the exported codes are those the production kernel computes.  P codes may
differ only where the hardware exp2 (not correctly rounded) lands on the other side of an e4m3
rounding boundary (int8 PV: a rint boundary): at most one in 10^4, each one code step apart."""
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


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


# (name, k_gran, q_gran, seed, d, pv_mode): 8 query heads over 2 kv heads, 150 queries at the end
# of 1000 keys (15 full tiles and a 40-key tail).  With d = 128 and e4m3 PV the unmasked tiles take
# the hand-scheduled step; the d = 64 and int8-PV cases check the compiler-scheduled step's
# per-token K path (the scales read from the same LDS slot).
CASES = [
    ("kchan", B.GRAN_CHANNEL, B.GRAN_TOKEN, 301, 128, B.PV_FP8),
    ("ktok", B.GRAN_TOKEN, B.GRAN_TOKEN, 302, 128, B.PV_FP8),
    ("kblk_qblk", B.GRAN_BLOCK, B.GRAN_BLOCK, 303, 128, B.PV_FP8),
    ("ktok_d64", B.GRAN_TOKEN, B.GRAN_TOKEN, 304, 64, B.PV_FP8),
    ("ktok_int8pv", B.GRAN_TOKEN, B.GRAN_TOKEN, 305, 128, B.PV_INT8),
]


@pytest.mark.parametrize("name,kg,qg,seed,d,pv", CASES, ids=[c[0] for c in CASES])
def test_hot_step_scores_and_p_codes(name, kg, qg, seed, d, pv):
    c = inputs.small_case(seed, hq=8, hkv=2, q_len=150, kv_len=1000, d=d, causal=True)
    Bn, Hq, L, D = c.q.shape
    N = c.k.shape[2]
    cap = (N + 63) // 64 * 64
    print(f"  hot step {name}: shape={c.shape}", flush=True)
    g = B.alloc_cache(Bn, 2, cap, D, kg, B.GRAN_CHANNEL, DEV, v_op_format=pv)
    B.kv_quantize_i8(dev(c.k), dev(c.v), g)
    opv = oracle.PV_FP8 if pv == B.PV_FP8 else oracle.PV_INT8
    o = oracle.kv_quantize(c.k, c.v, kg, oracle.GRAN_CHANNEL, capacity=cap, v_op_format=opv)
    ds = torch.full((Bn, Hq, L, N), -(2 ** 31), dtype=torch.int32, device=DEV)
    dp = torch.full((Bn, Hq, L, N), 0xFF, dtype=torch.uint8, device=DEV)
    kw = dict(kv_len=N, q_offset=c.q_offset, causal=True, q_gran=qg, out_dtype=B.OUT_F32, pv_mode=pv)
    out_dbg = B.attn_q_prefill(dev(c.q), g, debug_s=ds, debug_p=dp, **kw).clone()
    out = B.attn_q_prefill(dev(c.q), g, **kw)
    torch.cuda.synchronize()
    ref = oracle.prefill_emulate(c.q, o, kv_len=N, q_offset=c.q_offset, causal=True, q_gran=qg,
                                 pv_mode=opv, want_s=True, want_p=True)
    vis = np.arange(N)[None, :] <= (c.q_offset + np.arange(L))[:, None]
    vis = np.broadcast_to(vis, ds.shape)
    assert np.array_equal(ds.cpu().numpy()[vis], ref.s_i32[vis])
    got = dp.cpu().numpy()
    diff = (got != ref.p_codes) & vis
    n = int(diff.sum())
    print(f"    P-code mismatches {n} of {int(vis.sum())}", flush=True)
    assert n <= int(vis.sum()) // 10000
    if n:
        assert np.all(np.abs(got[diff].astype(np.int64) - ref.p_codes[diff].astype(np.int64)) == 1)
    # the production instantiation computes the same values as the exporting one
    assert torch.equal(out, out_dbg)

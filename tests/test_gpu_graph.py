"""The three calls captured in one HIP graph: every replay must reproduce the eager
results bit for bit (same kernels on the same inputs), with eager work and
synchronisation between the replays and the outputs overwritten before each one.
The workspaces are created by an eager warm-up, so nothing allocates under capture,
and no call records a memset (the quantizer's accumulators are left zero by every
call instead)."""
import numpy as np
import pytest
import torch

from quantized_attention_attn_amd import binding as B
from quantized_attention_attn_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _fields(c):
    return [getattr(c, f) for f in ("k_codes", "v_codes", "k_scales", "v_scales", "k_mean", "v_op")]


def test_graph_replays_match_eager():
    c = inputs.small_case(81, hq=8, hkv=2, q_len=150, kv_len=700, causal=True)
    k, v, q = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (c.k, c.v, c.q))
    qd = torch.from_numpy(np.ascontiguousarray(c.q[:, :, -1])).to(DEV)
    Bn, Hkv, N, D = c.k.shape
    Hq = c.q.shape[1]
    cap = (N + 63) // 64 * 64

    def make():
        cache = B.alloc_cache(Bn, Hkv, cap, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, DEV, v_op_format=B.PV_FP8)
        out = torch.empty((Bn, Hq, c.q.shape[2], D), dtype=torch.float32, device=DEV)
        dout = torch.empty((Bn, Hq, D), dtype=torch.float32, device=DEV)
        return cache, out, dout

    def run(cache, out, dout):
        B.kv_quantize_i8(k, v, cache)
        B.attn_q_prefill(q, cache, kv_len=N, q_offset=c.q_offset, causal=True, out=out)
        B.attn_q_decode(qd, cache, kv_len=N, out=dout)

    # eager reference (also creates every workspace)
    ref = make()
    run(*ref)
    torch.cuda.synchronize()

    cap_bufs = make()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*cap_bufs)          # warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run(*cap_bufs)
    torch.cuda.synchronize()

    scratch = make()
    for rep in range(3):
        print(f"  graph replay {rep}", flush=True)
        cache_g, out_g, dout_g = cap_bufs
        for t in _fields(cache_g) + [out_g, dout_g]:
            if t is not None:
                t.fill_(0x7F if t.dtype in (torch.int8, torch.uint8) else float("nan"))
        run(*scratch)           # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("k_codes", "v_codes", "k_scales", "v_scales", "k_mean", "v_op"),
                              _fields(cache_g), _fields(ref[0])):
            if a is None:
                continue
            if name in ("k_codes", "v_codes"):    # (rows from N to the capacity are not written)
                a, b = a[:, :, :N], b[:, :, :N]
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        assert torch.equal(out_g, ref[1]), f"replay {rep}: prefill output differs"
        assert torch.equal(dout_g, ref[2]), f"replay {rep}: decode output differs"


def test_graph_replays_match_eager_append_short_split24():
    """The later calls in one graph: a prompt quantized with its K-sum header, a one-token
    and a 70-token append (one and three launches), decode over the grown cache, the
    short-sequence kernel and the precision-mode prefill.  Re-quantizing the prompt at the
    start of each replay resets the header, so every replay must reproduce the eager bytes."""
    c = inputs.config4(kv_len=640)[0]
    P, N = 569, 640
    k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (c.k, c.v))
    q1 = torch.from_numpy(np.ascontiguousarray(c.q[:, :, 0])).to(DEV)
    sv = inputs.vision("A2", 2)
    qs, ks, vs = (torch.from_numpy(x).to(DEV) for x in (sv.q, sv.k, sv.v))
    p3 = inputs.small_case(82, hq=8, hkv=2, q_len=96, kv_len=300, causal=True)
    k3, v3, q3 = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (p3.k, p3.v, p3.q))
    Bn, Hkv, _, D = c.k.shape

    def make():
        cache = B.alloc_cache(Bn, Hkv, N, D, B.GRAN_TOKEN, B.GRAN_TOKEN, DEV, v_op_format=None, header=True)
        c3 = B.alloc_cache(1, 2, 320, 128, B.GRAN_CHANNEL, B.GRAN_CHANNEL, DEV, v_op_format=B.PV_INT8)
        outs = (torch.empty((Bn, c.q.shape[1], D), dtype=torch.float32, device=DEV),
                torch.empty(sv.q.shape, dtype=torch.float16, device=DEV),
                torch.empty(p3.q.shape, dtype=torch.float32, device=DEV))
        return cache, c3, outs

    # (slices of k and v are views; the calls need contiguous tensors)
    k, v = k.contiguous(), v.contiguous()
    kp, vp = k[:, :, :P].contiguous(), v[:, :, :P].contiguous()
    k1, v1 = k[:, :, P:P + 1].contiguous(), v[:, :, P:P + 1].contiguous()
    kr, vr = k[:, :, P + 1:].contiguous(), v[:, :, P + 1:].contiguous()

    def run_c(cache, c3, outs):
        B.kv_quantize_i8(kp, vp, cache)
        B.attn_q_kv_append_i8(k1, v1, cache)
        B.attn_q_kv_append_i8(kr, vr, cache)
        B.attn_q_decode(q1, cache, kv_len=N, out=outs[0])
        B.attn_q_short_fused(qs, ks, vs, out=outs[1])
        B.kv_quantize_i8(k3, v3, c3)
        B.attn_q_prefill(q3, c3, kv_len=300, q_offset=p3.q_offset, causal=True, out=outs[2],
                         pv_mode=B.PV_SPLIT24)

    ref = make()
    run_c(*ref)
    torch.cuda.synchronize()
    cap = make()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_c(*cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run_c(*cap)
    torch.cuda.synchronize()
    scratch = make()
    for rep in range(3):
        print(f"  graph replay {rep}", flush=True)
        cache_g, c3_g, outs_g = cap
        for t in (cache_g.k_codes, cache_g.v_codes, cache_g.k_sum, c3_g.k_codes) + outs_g:
            t.fill_(0x7F if t.dtype in (torch.int8, torch.uint8) else 0)
        run_c(*scratch)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache_g.k_codes[:, :, :N], ref[0].k_codes[:, :, :N])
        assert torch.equal(cache_g.v_codes[:, :, :N], ref[0].v_codes[:, :, :N])
        assert torch.equal(cache_g.k_sum, ref[0].k_sum)
        for a, b in zip(outs_g, ref[2]):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                               b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def test_graph_replay_mx_path_matches_eager():
    """kv_quantize_i8, attn_q_k_quantize_mx and attn_q_prefill_mx (fp4 K, fp6 Q) captured in one
    HIP graph: every replay, with eager work between, gives the eager bytes."""
    c = inputs.small_case(41, hq=8, hkv=2, q_len=100, kv_len=700, causal=True)
    Bn, Hq, L, D = c.q.shape
    H, N = c.k.shape[1], c.k.shape[2]
    k, v, q = (torch.from_numpy(x).to(DEV) for x in (c.k, c.v, c.q))

    def make():
        cache = B.alloc_cache(Bn, H, 704, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, DEV, v_op_format=B.PV_FP8)
        keys = B.alloc_mx_keys(Bn, H, 704, D, B.MX_FP4, DEV)
        return cache, keys, torch.empty((Bn, Hq, L, D), dtype=torch.float32, device=DEV)

    def run(cache, keys, out):
        B.kv_quantize_i8(k, v, cache)
        B.attn_q_k_quantize_mx(k, cache.k_mean, keys)
        B.attn_q_prefill_mx(q, keys, cache, kv_len=N, q_fmt=B.MX_FP6, q_offset=c.q_offset, causal=True, out=out)

    ref = make()
    run(*ref)
    torch.cuda.synchronize()
    cap = make()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run(*cap)
    torch.cuda.synchronize()
    scratch = make()
    for rep in range(3):
        print(f"  MX graph replay {rep}", flush=True)
        cap[1].codes.fill_(0x5A)
        cap[1].scales.fill_(0)
        cap[2].fill_(float("nan"))
        run(*scratch)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # (rows past the N keys are documented as untouched)
        assert torch.equal(cap[1].codes[:, :, :N], ref[1].codes[:, :, :N])
        assert torch.equal(cap[1].scales[:, :, :N], ref[1].scales[:, :, :N])
        assert torch.equal(cap[2], ref[2])

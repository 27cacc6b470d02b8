"""Benchmark of the quantized-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. kv_quantize_i8 : 32768-key fp16 K/V cache of the LLM prompt-chunk workload
                      (GQA 16 q / 4 kv heads, d=128) -> int8 cache with per-channel
                      scales, K-mean subtracted, e4m3 PV operand;
  2. attn_q_prefill : the 2048-query chunk at the end of that context, causal within
                      the chunk, int8 QK^T / fp32 online softmax / e4m3-P fp8 PV;
  3. attn_q_decode  : the next token's 16 query heads against the same int8 cache.
``value`` = algorithmic tera-ops of a step / step wall time (inputs resident in HBM); the
step's launches are replayed as one captured HIP graph (``--no-graphs``: eager launches).
The ``roofline`` object reports the dominant kernel (attn_q_prefill) against the
dense int8/fp8 matrix-core peak; ``decode`` reports the int8-KV decode kernel on the
32768-token per-token-scale cache, rotated over 32 distinct copies so it is not
served from the 256 MB on-die cache, against HBM peak.  ``kv_append`` reports the
decode-time cache update (attn_q_kv_append_i8: the new token appended with the running
K mean of the cache header), alone and followed by the decode, and a 1024-token chunk.
``prefill_split24`` times the precision mode (24-bit operand split) on the same prompt chunk.
``prefill_mx`` times it with Q and K as MX fp4 / fp6 operands (attn_q_prefill_mx), and the
accuracy report carries those variants at 256 and 32768 keys.
``short_fused`` reports the one-pass short-sequence kernel at the vision shapes against
HBM peak (and, at ViT-B, the two-kernel quantize + prefill path on the same tensors).
``prefill_long_context`` times all 16 causal chunks of the 131072-key prompt (GQA 32/8,
cache quantized once).  ``accuracy`` reports fp8-PV and int8-PV outputs against fp64 at
256, 32768 and 131072 keys, with the softmax mass whose P code is zero.
``cpu_baseline`` times the oracle on the host cores (emulation and fp64 exact path; one
thread on the 256-key outlier case).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--warmup-ms 250]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attention TOPS (% int8/fp8 MFMA peak); int8-KV decode GB/s (% HBM)"
PEAK_TOPS = 5000.0      # MI355X dense int8 = dense fp8 = 5.0 POP/s
PEAK_GBS = 8000.0       # MI355X HBM3E 8 TB/s
D = 128


def measured_traffic(kernel: str, sources):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None when the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec:
        return None
    m = hashlib.sha256()
    for f in sources:
        m.update(open(os.path.join(ROOT, f), "rb").read())
    return rec["hbm_bytes_per_launch"] if m.hexdigest() == rec["source_sha256"] else None


def visible_pairs(q_len, kv_len, q_offset, heads, causal=True):
    i = np.arange(q_len, dtype=np.int64)
    vis = np.minimum(kv_len, q_offset + i + 1) if causal else np.full(q_len, kv_len)
    return int(vis.sum()) * heads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warmup-ms", type=float, default=250.0,
                    help="after the warmup steps, keep running untimed steps for this much wall "
                         "time: the GPU raises its clock over the first ~30 ms of work")
    ap.add_argument("--decode-caches", type=int, default=32)
    ap.add_argument("--decode-reps", type=int, default=10,
                    help="graph replays of the rotated-cache decode timing (0: skip it)")
    ap.add_argument("--append-reps", type=int, default=10,
                    help="graph replays of the KV-append timings (0: skip them)")
    ap.add_argument("--split-reps", type=int, default=5,
                    help="launches of the precision-mode prefill timing (0: skip it)")
    ap.add_argument("--mx-reps", type=int, default=5,
                    help="launches timed for the MX (fp6 / fp4 Q and K) prefill on the prompt chunk (0 = skip)")
    ap.add_argument("--short-reps", type=int, default=10,
                    help="replays of the short-sequence (vision) timings (0: skip them)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="time the step, append and short-sequence sections with eager launches (for counter runs)")
    ap.add_argument("--c5-reps", type=int, default=3,
                    help="timed passes over the 16 chunks of the long-context prefill (0: skip it)")
    ap.add_argument("--no-accuracy", action="store_true",
                    help="skip the accuracy report (fp8-PV and int8-PV against fp64)")
    ap.add_argument("--cpu-rows-step", type=int, default=1,
                    help="oracle CPU baseline: every n-th query row of every head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(the sharding plan is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_attention_attn_amd import binding as B
    from quantized_attention_attn_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    B.lib()
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------ inputs
    t0 = time.time()
    c = inputs.config3()
    Hq, L, KV, q_off = 16, 2048, 32768, 32768 - 2048
    k16 = torch.from_numpy(c.k).to(dev)
    v16 = torch.from_numpy(c.v).to(dev)
    q16 = torch.from_numpy(c.q).to(dev)
    qdec = torch.from_numpy(np.ascontiguousarray(c.q[:, :, -1])).to(dev)
    cache = B.alloc_cache(1, 4, KV, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, dev, v_op_format=B.PV_FP8)
    out = torch.empty((1, Hq, L, D), dtype=torch.float16, device=dev)
    dout = torch.empty((1, Hq, D), dtype=torch.float16, device=dev)
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    pairs = visible_pairs(L, KV, q_off, Hq)
    prefill_ops = 4 * D * pairs
    decode_ops = 4 * D * KV * Hq
    step_ops = prefill_ops + decode_ops

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        B.kv_quantize_i8(k16, v16, cache)
        if ev:
            ev[1].record(stream)
        B.attn_q_prefill(q16, cache, kv_len=KV, q_offset=q_off, causal=True, out=out)
        if ev:
            ev[2].record(stream)
        B.attn_q_decode(qdec, cache, kv_len=KV, out=dout)
        if ev:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ------------------------------------------------------------ timed steps
    # The step's launches are captured once as a HIP graph and the graph is replayed per step
    # (the same kernels on the same buffers; the graph replay matches eager launches byte for
    # byte, tests/test_gpu_graph.py), so the host's per-call marshalling stays out of the
    # device timeline.  --no-graphs times eager launches instead.
    run_step = step
    if not args.no_graphs:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        torch.cuda.synchronize()
        step_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(step_graph, stream=side):
            step()
        torch.cuda.synchronize()
        step_graph.replay()
        torch.cuda.synchronize()
        run_step = step_graph.replay
    # (measured: the prompt chunk's prefill takes ~400 us in the first launches of a process
    #  and settles at ~335 us after ~60 launches, and the clock drops again while the GPU idles,
    #  e.g. during the graph capture above; so the untimed steps run right before the timed
    #  ones, with the same launches, and the timed steps measure the settled clock)
    n_clock_warm = 0
    t_w = time.perf_counter()
    while (time.perf_counter() - t_w) * 1e3 < args.warmup_ms:
        for _ in range(8):      # (back to back, as the timed steps run)
            run_step()
        torch.cuda.synchronize()
        n_clock_warm += 8
    print(f"# clock warm-up: {n_clock_warm} untimed steps in {args.warmup_ms:.0f} ms", file=sys.stderr, flush=True)
    t_start = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps

    # per-kernel durations with events on the launch stream (separate pass)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    kvq_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    pre_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    pre_tops = prefill_ops / (pre_ms * 1e-3) / 1e12
    print(f"# step {ms_per_step:.3f} ms | kv_quantize {kvq_ms * 1e3:.1f} us | prefill "
          f"{pre_ms * 1e3:.1f} us = {pre_tops:.1f} TOPS | decode (same cache) {dec_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    # ------------------------------------------------------------ precision mode
    # the same prompt chunk with pv_mode ATTN_Q_PV_SPLIT24 (24-bit operand split, int8 matrix
    # cores for both products; three digit passes each, so 3x the matrix-core work)
    split = None
    if args.split_reps > 0:
        cache8 = B.alloc_cache(1, 4, KV, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, dev, v_op_format=B.PV_INT8)
        B.kv_quantize_i8(k16, v16, cache8)

        def split_call():
            B.attn_q_prefill(q16, cache8, kv_len=KV, q_offset=q_off, causal=True, out=out, pv_mode=B.PV_SPLIT24)

        split_call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.split_reps):
            split_call()
        e1.record(stream)
        torch.cuda.synchronize()
        sp_us = e0.elapsed_time(e1) * 1e3 / args.split_reps
        split = {"kernel": "prefill_split24_kernel", "launch_us": sp_us,
                 "algorithmic_TOPS": prefill_ops / (sp_us * 1e-6) / 1e12,
                 "int8_mfma_TOPS_executed": 3 * prefill_ops / (sp_us * 1e-6) / 1e12,
                 "frac_int8_peak_executed": 3 * prefill_ops / (sp_us * 1e-6) / 1e12 / PEAK_TOPS}
        print(f"# prefill split24 (precision mode): {sp_us:.1f} us = {split['algorithmic_TOPS']:.0f} TOPS "
              f"algorithmic, {split['int8_mfma_TOPS_executed']:.0f} TOPS executed on int8 MFMA",
              file=sys.stderr, flush=True)
        del cache8

    # ------------------------------------------------------------ Q and K below 8 bits
    # The prompt chunk with Q and K as MX operands (E2M1 or E2M3 elements, one E8M0 scale per
    # 32 channels) on the scaled fp4 / fp6 matrix cores; the same V operand, P and softmax.
    # Half the algorithmic ops (QK) run on fp4 / fp6, half (PV) on fp8: the dense peak of that
    # mix is 1 / (0.5 / 10.1 + 0.5 / 5.0) = 6.69 POP/s.
    mxrec = None
    if args.mx_reps > 0:
        mxrec = {"workload": "the prompt chunk (GQA 16/4, d=128, 2048 queries x 32768 keys, causal) with Q and K "
                             "MX-encoded", "peak_TOPS_mixed": 1.0 / (0.5 / 10100.0 + 0.5 / 5000.0)}
        for name, fmt in (("mxfp4", B.MX_FP4), ("mxfp6", B.MX_FP6)):
            keys = B.alloc_mx_keys(1, 4, KV, D, fmt, dev)
            B.attn_q_k_quantize_mx(k16, cache.k_mean, keys)
            B.attn_q_prefill_mx(q16, keys, cache, kv_len=KV, q_fmt=fmt, q_offset=q_off, causal=True, out=out)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            for _ in range(args.mx_reps):
                B.attn_q_k_quantize_mx(k16, cache.k_mean, keys)
            ev[1].record(stream)
            for _ in range(args.mx_reps):
                B.attn_q_prefill_mx(q16, keys, cache, kv_len=KV, q_fmt=fmt, q_offset=q_off, causal=True, out=out)
            ev[2].record(stream)
            torch.cuda.synchronize()
            kq_us = ev[0].elapsed_time(ev[1]) * 1e3 / args.mx_reps
            p_us = ev[1].elapsed_time(ev[2]) * 1e3 / args.mx_reps
            tops = prefill_ops / (p_us * 1e-6) / 1e12
            mxrec[name] = {"kernel": "prefill_mx_kernel", "launch_us": p_us, "TOPS": tops,
                           "frac_mixed_peak": tops / mxrec["peak_TOPS_mixed"], "k_quantize_mx_us": kq_us}
            print(f"# prefill {name} (Q, K): {p_us:.1f} us = {tops:.0f} TOPS; K encoding {kq_us:.1f} us",
                  file=sys.stderr, flush=True)
            del keys

    # ------------------------------------------------------------ decode vs HBM
    c4 = inputs.config4()[0]
    base = B.alloc_cache(1, 4, KV, D, B.GRAN_TOKEN, B.GRAN_TOKEN, dev, v_op_format=None)
    B.kv_quantize_i8(torch.from_numpy(c4.k).to(dev), torch.from_numpy(c4.v).to(dev), base)
    q4 = torch.from_numpy(np.ascontiguousarray(c4.q[:, :, 0])).to(dev)
    caches = []
    for _ in range(args.decode_caches):
        cc = B.alloc_cache(1, 4, KV, D, B.GRAN_TOKEN, B.GRAN_TOKEN, dev, v_op_format=None)
        for f in ("k_codes", "v_codes", "k_scales", "v_scales", "k_mean"):
            getattr(cc, f).copy_(getattr(base, f))
        caches.append(cc)
    dec_bytes = 2 * 4 * KV * D + 2 * 4 * KV * 2 + Hq * D * 2 * 2
    # One HIP graph replays the 32 launches back to back, so the figure is the
    # device time of the decode kernels, not the Python launch path between them.
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for cc in caches[:2]:
            B.attn_q_decode(q4, cc, kv_len=KV, out=dout)
    torch.cuda.synchronize()
    dts = []
    if args.decode_reps > 0:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for cc in caches:
                B.attn_q_decode(q4, cc, kv_len=KV, out=dout)
        graph.replay()
        torch.cuda.synchronize()
        # (the clock settles under back-to-back replays first, as for the step)
        t_w = time.perf_counter()
        while (time.perf_counter() - t_w) * 1e3 < min(args.warmup_ms, 50.0):
            for _ in range(4):
                graph.replay()
            torch.cuda.synchronize()
    for _ in range(args.decode_reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        dts.append(e0.elapsed_time(e1) / len(caches))
    dec4_us = dec_gbs = None
    if dts:
        dec4_us = float(np.median(dts)) * 1e3
        dec_gbs = dec_bytes / (dec4_us * 1e-6) / 1e9
        print(f"# decode (graph of 32 rotated per-token caches): median {dec4_us:.2f} us = "
              f"{dec_gbs:.0f} GB/s", file=sys.stderr, flush=True)

    # ------------------------------------------------------------ KV append
    # The decode-time cache update: the token after a 32767-token prompt is appended to
    # each of the rotated caches with the running K mean of its header (one launch per
    # call), alone and followed by the decode of the grown cache (the whole per-token
    # step); then a 1024-token chunk after a 31744-token prompt (chunk sums, scan, codes).
    app = None

    def graph_us(body, reps, per):
        body()                                   # warm-up outside capture (workspaces)
        torch.cuda.synchronize()
        if args.no_graphs:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                body()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * per)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            body()
        g.replay()
        torch.cuda.synchronize()
        # (the clock settles under back-to-back replays first, as for the step)
        t_w = time.perf_counter()
        while (time.perf_counter() - t_w) * 1e3 < min(args.warmup_ms, 50.0):
            for _ in range(4):
                g.replay()
            torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / per)
        return float(np.median(ts))

    if args.append_reps > 0:
        k4, v4 = torch.from_numpy(c4.k).to(dev), torch.from_numpy(c4.v).to(dev)
        P1 = KV - 1
        hdr = B.alloc_cache(1, 4, KV, D, B.GRAN_TOKEN, B.GRAN_TOKEN, dev, v_op_format=None, header=True)
        B.kv_quantize_i8(k4[:, :, :P1].contiguous(), v4[:, :, :P1].contiguous(), hdr)
        for cc in caches:
            for f in ("k_codes", "v_codes", "k_scales", "v_scales", "k_mean"):
                getattr(cc, f).copy_(getattr(hdr, f))
            cc.k_sum = hdr.k_sum.clone()
        k1, v1 = k4[:, :, P1:].contiguous(), v4[:, :, P1:].contiguous()

        def appends(decode: bool):
            def body():
                for cc in caches:
                    cc.seq_len = P1
                    B.attn_q_kv_append_i8(k1, v1, cc)
                    if decode:
                        B.attn_q_decode(q4, cc, kv_len=KV, out=dout)
            return body

        app1_us = graph_us(appends(False), args.append_reps, len(caches))
        step_us = graph_us(appends(True), args.append_reps, len(caches))
        k1d, v1d = k1[:, :, 0].contiguous(), v1[:, :, 0].contiguous()

        def fused():
            for cc in caches:
                cc.seq_len = P1
                B.attn_q_decode_append(q4, k1d, v1d, cc, out=dout)

        fused_us = graph_us(fused, args.append_reps, len(caches))
        T = 1024
        P2 = KV - T
        big = B.alloc_cache(1, 4, KV, D, B.GRAN_TOKEN, B.GRAN_TOKEN, dev, v_op_format=None, header=True)
        B.kv_quantize_i8(k4[:, :, :P2].contiguous(), v4[:, :, :P2].contiguous(), big)
        kT, vT = k4[:, :, P2:].contiguous(), v4[:, :, P2:].contiguous()
        s0 = big.k_sum.clone()

        def chunk():
            for _ in range(8):
                big.seq_len = P2
                B.attn_q_kv_append_i8(kT, vT, big)

        appT_us = graph_us(chunk, args.append_reps, 8)
        big.k_sum.copy_(s0)

        def app_bytes(t):   # fp16 K, V in; int8 codes and fp16 scales out; header in and out; mean out
            return t * 4 * D * (2 + 2 + 1 + 1) + t * 4 * 2 * 2 + 4 * D * (8 + 8 + 4)

        app = {"kernel": "attn_q_kv_append_i8",
               "workload": "append after a 32767-token prompt, GQA 4 kv heads, d=128, per-token fp16 "
                           "scales, 32 rotated caches replayed as one HIP graph",
               "bytes_per_call": app_bytes(1), "median_call_us": app1_us, "bound": "launch latency",
               "decode_step_us": step_us,
               "decode_step": "append of the new token + attn_q_decode over the 32768-token cache",
               "fused_step_us": fused_us,
               "fused_step": "attn_q_decode_append: the same step in one launch (the decode workgroup "
                             "holding the new key appends it)",
               "chunk_tokens": T, "chunk_call_us": appT_us, "chunk_bytes": app_bytes(T),
               "chunk_GBs": app_bytes(T) / (appT_us * 1e-6) / 1e9}
        print(f"# append 1 token: {app1_us:.2f} us | append + decode: {step_us:.2f} us | fused step: "
              f"{fused_us:.2f} us | append {T} "
              f"tokens: {appT_us:.2f} us = {app['chunk_GBs']:.0f} GB/s", file=sys.stderr, flush=True)

    # ------------------------------------------------------------ short sequences
    # attn_q_short_fused (quantization + attention of a head in one kernel) at the ViT-B
    # shape of the vision workload (batch 64, 12 heads, 197 tokens, d = 64) and at Swin's
    # first stage (QFlash Table 1, A4) at batch 8; at ViT-B also the two-kernel path
    # (kv_quantize_i8 + attn_q_prefill, per-tensor Q and K scales) on the same tensors.
    short = None
    if args.short_reps > 0:
        short = {}
        for label, cs in (("vit_b_x64", inputs.config2()), ("swin_a4_x8", inputs.vision("A4", 8))):
            qs_, ks_, vs_ = (torch.from_numpy(x).to(dev) for x in (cs.q, cs.k, cs.v))
            so = torch.empty(qs_.shape, dtype=torch.float16, device=dev)

            def fused(qs_=qs_, ks_=ks_, vs_=vs_, so=so):
                for _ in range(10):
                    B.attn_q_short_fused(qs_, ks_, vs_, out=so)

            us = graph_us(fused, args.short_reps, 10)
            Bn, Hh, Nn, Dd = cs.q.shape
            nbytes = 4 * Bn * Hh * Nn * Dd * 2          # fp16 Q, K, V in, fp16 O out
            ops = 4 * Dd * Nn * Nn * Bn * Hh
            rec_s = {"shape_BHNd": [Bn, Hh, Nn, Dd], "launch_us": us, "bytes_per_launch": nbytes,
                     "achieved_GBs": nbytes / (us * 1e-6) / 1e9,
                     "frac_hbm": nbytes / (us * 1e-6) / 1e9 / PEAK_GBS, "TOPS": ops / (us * 1e-6) / 1e12}
            if label == "vit_b_x64":
                rec_s["traffic"] = measured_traffic("attn_q_short_fused", [
                    "quantized_attention_attn_amd/csrc/short_fused.hip",
                    "quantized_attention_attn_amd/csrc/common.h"])
                cap = (Nn + 63) // 64 * 64
                vc = B.alloc_cache(Bn, Hh, cap, Dd, B.GRAN_TENSOR, B.GRAN_CHANNEL, dev, v_op_format=B.PV_FP8)
                po = torch.empty(qs_.shape, dtype=torch.float16, device=dev)

                def two_kernel(qs_=qs_, ks_=ks_, vs_=vs_, vc=vc, po=po):
                    B.kv_quantize_i8(ks_, vs_, vc)
                    B.attn_q_prefill(qs_, vc, kv_len=Nn, q_gran=B.GRAN_TENSOR, out=po)

                rec_s["two_kernel_path_us"] = graph_us(two_kernel, args.short_reps, 1)
            short[label] = rec_s
            print(f"# short {label} {[Bn, Hh, Nn, Dd]}: {us:.2f} us = {rec_s['achieved_GBs']:.0f} GB/s"
                  + (f" | two-kernel path {rec_s['two_kernel_path_us']:.2f} us" if "two_kernel_path_us" in rec_s else ""),
                  file=sys.stderr, flush=True)

    # ------------------------------------------------------------ long-context prefill
    # GQA 32 q / 8 kv heads, d = 128, 131072 keys quantized once (per-channel K and V, K mean
    # subtracted), then the prompt's 16 chunks of 8192 queries, chunk c causal at q_offset
    # 8192c over the first 8192(c+1) keys: 140.7 Tops of algorithmic work per pass.
    c5rec = None
    c5 = None
    if args.c5_reps > 0 or not args.no_accuracy:
        t0 = time.time()
        k5, v5, par5 = inputs.config5_kv()
        cache5 = B.alloc_cache(1, 8, 131072, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, dev, v_op_format=B.PV_FP8,
                               v_codes=False)   # (prefill only: no int8 V codes beside the operand)
        k5d, v5d = torch.from_numpy(k5).to(dev), torch.from_numpy(v5).to(dev)
        B.kv_quantize_i8(k5d, v5d, cache5)
        c5 = dict(k=k5, v=v5, par=par5, cache=cache5, kd=k5d, vd=v5d)
        print(f"# long-context cache ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    if args.c5_reps > 0:
        t0 = time.time()
        q5 = [torch.from_numpy(inputs.config5_chunk_q(c5["par"], ch)).to(dev) for ch in range(16)]
        print(f"# long-context queries ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        out5 = torch.empty((1, 32, 8192, D), dtype=torch.float16, device=dev)
        c5_ops = [4 * D * visible_pairs(8192, 8192 * (ch + 1), 8192 * ch, 32) for ch in range(16)]

        def c5_pass(evs=None):
            for ch in range(16):
                if evs:
                    evs[ch].record(stream)
                B.attn_q_prefill(q5[ch], cache5, kv_len=8192 * (ch + 1), q_offset=8192 * ch, causal=True,
                                 out=out5)
            if evs:
                evs[16].record(stream)

        c5_pass()
        torch.cuda.synchronize()
        passes = []
        for _ in range(args.c5_reps):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(17)]
            c5_pass(evs)
            torch.cuda.synchronize()
            passes.append([evs[ch].elapsed_time(evs[ch + 1]) for ch in range(16)])
        per_chunk_ms = np.median(np.array(passes), axis=0)
        tot_ms = float(np.sum(per_chunk_ms))
        tops5 = sum(c5_ops) / (tot_ms * 1e-3) / 1e12
        c5rec = {"kernel": "attn_q_prefill",
                 "workload": "long-context prefill: GQA 32q/8kv, d=128, 131072-key int8 cache quantized once, "
                             "16 causal chunks of 8192 queries (q_offset 8192c)",
                 "ops_per_pass": sum(c5_ops), "ms_per_pass": tot_ms, "TOPS": tops5,
                 "frac_peak": tops5 / PEAK_TOPS, "target_ms_at_half_peak": sum(c5_ops) / (0.5 * PEAK_TOPS * 1e12) * 1e3,
                 "chunk_ms": [round(float(x), 3) for x in per_chunk_ms],
                 "chunk_TOPS": [round(o / (t * 1e-3) / 1e12, 1) for o, t in zip(c5_ops, per_chunk_ms)]}
        print(f"# long-context prefill: 16 chunks {tot_ms:.2f} ms = {tops5:.0f} TOPS ({tops5 / PEAK_TOPS:.3f} of "
              f"peak); last chunk {per_chunk_ms[-1]:.2f} ms", file=sys.stderr, flush=True)
        del q5

    # ------------------------------------------------------------ accuracy report
    # fp8-PV and int8-PV outputs of the GPU (fp32 output) against fp64 attention on the fp16
    # inputs, at 256 keys (the outlier case), 32768 keys (the prompt chunk, every 64th query
    # row of every head and each head's last row) and 131072 keys (the long-context prompt's
    # last chunk, every 1024th row and each head's last); flushed mass = the share of the
    # softmax mass whose P code is 0 (the oracle's emulation of the same rows, whose P codes
    # the GPU's equal), averaged over the rows.
    acc = None
    if not args.no_accuracy:
        import oracle

        def sample_rows(Hq_, L_, step_):
            r = []
            for h in range(Hq_):
                r.extend(h * L_ + i for i in list(range(0, L_, step_)) + [L_ - 1])
            return np.array(sorted(set(r)), np.int64)

        def metrics(o, e):
            o, e = np.asarray(o, np.float64), np.asarray(e, np.float64)
            den = np.abs(e).max(axis=-1, keepdims=True)
            return {"cos": float((o.ravel() @ e.ravel()) / np.sqrt((o.ravel() @ o.ravel()) * (e.ravel() @ e.ravel()))),
                    "max_rel_err": float(np.max(np.abs(o - e) / den)),
                    "rel_l2": float(np.linalg.norm(o - e) / np.linalg.norm(e))}

        def acc_case(label, q_np, k_np, v_np, causal, q_off, kv_len, rows, cache_fp8, cache_i8, kd=None, vd=None):
            t0 = time.time()
            Hq_, L_, D_ = q_np.shape[1], q_np.shape[2], q_np.shape[3]
            exact = oracle.attn_exact(q_np, k_np, v_np, causal=causal, q_offset=q_off, rows=rows)
            exact = exact.reshape(-1, D_) if rows is None else exact.reshape(-1, D_)[rows]
            oc = oracle.kv_quantize(k_np, v_np, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL)
            rec_a = {"keys": kv_len, "rows": int(exact.shape[0])}
            qd = torch.from_numpy(q_np).to(dev)
            for name, pv, cch in (("fp8_pv", B.PV_FP8, cache_fp8), ("int8_pv", B.PV_INT8, cache_i8)):
                o = B.attn_q_prefill(qd, cch, kv_len=kv_len, q_offset=q_off, causal=causal, pv_mode=pv,
                                     out_dtype=B.OUT_F32)
                torch.cuda.synchronize()
                o = o.cpu().numpy().reshape(-1, D_)
                o = o if rows is None else o[rows]
                m = metrics(o, exact)
                em = oracle.prefill_emulate(q_np, oc, kv_len=kv_len, q_offset=q_off, causal=causal, pv_mode=pv,
                                            rows=rows)
                fm = em.flushed_mass.reshape(-1)
                m["flushed_mass"] = float(np.mean(fm if rows is None else fm[rows]))
                rec_a[name] = m
            rec_a["int8_over_fp8_rel_l2"] = rec_a["int8_pv"]["rel_l2"] / rec_a["fp8_pv"]["rel_l2"]
            if kd is not None:   # Q and K as MX operands (fp8 PV on the same cache)
                for name, fmt in (("mxfp6_qk", B.MX_FP6), ("mxfp4_qk", B.MX_FP4)):
                    keys = B.alloc_mx_keys(1, k_np.shape[1], cache_fp8.capacity, D_, fmt, dev)
                    B.attn_q_k_quantize_mx(kd, cache_fp8.k_mean, keys)
                    o = B.attn_q_prefill_mx(qd, keys, cache_fp8, kv_len=kv_len, q_fmt=fmt, q_offset=q_off,
                                            causal=causal, out_dtype=B.OUT_F32)
                    torch.cuda.synchronize()
                    o = o.cpu().numpy().reshape(-1, D_)
                    rec_a[name] = metrics(o if rows is None else o[rows], exact)
                    del keys
            print(f"# accuracy {label} ({kv_len} keys, {rec_a['rows']} rows): fp8-PV cos "
                  f"{rec_a['fp8_pv']['cos']:.6f} rel-L2 {rec_a['fp8_pv']['rel_l2']:.4f} | int8-PV cos "
                  f"{rec_a['int8_pv']['cos']:.6f} rel-L2 {rec_a['int8_pv']['rel_l2']:.4f} | flushed mass "
                  f"{rec_a['fp8_pv']['flushed_mass']:.2e} vs {rec_a['int8_pv']['flushed_mass']:.3f} "
                  f"({time.time() - t0:.1f}s)", file=sys.stderr, flush=True)
            if "mxfp6_qk" in rec_a:
                print(f"#   with Q and K as MX operands: fp6 cos {rec_a['mxfp6_qk']['cos']:.6f}, fp4 cos "
                      f"{rec_a['mxfp4_qk']['cos']:.6f}", file=sys.stderr, flush=True)
            return rec_a

        def i8_cache(kd, vd, Hkv_, cap_):
            ci = B.alloc_cache(1, Hkv_, cap_, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, dev, v_op_format=B.PV_INT8)
            B.kv_quantize_i8(kd, vd, ci)
            return ci

        acc = {}
        c1 = inputs.config1()
        k1d, v1d = torch.from_numpy(c1.k).to(dev), torch.from_numpy(c1.v).to(dev)
        c1f = B.alloc_cache(1, 1, 256, D, B.GRAN_CHANNEL, B.GRAN_CHANNEL, dev, v_op_format=B.PV_FP8)
        B.kv_quantize_i8(k1d, v1d, c1f)
        acc["outlier_256"] = acc_case("outlier case", c1.q, c1.k, c1.v, False, 0, 256, None, c1f,
                                      i8_cache(k1d, v1d, 1, 256), kd=k1d)
        acc["prompt_chunk_32768"] = acc_case("prompt chunk", c.q, c.k, c.v, True, q_off, KV,
                                             sample_rows(Hq, L, 64), cache, i8_cache(k16, v16, 4, KV), kd=k16)
        q5l = inputs.config5_chunk_q(c5["par"], 15)
        acc["long_context_last_chunk_131072"] = acc_case(
            "long-context last chunk", q5l, c5["k"], c5["v"], True, 131072 - 8192, 131072,
            sample_rows(32, 8192, 1024), c5["cache"], i8_cache(c5["kd"], c5["vd"], 8, 131072), kd=c5["kd"])
        acc["gap_grows_with_context"] = bool(
            acc["outlier_256"]["int8_over_fp8_rel_l2"] < acc["prompt_chunk_32768"]["int8_over_fp8_rel_l2"]
            < acc["long_context_last_chunk_131072"]["int8_over_fp8_rel_l2"])
    c5 = None

    # ------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oc = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL)
        rows = []
        for h in range(Hq):
            rows.extend(h * L + i for i in range(0, L, args.cpu_rows_step))
        rows = np.array(rows, np.int64)
        threads = oracle.num_threads()
        t1 = time.perf_counter()
        oracle.prefill_emulate(c.q, oc, kv_len=KV, q_offset=q_off, causal=True, rows=rows)
        cpu_s = time.perf_counter() - t1
        i_s = rows % L
        sample_pairs = int(np.minimum(KV, q_off + i_s + 1).sum())
        cpu_tops = 4 * D * sample_pairs / cpu_s / 1e12
        # the fp64 exact attention on every 16th of the same rows (its inner loops read fp16 K/V)
        rows_x = rows[::16]
        t1 = time.perf_counter()
        oracle.attn_exact(c.q, c.k, c.v, causal=True, q_offset=q_off, rows=rows_x)
        exact_s = time.perf_counter() - t1
        exact_pairs = int(np.minimum(KV, q_off + rows_x % L + 1).sum())
        # one thread: the outlier case (256 x 256, one head), emulation and exact
        c1o = inputs.config1()
        o1 = oracle.kv_quantize(c1o.k, c1o.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL)
        oracle.set_threads(1)
        t1 = time.perf_counter()
        oracle.prefill_emulate(c1o.q, o1, kv_len=256, q_offset=0, causal=False)
        one_emu_s = time.perf_counter() - t1
        t1 = time.perf_counter()
        oracle.attn_exact(c1o.q, c1o.k, c1o.v)
        one_exact_s = time.perf_counter() - t1
        oracle.set_threads(threads)
        cpu_model = ""
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = {"value": cpu_tops, "unit": "TOPS", "cores": threads, "kind": "oracle",
               "sample": (f"prefill emulation of {'all' if args.cpu_rows_step == 1 else f'every {args.cpu_rows_step}-th of the'} "
                          f"{L} query rows of all {Hq} heads of the prompt chunk ({len(rows)} rows, {sample_pairs} "
                          f"query-key pairs) in {cpu_s:.2f} s"),
               "cpu_model": cpu_model, "os_cpu_count": os.cpu_count(),
               "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
               "exact_fp64": {"TOPS": 4 * D * exact_pairs / exact_s / 1e12, "seconds": exact_s,
                              "sample": f"fp64 exact attention of {len(rows_x)} of the same rows ({exact_pairs} pairs)"},
               "one_thread_outlier_256": {"emulation_s": one_emu_s, "exact_fp64_s": one_exact_s,
                                          "emulation_TOPS": 4 * D * 256 * 256 / one_emu_s / 1e12,
                                          "exact_TOPS": 4 * D * 256 * 256 / one_exact_s / 1e12}}
        print(f"# cpu oracle ({cpu_model}): {cpu_tops * 1e3:.3f} GOPS emulation, "
              f"{cpu['exact_fp64']['TOPS'] * 1e3:.3f} GOPS fp64 exact, on {threads} threads ({cpu_s:.1f} s); "
              f"1 thread, outlier case: emulation {one_emu_s * 1e3:.1f} ms, exact {one_exact_s * 1e3:.1f} ms",
              file=sys.stderr, flush=True)

    rec = {
        "metric": METRIC,
        "value": step_ops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_ms": args.warmup_ms,
        "ms_per_step": ms_per_step,
        "step_launch": "eager" if args.no_graphs else "hip_graph",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xi8->i32 QK, e4m3xe4m3->f32 PV, f32 softmax",
        "data": "synthetic",
        "config": {"workload": "LLM prompt chunk: GQA 16q/4kv, d=128, 2048 queries x 32768-key int8 KV "
                               "cache, causal in chunk; step = kv_quantize_i8 + attn_q_prefill + "
                               "attn_q_decode (next token)",
                   "global_batch": 1, "seq_len": KV, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "attn_q_prefill", "achieved": pre_tops, "peak": PEAK_TOPS,
                     "unit": "TOPS", "frac": pre_tops / PEAK_TOPS,
                     "traffic": measured_traffic("attn_q_prefill", [
                         "quantized_attention_attn_amd/csrc/prefill.hip",
                         "quantized_attention_attn_amd/csrc/common.h"]),
                     "ops_per_launch": prefill_ops, "avg_launch_us": pre_ms * 1e3},
        "decode": {"kernel": "attn_q_decode", "workload": "GQA 16/4, d=128, 32768-token int8 cache, "
                   "per-token fp16 K/V scales, 32 rotated copies replayed as one HIP graph", "bytes_per_launch": dec_bytes,
                   "median_launch_us": dec4_us, "achieved_GBs": dec_gbs, "peak_GBs": PEAK_GBS,
                   "frac": dec_gbs / PEAK_GBS if dec_gbs else None,
                   "traffic": measured_traffic("attn_q_decode", [
                       "quantized_attention_attn_amd/csrc/decode.hip",
                       "quantized_attention_attn_amd/csrc/common.h"]),
                   "tok_per_s_per_layer": 1e6 / dec4_us if dec4_us else None},
        "prefill_long_context": c5rec,
        "accuracy": acc,
        "prefill_split24": split,
        "prefill_mx": mxrec,
        "kv_append": app,
        "short_fused": short,
        "kv_quantize_us": kvq_ms * 1e3,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

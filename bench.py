"""Benchmark of the quantized-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. kv_quantize_i8 : 32768-key fp16 K/V cache of the LLM prompt-chunk workload
                      (GQA 16 q / 4 kv heads, d=128) -> int8 cache with per-channel
                      scales, K-mean subtracted, e4m3 PV operand;
  2. attn_q_prefill : the 2048-query chunk at the end of that context, causal within
                      the chunk, int8 QK^T / fp32 online softmax / e4m3-P fp8 PV;
  3. attn_q_decode  : the next token's 16 query heads against the same int8 cache.
``value`` = algorithmic tera-ops of a step / step wall time (inputs resident in HBM).
The ``roofline`` object reports the dominant kernel (attn_q_prefill) against the
dense int8/fp8 matrix-core peak; ``decode`` reports the int8-KV decode kernel on the
32768-token per-token-scale cache, rotated over 32 distinct copies so it is not
served from the 256 MB on-die cache, against HBM peak.  ``kv_append`` reports the
decode-time cache update (attn_q_kv_append_i8: the new token appended with the running
K mean of the cache header), alone and followed by the decode, and a 1024-token chunk.
``prefill_split24`` times the precision mode (24-bit operand split) on the same prompt chunk.
``short_fused`` reports the one-pass short-sequence kernel at the vision shapes against
HBM peak (and, at ViT-B, the two-kernel quantize + prefill path on the same tensors).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
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
    ap.add_argument("--decode-caches", type=int, default=32)
    ap.add_argument("--decode-reps", type=int, default=10,
                    help="graph replays of the rotated-cache decode timing (0: skip it)")
    ap.add_argument("--append-reps", type=int, default=10,
                    help="graph replays of the KV-append timings (0: skip them)")
    ap.add_argument("--split-reps", type=int, default=5,
                    help="launches of the precision-mode prefill timing (0: skip it)")
    ap.add_argument("--short-reps", type=int, default=10,
                    help="replays of the short-sequence (vision) timings (0: skip them)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="time the append and short-sequence sections eagerly (for counter runs)")
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
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
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

    # ------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oc = oracle.kv_quantize(c.k, c.v, oracle.GRAN_CHANNEL, oracle.GRAN_CHANNEL)
        rows = []
        for h in range(Hq):
            rows.extend(h * L + i for i in range(0, L, args.cpu_rows_step))
        rows = np.array(rows, np.int64)
        t1 = time.perf_counter()
        oracle.prefill_emulate(c.q, oc, kv_len=KV, q_offset=q_off, causal=True, rows=rows)
        cpu_s = time.perf_counter() - t1
        i_s = rows % L
        sample_pairs = int(np.minimum(KV, q_off + i_s + 1).sum())
        cpu_tops = 4 * D * sample_pairs / cpu_s / 1e12
        cpu = {"value": cpu_tops, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": (f"prefill emulation of {'all' if args.cpu_rows_step == 1 else f'every {args.cpu_rows_step}-th of the'} "
                          f"{L} query rows of all {Hq} heads ({len(rows)} rows, {sample_pairs} query-key pairs) "
                          f"in {cpu_s:.2f} s")}
        print(f"# cpu oracle: {cpu_tops * 1e3:.3f} GOPS on {cpu['cores']} threads ({cpu_s:.1f} s)",
              file=sys.stderr, flush=True)

    rec = {
        "metric": METRIC,
        "value": step_ops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
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
        "prefill_split24": split,
        "kv_append": app,
        "short_fused": short,
        "kv_quantize_us": kvq_ms * 1e3,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

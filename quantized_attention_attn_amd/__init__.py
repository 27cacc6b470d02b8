"""attn_q: quantized flash attention for MI355X (gfx950).

int8 QK^T after per-channel K-mean subtraction, fp32 online softmax, e4m3 P with
a static scale of 448 and fp8 PV, plus an int8-KV decode path -- hand-written
HIP kernels behind the C ABI in ``include/attn_q.h``.  The Python side only
marshals arguments (``quantized_attention_attn_amd.binding``); ``inputs`` holds
the seeded synthetic workloads.
"""
__all__ = ["binding", "inputs"]

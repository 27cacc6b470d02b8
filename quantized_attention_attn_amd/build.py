"""Build libattn_q.so (gfx950) in-tree with hipcc.

    python -m quantized_attention_attn_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_q.so")
SOURCES = ["attn_q_host.cpp", "kv_quantize.hip", "kv_append.hip", "prefill.hip", "decode.hip",
           "short_fused.hip", "prefill_split24.hip", "v_operand.hip", "mx.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # fp32 division and sqrt stay correctly rounded; no fast-math anywhere
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # keep MFMA accumulators in ordinary VGPRs (no per-tile AGPR<->VGPR copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libattn_q.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

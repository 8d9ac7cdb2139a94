"""Build libpagedattn.so (HIP, gfx950) in place, next to this file.

Every source is compiled with hipcc for gfx950 only.  Packed-FP32 instruction selection is
turned off (-packed-fp32-ops) and the host pass's warning about that feature is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libpagedattn.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "kv_write.hip", "block_copy.hip", "plan.hip", "attn_valu.hip", "attn_decode_mfma.hip",
           "attn_prefill_mfma.hip", "fp8_stage.hip", "hbm_probe.hip",
           "mfma_probe.hip", "v16_stage.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Per-file extra flags.  The prefill kernel never carries NaN through its arithmetic (keys
# past the visible range are clamped to finite data, masked scores are -inf), so it runs
# with the IEEE mode bit off: max/min then need no operand canonicalisation.
EXTRA = {"attn_prefill_mfma.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()

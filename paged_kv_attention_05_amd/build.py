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
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC,
         "-Rpass-analysis=kernel-resource-usage"]
# Per-kernel resources as the compiler reports them, one line per kernel (written by build()).
RESOURCES = os.path.join(BUILD, "kernel_resources.tsv")
_RES_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
               "Occupancy [waves/SIMD]": "occupancy", "VGPRs Spill": "vgpr_spill",
               "LDS Size [bytes/block]": "lds"}


def _resources(stderr: str) -> list[dict]:
    """The kernel-resource-usage remarks of one compile, one dict per kernel."""
    kernels, cur = [], None
    for line in stderr.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = {"name": val}
            kernels.append(cur)
        elif cur is not None and key in _RES_FIELDS:
            cur[_RES_FIELDS[key]] = int(val)
    return kernels


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    lines = res.stderr.splitlines()
    # drop the remarks and the source excerpts printed under them
    noise, skip = [], 0
    for l in lines:
        if "kernel-resource-usage" in l:
            skip = 2
            continue
        if skip and (l.lstrip().startswith("|") or l.strip()[:1].isdigit()):
            skip -= 1
            continue
        skip = 0
        if "packed-fp32-ops" not in l and l.strip():
            noise.append(l)
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")
    return obj, [dict(k, source=src) for k in _resources(res.stderr)]


def build(verbose: bool = True) -> str:
    """Compile every source, link the library, and write the per-kernel resource report.
    A kernel that spills to scratch fails the build: every kernel here is sized to fit its
    registers, and a spill (a per-lane memory round trip) is a regression."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    kernels = [k for _, ks in done for k in ks]
    cols = ["source", "name", "vgprs", "agprs", "vgpr_spill", "scratch", "lds", "occupancy"]
    with open(RESOURCES, "w") as f:
        f.write("\t".join(cols) + "\n")
        for k in kernels:
            f.write("\t".join(str(k.get(c, "")) for c in cols) + "\n")
    spilled = [k["name"] for k in kernels if k.get("scratch", 0) or k.get("vgpr_spill", 0)]
    if spilled:
        raise RuntimeError("kernels spill registers to scratch: " + ", ".join(spilled))
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()

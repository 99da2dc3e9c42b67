"""Build libmsa.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Run as ``python -m block_sparse_long_qk_amd.build``; no GPU is needed.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmsa.so")
SOURCES = ["index_scores.hip", "block_topk.hip", "gather_plan.hip", "sparse_attn.hip", "decode.hip", "kl.hip",
           "dense.hip", "bwd.hip", "noalloc.hip", "abi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         # keep the compiler from emitting packed fp32 arithmetic
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # inputs are NaN-free by contract: max/min need no NaN quieting
         "-fno-honor-nans",
         # MFMA results in VGPRs (no AGPR round trips before the VALU epilogues)
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def resource_report() -> dict:
    """Per-kernel register, LDS, scratch and occupancy figures from the compiler
    (kernel-resource-usage remarks), keyed by mangled kernel name."""
    import re
    report = {}

    def one(src):
        if not src.endswith(".hip"):
            return ""
        cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage"]
        return subprocess.run(cmd, capture_output=True, text=True).stderr

    with ThreadPoolExecutor(max_workers=4) as ex:
        outs = list(ex.map(one, SOURCES))
    for text in outs:
        name = None
        for line in text.splitlines():
            m = re.search(r"remark:\s+(.*?)\s*\[-Rpass", line)
            if not m:
                continue
            body = m.group(1)
            if body.startswith("Function Name:"):
                name = body.split(":", 1)[1].strip()
                report[name] = {}
            elif name and ":" in body:
                k, v = body.split(":", 1)
                try:
                    report[name][k.strip()] = int(v.strip())
                except ValueError:
                    pass
    return report


if __name__ == "__main__":
    build(verbose=True)

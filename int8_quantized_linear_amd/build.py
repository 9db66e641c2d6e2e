"""Build ``libi8ql.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled on every call (the build is the "does it compile" check), in
parallel, then linked into ``int8_quantized_linear_amd/libi8ql.so``.  Flags: -O3, no
fast-math (the quantizer needs correctly rounded float32 division), and packed-fp32
instruction selection switched off.  The compiler's per-kernel resource report is read
back, and the build fails if any kernel spills registers to scratch memory: every kernel
here is sized to fit its registers, and a spill is a performance bug to fix in the code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libi8ql.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Rpass-analysis=kernel-resource-usage"]
SOURCES = ["api.cpp", "quantize_rows.hip", "w8a8_gemm.hip", "w8a16_gemm.hip",
           "grouped_w8a16.hip", "moe_steps.hip"]


def kernel_resources(stderr: str) -> dict:
    """{kernel: {"vgpr": .., "agpr": .., "spill": .., "scratch": ..}} from the compiler's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: .*Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark: .*?(VGPRs Spill|AGPRs|VGPRs|ScratchSize \[bytes/lane\]): (\d+)",
                      line)
        if m and cur is not None:
            key = {"VGPRs Spill": "spill", "AGPRs": "agpr", "VGPRs": "vgpr"}.get(m.group(1),
                                                                              "scratch")
            cur[key] = int(m.group(2))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    lines = [l for l in r.stderr.splitlines() if noise not in l]
    # (drop the remarks and the source lines the compiler echoes under them)
    err = "\n".join(l for l in lines if "remark:" not in l and not re.match(r"^\s*\d*\s*\|", l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    bad = {k: v for k, v in kernel_resources(r.stderr).items()
           if v.get("spill", 0) or v.get("scratch", 0)}
    if bad:
        raise RuntimeError(f"{src}: kernels spill registers to scratch: {bad}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)

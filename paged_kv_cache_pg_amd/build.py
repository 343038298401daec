"""Build libpagedattn.so for gfx950 in-tree (hipcc, one object per source, then link).

    python -m paged_kv_cache_pg_amd.build          # or __graft_entry__.build()
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-Wall", "-Wno-unused-function",
]


# Per-source extra flags.  prefill.hip: MFMA accumulators in VGPRs, so the softmax's rescale of
# the output accumulators does not move them between AGPRs and VGPRs every tile.
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


# The compiler's per-kernel resource remarks ("Function Name: ...", then "VGPRs: n", "ScratchSize
# [bytes/lane]: n", "VGPRs Spill: n", ...), parsed so that a kernel that spills or uses scratch fails
# the build instead of passing unnoticed.
_REMARK = re.compile(r"remark:\s+(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")


def _resources(stderr: str) -> list:
    """One dict a kernel, in the order the compiler reports them."""
    out = []
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            out.append({"kernel": val})
        elif out:
            out[-1][key.split(" [")[0]] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-Rpass-analysis=kernel-resource-usage",
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    res = _resources(r.stderr)
    # the remarks (and the source lines they quote) are parsed, not echoed
    keep, skip = [], 0
    for line in r.stderr.splitlines():
        if skip:
            skip -= 1
            continue
        if "kernel-resource-usage" in line:
            skip = 2 if "Function Name" in line else 0
            continue
        if "is not a recognized feature" in line:
            continue
        keep.append(line)
    err = "\n".join(keep)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj, res


def check_resources(res: list) -> None:
    """Refuse a kernel that uses scratch memory or spills registers."""
    bad = [k for k in res if k.get("ScratchSize", 0) or k.get("VGPRs Spill", 0) or k.get("SGPRs Spill", 0)]
    if bad:
        lines = "\n".join(f"  {k['kernel']}: scratch {k.get('ScratchSize')} B/lane, VGPR spill "
                          f"{k.get('VGPRs Spill')}, SGPR spill {k.get('SGPRs Spill')}" for k in bad)
        raise RuntimeError(f"kernels that spill or use scratch memory:\n{lines}")


def build(jobs: int = 8) -> str:
    """Compile every HIP source of the library for gfx950 and link the shared library.  Fails when a
    kernel spills registers or uses scratch memory; the per-kernel resources go to _build/resources.txt."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    res = [k for _, r in done for k in r]
    with open(os.path.join(BUILD, "resources.txt"), "w") as f:
        for k in res:
            f.write(f"{k['kernel']}: VGPRs {k.get('VGPRs')} AGPRs {k.get('AGPRs')} SGPRs {k.get('TotalSGPRs')} "
                    f"scratch {k.get('ScratchSize')} LDS {k.get('LDS Size')} occupancy {k.get('Occupancy')}\n")
    check_resources(res)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())

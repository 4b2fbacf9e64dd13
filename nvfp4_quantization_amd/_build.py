"""Build the HIP library (libnvfp4_hip.so) for gfx950 with hipcc, and the streaming kernel the benchmark
compares against (libnvfp4_bench.so, not part of the C ABI).

The libraries are built in-tree next to this file so that they travel with the source tree.  Object files go to
``_build/`` at the repository root.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libnvfp4_hip.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["nvfp4_kernels.hip", "nvfp4_capi.hip"]
BENCH_LIB_PATH = os.path.join(PKG_DIR, "libnvfp4_bench.so")
BENCH_SOURCES = ["bench_stream.hip"]
ARCH = "gfx950"

# -ffp-contract=off: every a*b+c stays two correctly rounded operations (the rounding of each step is part of the
# method).  No fast-math.  Packed FP32 instructions are disabled for the device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the NVFP4 HIP library cannot be built")


RESOURCE_REPORT = os.path.join(ROOT, "_build", "kernel_resources.txt")


def _run(cmd: list[str]) -> str:
    """Runs hipcc; returns the kernel resource-usage remarks it printed (other output is passed through)."""
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass of hipcc does not know the device-only feature flag; that warning is expected
    noise = ("packed-fp32-ops", "warning: unknown target feature", "1 warning generated")
    remarks, kept, in_remark = [], [], False
    for l in (p.stdout + p.stderr).splitlines():
        if "kernel-resource-usage" in l:
            remarks.append(l)
            in_remark = True
        elif in_remark and re.match(r"^\s*\d*\s*\|", l):
            continue                     # the source excerpt clang prints under a remark
        else:
            in_remark = False
            if not any(n in l for n in noise):
                kept.append(l)
    msg = "\n".join(kept)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (p.returncode, " ".join(cmd), msg))
    if msg.strip():
        print(msg)
    return "\n".join(remarks)


def resource_table(remarks: str) -> list[dict]:
    """Per kernel: name, VGPRs, AGPRs, spilled VGPRs and SGPRs, scratch bytes per lane, LDS bytes, occupancy."""
    rows, cur = [], None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill",
            "ScratchSize [bytes/lane]": "scratch", "LDS Size [bytes/block]": "lds",
            "Occupancy [waves/SIMD]": "occupancy"}
    for line in remarks.splitlines():
        body = line.split("remark:", 1)[-1].split("[-Rpass", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = {"name": body.split(":", 1)[1].strip()}
            rows.append(cur)
            continue
        key, sep, val = body.partition(":")
        if cur is not None and sep and key.strip() in keys and val.strip().isdigit():
            cur[keys[key.strip()]] = int(val)
    return rows


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library (always rebuilds)."""
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs, remarks = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", f"-I{INCLUDE}", f"-I{CSRC}", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        remarks.append(_run(cmd))
        objs.append(obj)
    # registers, spills, LDS and occupancy of every kernel, for the build's own check (tests read this file)
    with open(RESOURCE_REPORT, "w") as f:
        for r in resource_table("\n".join(remarks)):
            f.write(" ".join(f"{k}={v}" for k, v in r.items()) + "\n")
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    tmp = BENCH_LIB_PATH + ".tmp%d" % os.getpid()
    _run([hipcc(), *HIPCC_FLAGS, "-shared", *(os.path.join(CSRC, s) for s in BENCH_SOURCES), "-o", tmp])
    os.replace(tmp, BENCH_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libtidar.so for gfx950 in-tree with hipcc (no JIT cache, no install).

The library is the only native artefact: the kernels (attention, verify,
commit) and the C ABI of include/tidar.h.  Every HIP source is compiled with
packed fp32 instructions disabled and MFMA results kept in arch VGPRs.

libtidar_checked.so is the same sources with TIDAR_CHECKED=1: device-side
bounds tests that record the first failure instead of trapping (a debugging
build; tidar_check_read() returns the record)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtidar.so")
LIB_CHECKED = os.path.join(HERE, "libtidar_checked.so")
SOURCES = ["attention.hip", "attention_pp.hip", "verify.hip", "verify_fused.hip", "verify_sample.hip", "lmhead.hip", "commit.hip", "read_probe.hip", "mfma_probe.hip", "capi.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the TiDAR library needs ROCm's hipcc to build")


def _quiet(text: str) -> str:
    # the host pass does not know the packed-fp32 feature flag; that warning is expected
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def _build_one(hipcc: str, lib: str, objdir: str, defines: list, verbose: bool) -> list:
    """Start the compiles of one library variant; returns (src, cmd, proc) triples."""
    os.makedirs(objdir, exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
             "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA results in arch VGPRs: the attention loop feeds its score
             # accumulators straight to the VALU softmax, so results parked in
             # AGPRs would cost a copy per element
             "-mllvm", "-amdgpu-mfma-vgpr-form"] + defines
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc] + flags + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, obj, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    return procs


def _finish(hipcc: str, lib: str, procs: list, verbose: bool) -> str:
    failed, objs = [], []
    for src, obj, cmd, p in procs:
        out, _ = p.communicate()
        out = _quiet(out)
        objs.append(obj)
        if p.returncode != 0:
            failed.append(f"{src}: {' '.join(cmd)}\n{out}")
        elif verbose and out.strip():
            print(out, file=sys.stderr)
    if failed:
        raise RuntimeError("HIP build failed:\n" + "\n".join(failed))
    tmp = lib + ".tmp"
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed: " + " ".join(link) + "\n" + p.stdout)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, checked: bool = True) -> str:
    """Compile every source and link libtidar.so (and, with `checked`,
    libtidar_checked.so); returns the release library's path."""
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    release = _build_one(hipcc, LIB, objdir, [], verbose)
    if checked:  # both variants compile at once (the attention sources dominate either)
        chk = _build_one(hipcc, LIB_CHECKED, os.path.join(objdir, "checked"), ["-DTIDAR_CHECKED=1"], verbose)
        _finish(hipcc, LIB, release, verbose)
        _finish(hipcc, LIB_CHECKED, chk, verbose)
        return LIB
    return _finish(hipcc, LIB, release, verbose)


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the in-tree HIP library libeqlin.so for gfx950 with hipcc.

Usage: python -m group_circulant_linear_amd.build [--verbose] [--resource-usage]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libeqlin.so")
SOURCES = ("eqlin_api.hip", "eqlin_kernels.hip", "eqlin_kernels_c8.hip", "eqlin_kernels_p4m.hip", "eqconv_kernels.hip")
# standalone programs: the measured ceilings of the GPU (matrix-core rates, LDS
# reads, HBM copy), the stage timeline of the forward tile and the check of
# the direct global-to-LDS load the f16 tiles use
PROGRAMS = {"ceilings.hip": os.path.join(LIBDIR, "eqlin_ceilings"),
            "stage_trace.hip": os.path.join(LIBDIR, "eqlin_stage_trace"),
            "dma_check.hip": os.path.join(LIBDIR, "eqlin_dma_check")}
CEILINGS = PROGRAMS["ceilings.hip"]
ARCH = "gfx950"


def hipcc_path() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    found = shutil.which("hipcc")
    return found or "/opt/rocm/bin/hipcc"


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep hipcc from emitting packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    tmpdir = os.path.join(LIBDIR, ".obj")
    os.makedirs(tmpdir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
        cmd = [hipcc_path(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for src, exe in PROGRAMS.items():
        cmd = [hipcc_path(), *compile_flags(), os.path.join(CSRC, src), "-o", exe + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or resource_usage or p.returncode):
            print("\n".join(lines), flush=True)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc_path(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for exe in PROGRAMS.values():
        os.replace(exe + ".tmp", exe)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, resource_usage="--resource-usage" in sys.argv)
    print(LIB)

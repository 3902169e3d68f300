"""Build libwsg.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each translation unit compiles in parallel to an object under _build/, then
one link step writes warp_specialized_gemm_amd/libwsg.so. The build runs
entirely on the CPU (hipcc cross-compiles gfx950 code objects).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwsg.so")
SOURCES = ["abi.hip", "staged_copy.hip", "gemm_bias_relu.hip", "attention.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libwsg.so)")


def compile_flags() -> list:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-I", os.path.join(ROOT, "include"),
        # keep hipcc from forming packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [cc] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.append("--save-temps")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, cwd=BUILD_DIR, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(text, file=sys.stderr)
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)

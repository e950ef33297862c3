"""Builds libvdit.so (HIP, gfx950) in place with hipcc.

    python -m video_diffusion_transformer_rope3d_amd.build [--jobs N]

Every source is compiled for gfx950 only, with packed fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); objects are linked into one shared
library next to this file.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvdit.so")
SOURCES = ["vdit_api.hip", "vdit_kernels.hip", "vdit_attn.hip", "vdit_dynamic.hip", "vdit_reuse.hip",
           "vdit_proj.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def build(jobs: int = 4, verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in ln)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizers: the host code of every source (argument validation, the host plan
# builder, RoPE tables, launch set-up) is built with AddressSanitizer and UndefinedBehaviour-
# Sanitizer; the device code is built as usual.  The library links the shared sanitizer
# runtime, which a process that loads it must preload (sanitizer_runtime()).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtime() -> str:
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for pat in (os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"),
                os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"),
                "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    raise RuntimeError("the shared AddressSanitizer runtime of hipcc's clang was not found")


def build_sanitized(out_dir: str, jobs: int = 4) -> str:
    """libvdit.so with sanitized host code, built under out_dir; returns its path."""
    cc = hipcc()
    os.makedirs(out_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        r = subprocess.run([cc, *flags(), *SANITIZE, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = os.path.join(out_dir, "libvdit.so")
    r = subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))

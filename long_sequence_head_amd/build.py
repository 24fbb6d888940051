"""Builds liblsh.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m long_sequence_head_amd.build [-v]

Every call compiles; the library lands in long_sequence_head_amd/lib/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "liblsh.so"
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "aux_kernels.hip", "api.hip"]
# Per-file code generation options. Every attention file keeps MFMA results
# in VGPRs: the scores feed VALU work directly and the register allocator
# otherwise shuttles them through AGPRs. The dK/dV kernel (attn_bwd.hip)
# pins its 128 accumulators to AGPRs through an inline-asm MFMA instead.
FILE_FLAGS = {"attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "attn_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-variable",
            "-Wno-unused-function"]


def _compile(src: str, obj: str, extra, verbose: bool):
    cmd = [hipcc()] + common_flags() + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l or "error" in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s),
                          os.path.join(BUILD_DIR, s.replace(".hip", ".o")),
                          FILE_FLAGS.get(s, []) + list(extra_flags), verbose)
                for s in SOURCES]
        for f in futs:
            objs.append(f.result())
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    # A kernel whose host-side instantiation was silently dropped leaves an
    # undefined launch stub behind; refuse such a library.
    nm = subprocess.run(["nm", "-u", "-C", tmp], capture_output=True, text=True)
    missing = [l.strip() for l in nm.stdout.splitlines() if "lsh::" in l]
    if missing:
        raise RuntimeError("liblsh.so has undefined symbols of its own:\n" + "\n".join(missing))
    os.replace(tmp, out)
    build_c_abi_check()
    return out


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "lsh_c_abi_check.c")
C_CHECK_BIN = os.path.join(LIBDIR, "lsh_c_abi_check")


def build_c_abi_check() -> str:
    """Compiles the plain-C user of the library (tests/c_abi) with the host
    C compiler against include/lsh.h and the HIP runtime; it finds liblsh.so
    beside itself."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler for the C ABI check")
    tmp = C_CHECK_BIN + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_CHECK_SRC,
           "-L", LIBDIR, "-llsh", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C ABI check build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, C_CHECK_BIN)
    return C_CHECK_BIN


if __name__ == "__main__":
    v = "-v" in sys.argv
    extra = ["-Rpass-analysis=kernel-resource-usage"] if "--usage" in sys.argv else []
    print(build(verbose=v or bool(extra), extra_flags=extra))

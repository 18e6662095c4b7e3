"""Build the HIP library ``libkvq.so`` for gfx950 with hipcc (no torch involved).

Usage: ``python -m quantized_kv_cache_quant_amd.build`` (or ``build()``).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkvq.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (the compiler would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]
# per-source extra flags: the quantizer must round every fp32 step on its own
SOURCES = {
    "kvq_host.cpp": [],
    "kvq_append.hip": ["-ffp-contract=off"],
    "kvq_attn.hip": [],
    "kvq_probe.hip": [],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq.so)")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(bdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = OUT + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


def sanitizer_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (preloaded by a host process that loads
    the sanitizer build)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for pat in (os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"),
                "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    raise RuntimeError("libclang_rt.asan-x86_64.so not found")


def build_host_sanitized(verbose: bool = False) -> str:
    """A copy of the library whose host code (the C ABI: validation, sizing, routing, launch
    set-up) is built with AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests of
    the ABI.  The kernels' objects come from the regular build (compiled first if missing);
    the sanitizers apply to host code only.  Written to _build/sanitized/libkvq.so."""
    cc = hipcc()
    bdir = os.path.join(ROOT, "_build")
    sdir = os.path.join(bdir, "sanitized")
    os.makedirs(sdir, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(bdir, src + ".o")
        if src.endswith(".hip"):
            if not os.path.exists(obj):
                subprocess.run([cc, *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj], check=True)
        else:
            obj = os.path.join(sdir, src + ".o")
            san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
            cmd = [cc, *COMMON, *extra, *san, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
        objs.append(obj)
    out = os.path.join(sdir, "libkvq.so")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

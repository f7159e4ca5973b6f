"""Builds libhgqa.so in this package directory with hipcc for gfx950.

    python -m full_gqa_attention_layer_amd.build [-v]
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libhgqa.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "hgqa_api.cpp")]


def command(out: str = LIB_PATH, extra=()):
    # -z defs: an unresolved symbol (for instance a kernel whose host stub the
    # compiler did not emit) fails the link instead of the first dlopen.
    return ([hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
             "-Wl,-z,defs", "-Wall", "-Wno-unused-function"] + DEVICE_FLAGS + list(extra)
            + sources() + ["-o", out])


def build(verbose: bool = False) -> str:
    """Compile every source into libhgqa.so (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note.
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C-ABI
# front end (device code is built as usual). The runtime is not linked in:
# a process loads the library with the clang ASan runtime preloaded.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-shared-libsan"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that matches hipcc, or "" if absent."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "/opt/rocm/llvm/bin/clang"
    try:
        path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                              capture_output=True, text=True).stdout.strip()
    except OSError:
        return ""
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def build_sanitized(out: str) -> str:
    """libhgqa.so with its host code under ASan + UBSan, written to out."""
    cmd = [c for c in command(out, SANITIZE_HOST) if c != "-Wl,-z,defs"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

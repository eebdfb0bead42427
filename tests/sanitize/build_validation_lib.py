"""Build the host-only validation library for the sanitizer tests.

The C ABI's validation layer (flashattention_forward_amd/csrc/api.cpp) and
the host sizing rules (plan.cpp) are plain C++ that call the kernel launchers
and nothing else of HIP.  Here they are compiled with g++ for the CPU, with
AddressSanitizer and UndefinedBehaviorSanitizer, and linked against the stub
launchers of launch_stubs.cpp into one shared library that exports the same
C ABI (plus attn_stub_launches(), the number of launches asked for).  No
device code is compiled: this is a CPU build of host code only.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "flashattention_forward_amd", "csrc")
OUT = os.path.join(ROOT, "flashattention_forward_amd", "_build", "libattn_validate_san.so")

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build() -> str:
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"), os.path.join(HERE, "launch_stubs.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-shared", "-fPIC", "-Wall", "-Wno-unused-function",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *SANITIZE, "-o", OUT, *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("validation library build failed:\n" + r.stdout + r.stderr)
    return OUT


def runtime_preload() -> str:
    """The sanitizer runtimes to preload into a Python process that loads the
    library (they must come before every other preloaded library)."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p):
            raise RuntimeError(f"{name} not found")
        libs.append(p)
    return ":".join(libs)


if __name__ == "__main__":
    print(build())
    sys.exit(0)

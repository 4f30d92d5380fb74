"""Build the HIP library libtts.so (gfx950) in-tree.

    python -m autoregressive_tts_decode_amd.build [--no-trace]

The library is the whole compute path: C ABI (include/tts.h) + CDNA4 kernels.
libtts_trace.so is the same library built with TTS_PHASE_TRACE: the persistent
kernels stamp their phases (read by ``python -m autoregressive_tts_decode_amd.phase_trace``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libtts.so")
TRACE_LIB = os.path.join(PKG, "libtts_trace.so")
SOURCES = [os.path.join(PKG, "csrc", "tts.hip")]
HEADERS = [os.path.join(PKG, "csrc", "tts_device.h"), os.path.join(PKG, "csrc", "tts_xtp.h"),
           os.path.join(ROOT, "include", "tts.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtts.so)")


def build(verbose: bool = False, trace: bool = False) -> str:
    out = TRACE_LIB if trace else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           *(["-DTTS_PHASE_TRACE"] if trace else []),
           # packed fp32 VALU ops are kept off in all device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    if "--no-trace" not in sys.argv[1:]:
        print(build(verbose=True, trace=True))

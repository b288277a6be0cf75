"""Build the HIP library libmpfa.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmpfa.so")
SOURCES = ["api.hip", "quant.hip", "prefill.hip", "decode.hip"]
HEADERS = ["mpfa_device.hpp", "mpfa_internal.hpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmpfa.so)")


def flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed-FP32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


PEAKS = os.path.join(PKG, "mpfa_peaks")  # standalone probe of the device's ceilings (bench.py)
FP4_CHECK = os.path.join(PKG, "mpfa_fp4_check")  # hardware FP4 conversion check (tests)


def build(verbose: bool = False) -> str:
    """Compile every source into libmpfa.so, the peak probe into mpfa_peaks
    and the FP4 conversion check into mpfa_fp4_check (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    exe_flags = [f for f in flags() if f not in ("-fPIC", "-shared")] + ["-I", CSRC]
    for exe, src in ((PEAKS, "peaks.hip"), (FP4_CHECK, "fp4_check.hip")):
        cmd = [hipcc(), *exe_flags, "-o", exe + ".tmp", os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(exe + ".tmp", exe)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "mpfa.h")]
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


if __name__ == "__main__":
    print(build(verbose=True))

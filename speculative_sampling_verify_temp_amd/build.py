"""Compile the HIP library for gfx950 into the package directory.

    python speculative_sampling_verify_temp_amd/build.py

hipcc cross-compiles without a GPU.  The library lands next to this file as
libsdverify.so and is what the binding loads.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsdverify.so")
SOURCES = ["sd_verify.hip", "sd_confidence.hip", "sd_lmhead.hip"]
ARCH = os.environ.get("SDV_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++20", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # Packed fp32 instructions are kept out of the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The penalty's division must round like IEEE fp32 on both sides.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-result",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; cannot build the HIP library")
    return exe


def build(verbose=False):
    """Compile every HIP source into libsdverify.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

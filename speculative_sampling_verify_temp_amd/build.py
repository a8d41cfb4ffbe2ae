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
    """Compile every HIP source (side by side) and link them into
    libsdverify.so (always rebuilds)."""
    tmpdir = LIB + ".objs"
    os.makedirs(tmpdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-shared"], "-c", f"-I{INCLUDE}",
               f"-I{CSRC}", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            failed.append(f"hipcc failed on {src}:\n{out}")
    if failed:
        raise RuntimeError("\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build ``libmla_decode.so`` in-tree with hipcc for gfx950.

    python -m mla_split_kv_decode_amd.build [-v]

The library holds the HIP kernels and the C ABI of ``include/mla_decode.h``.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_decode.so")
# the same sources with the timeline stamps compiled in (bench.py --timeline only)
LIB_TIMELINE = os.path.join(PKG, "libmla_decode_timeline.so")
SOURCES = ["mla_kernels.hip", "mla_api.hip"]
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def flags():
    """Compiler flags of the library's sources (without inputs, outputs or -shared)."""
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed-fp32 VALU forms are kept out of the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the kernels' leading arguments (what a workgroup needs before its first loads)
        # arrive preloaded in SGPRs on gfx950 instead of through a kernel-argument load
        "-mllvm", "-amdgpu-kernarg-preload-count=14",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(REPO, "include"), "-I", CSRC,
    ]


def command(out=LIB, extra=()):
    return [hipcc(), *flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], *extra, "-o", out]


def device_asm(source, out):
    """Compile one source's device code to gfx950 assembly at `out` (for inspection)."""
    cmd = [hipcc(), *flags(), "--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    return out


def _compile(out, extra, verbose):
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose=False):
    """Compile the library (always, even when one is already built)."""
    return _compile(LIB, (), verbose)


def build_timeline(verbose=False):
    """Compile the timeline variant (include/mla_timeline.h): the same kernels, stamping."""
    return _compile(LIB_TIMELINE, ("-DMLA_TIMELINE=1",), verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--timeline" in sys.argv:
        print(build_timeline(verbose="-v" in sys.argv))

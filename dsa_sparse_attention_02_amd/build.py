"""Build libsparse_attn.so (gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    src = os.path.join(CSRC, "sparse_attn.hip")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libsparse_attn.so")
    if verbose:
        sys.stderr.write(res.stderr)
    # every kernel's host launch stub must be defined in the library
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if nm.returncode != 0 or missing:
        raise RuntimeError(f"libsparse_attn.so has undefined kernel stubs: {missing[:4]}")
    os.replace(tmp, LIB)
    return LIB


PROBE = os.path.join(HERE, "peak_probe")


def build_probe() -> str:
    """The peak-probe executable the benchmark runs for its roofline figures."""
    tmp = PROBE + ".tmp"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", os.path.join(CSRC, "peak_probe.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build peak_probe")
    os.replace(tmp, PROBE)
    return PROBE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe())

"""Build the gfx950 HIP library libpolyact.so in place (hipcc, no JIT cache)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "polyact.hip")
LIB = os.path.join(PKG, "libpolyact.so")

# -ffp-contract=off: every multiply and add is rounded exactly where the
# programs say (no silent fusion).  Packed FP32 instructions are disabled.
# Denormals are preserved (no -ffast-math, no flush-to-zero flags).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# the sources that define the elementwise streaming kernels and their launch
STREAM_SOURCES = ("ops.hpp", "stream.hpp", "stream_launch.hpp", "programs.hpp")


def source_digest(files=STREAM_SOURCES) -> str:
    """SHA-256 over the given csrc/ files (identifies the kernels a stored
    profile was taken from)."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libtes_sampler.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "tes_sampler.hip")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libtes_sampler.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # Packed fp32 instructions are disabled for all device code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The logit weights are a fixed sequence of IEEE fp32 operations: no
    # multiply-add fusion beyond the written ones, subnormals kept.
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise FileNotFoundError("hipcc not found")


def build(out: str = OUT, extra=()) -> str:
    """Compile the sampler (always recompiles) and return the library path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + ["-I" + INC, "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-4000:])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

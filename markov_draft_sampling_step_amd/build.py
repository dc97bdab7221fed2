"""Build ``libmarkov.so`` in-tree for gfx950 with hipcc.

Flags: -ffp-contract=off so every rounding in the kernels is where the source
writes it; packed-FP32 instructions are switched off for the device code
(the host pass warns that it does not know the feature: harmless).
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "csrc", "markov.hip")
OUTPUT = os.path.join(HERE, "libmarkov.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(output: str = OUTPUT):
    return [
        HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-o", output, SOURCE,
    ]


def build(verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed")
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))

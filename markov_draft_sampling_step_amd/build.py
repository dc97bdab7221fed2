"""Build ``libmarkov.so`` in-tree for gfx950 with hipcc.

The step kernels of each (rank class, variant) pair listed in
``MARKOV_STEP_INSTANCES`` (``csrc/step_kernel.h``) are compiled from
``csrc/step_inst.hip`` as a translation unit of their own, in parallel, next
to the host side (``csrc/markov.hip``); the objects are linked into one shared
library.

Flags: -ffp-contract=off so every rounding in the kernels is where the source
writes it; packed-FP32 instructions are switched off for the device code
(the host pass warns that it does not know the feature: harmless).
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
OUTPUT = os.path.join(HERE, "libmarkov.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def instances():
    """The (rank class, variant) pairs the header lists."""
    text = open(os.path.join(CSRC, "step_kernel.h")).read()
    body = text[text.index("#define MARKOV_STEP_INSTANCES(X)"):]
    body = body[: body.index("\n\n")]
    return [(int(a), int(b)) for a, b in re.findall(r"X\((\d+),\s*(\d+)\)", body)]


def units():
    """(source, object, extra flags) of every translation unit."""
    out = [(src, os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o"), [])
           for src in sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC))
           if src.endswith(".hip") and not src.endswith("step_inst.hip")]
    for kb, var in instances():
        out.append((os.path.join(CSRC, "step_inst.hip"),
                    os.path.join(OBJDIR, f"step_kb{kb}_v{var}.o"),
                    [f"-DSTEP_KB={kb}", f"-DSTEP_VAR={var}"]))
    return out


def compile_command(src: str, obj: str, extra=()):
    return [HIPCC, *FLAGS, *extra, "-c", "-o", obj, src]


def link_command(objs, output: str = OUTPUT):
    return [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", output, *objs]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed: {' '.join(cmd)}")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    us = units()
    objs = [o for _, o, _ in us]
    jobs = jobs or max(1, min(len(us), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda u: _run(compile_command(*u), verbose), us))
    tmp = OUTPUT + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))

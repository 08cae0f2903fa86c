"""Build libmk.so in-tree: host lowering + runtime, and one object per kernel
specialisation listed in csrc/specs.def (compiled in parallel), linked together."""
from __future__ import annotations

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmk.so")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def specs():
    """(name, args) of every MK_SPEC line in specs.def."""
    out = []
    for line in open(os.path.join(CSRC, "specs.def")):
        m = re.match(r"\s*MK_SPEC\((\w+),\s*([^)]*)\)", line)
        if m:
            out.append((m.group(1), ",".join(a.strip() for a in m.group(2).split(","))))
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    steps, objs = [], []
    for src in ("lower.cpp", "schedule.cpp", "runtime.hip"):
        o = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        steps.append(["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    for name, args in specs():
        o = os.path.join(OBJ, f"kern_{name}.o")
        steps.append(["hipcc", *HIP_FLAGS, f"-DMK_SPEC_FN=ks_{name}", f"-DMK_SPEC_ARGS={args}", "-c",
                      os.path.join(CSRC, "kern_spec.hip"), "-o", o])
        objs.append(o)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    _run(["hipcc", *HIP_FLAGS, "-shared", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

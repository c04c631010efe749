"""Microbenchmarks of the gfx950 instruction mixes the kernels are built from (not part of the
layer's path).

    python -m quantized_expert_grouped_amd.microbench        # build (if stale), run, print

mmq_core.hip times MFMA throughput and the grouped matmul's per-block compute core in registers
only, which bounds what the MMQ kernels can reach before any memory or synchronisation cost.
"""
from __future__ import annotations

import os
import subprocess
import sys

from .. import build as _build

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(_build.BUILD, "mmq_core")


def build_exe() -> str:
    os.makedirs(_build.BUILD, exist_ok=True)
    flags, skip = [], False
    for f in _build.FLAGS:          # the library's flags without its include paths
        if skip or f == "-I":
            skip = not skip
            continue
        flags.append(f)
    cmd = [_build.hipcc(), *flags, "-Wno-unused-value", os.path.join(HERE, "mmq_core.hip"),
           "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for mmq_core.hip:\n{r.stderr}")
    return EXE


def main() -> int:
    src = os.path.join(HERE, "mmq_core.hip")
    fresh = os.path.exists(EXE) and os.path.getmtime(EXE) >= os.path.getmtime(src)
    exe = EXE if fresh else build_exe()
    return subprocess.run([exe]).returncode


if __name__ == "__main__":
    sys.exit(main())

"""Build libw8a8.so (the C-ABI library of gfx950 HIP kernels) in-tree.

    python -m w8a8_int8_quantized_token_amd.build

Compiles every .hip source under csrc/ with hipcc for gfx950 only and links
one shared library next to this file. The measurement probe under probe/
(the GEMM's main loop alone, for its throughput ceiling) is linked into a
library of its own, libw8a8_probe.so, which only bench.py --ceiling loads.
The flags fix the floating-point contract the kernels rely on: no
fast-math, no implicit FMA contraction, IEEE fp32 division / square root,
denormals kept, and no packed-fp32 VALU instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw8a8.so")
PROBE_DIR = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libw8a8_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fno-fast-math",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _link(srcs: list[str], includes: list[str], out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS]
    for inc in includes:
        cmd += ["-I", inc]
    cmd += [*srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _link(sorted(os.path.join(PROBE_DIR, f) for f in os.listdir(PROBE_DIR) if f.endswith(".hip")),
          [], PROBE_LIB, verbose)
    return _link(sources(), [os.path.join(ROOT, "include"), CSRC], LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))

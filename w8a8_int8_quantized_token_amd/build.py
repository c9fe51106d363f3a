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

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

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


def _run(cmd: list[str], what: str, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + what)
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)


def _link(srcs: list[str], includes: list[str], out: str, verbose: bool) -> str:
    """Compile every source to an object of its own (in parallel: each
    translation unit carries its own device code, and none calls device code
    of another), then link the shared library."""
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    inc = [a for i in includes for a in ("-I", i)]
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="w8a8_build_") as objdir:
        objs = [os.path.join(objdir, f"{i}_{os.path.basename(s)}.o") for i, s in enumerate(srcs)]
        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            futures = [pool.submit(_run, [hipcc(), *compile_flags, *inc, "-c", s, "-o", o],
                                   os.path.basename(s), verbose)
                       for s, o in zip(srcs, objs)]
            for f in futures:
                f.result()
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
             os.path.basename(out), verbose)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _link(sorted(os.path.join(PROBE_DIR, f) for f in os.listdir(PROBE_DIR) if f.endswith(".hip")),
          [], PROBE_LIB, verbose)
    return _link(sources(), [os.path.join(ROOT, "include"), CSRC], LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))

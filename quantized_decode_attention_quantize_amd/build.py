"""Build libkvq.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m quantized_decode_attention_quantize_amd.build

The library lands next to this file, where the ctypes binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_api.hip", "kvq_quantize.hip", "kvq_decode_mfma.hip", "kvq_latent.hip"]
# The benchmark's read-only HBM stream kernel: a library of its own, so
# libkvq's exports stay exactly the ABI of include/kvq.h.
BENCH_LIB = os.path.join(HERE, "libkvqbench.so")
BENCH_SOURCE = "kvq_bench_stream.hip"

# -packed-fp32-ops: keep the compiler from emitting v_pk_{add,mul,fma}_f32.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
MFMA_PARTS = 5  # kvq_decode_mfma.hip is compiled once per part (-DKVQ_MFMA_PART=i)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libkvq needs ROCm's hipcc to build")


def _units():
    """(source, extra flags, object name) of every compilation unit."""
    units = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        stem = src.rsplit(".", 1)[0]
        if src == "kvq_decode_mfma.hip":
            units += [(path, [f"-DKVQ_MFMA_PART={i}"], f"{stem}_{i}.o") for i in range(MFMA_PARTS)]
        else:
            units.append((path, [], f"{stem}.o"))
    return units


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every unit to an object (in parallel) and link libkvq.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(unit):
        src, extra, obj = unit
        out = os.path.join(objdir, obj)
        cmd = [hipcc(), *HIP_FLAGS, *extra, *inc, "-c", src, "-o", out]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return out, res

    units = _units()
    jobs = jobs or min(len(units), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, units))
    for out, res in results:
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"libkvq build failed compiling {os.path.basename(out)}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("libkvq link failed")
    os.replace(tmp, LIB)
    tmp = BENCH_LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", os.path.join(CSRC, BENCH_SOURCE), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("libkvqbench build failed")
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds the gfx950 library in-tree: layer_wise_mixed_kvq_amd/libkvq.so (hipcc).

`python -m layer_wise_mixed_kvq_amd.build --phase-timers` builds the profiling variant
libkvq_phases.so instead: the same sources with KVQ_PHASE_TIMERS, whose decode kernel
records per-wave phase timestamps (layer_wise_mixed_kvq_amd/profiling.py phases).  Nothing
but that profiling command loads it."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")
# (source, extra flags): the decode kernels build in one translation unit per key bit width
UNITS = [("kvq_api.hip", []), ("kvq_debug.hip", []), ("kvq_quant.hip", []), ("kvq_dequant.hip", []), ("kvq_decode.hip", ["-DKVQ_DECODE_COMMON"]),
         ("kvq_decode.hip", ["-DKVQ_DECODE_KB=2"]), ("kvq_decode.hip", ["-DKVQ_DECODE_KB=4"]),
         ("kvq_decode.hip", ["-DKVQ_DECODE_KB=8"]), ("kvq_decode.hip", ["-DKVQ_DECODE_KB=16"])]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the decode kernel rescales them with VALU ops,
    # and the AGPR form would copy them across the register files around every MFMA
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # leading scalar kernel arguments (the decode kernel's prologue fields) preloaded into
    # scalar registers by the dispatch
    "-mllvm", "-amdgpu-kernarg-preload-count=10",
    "-Wall", "-Wno-unused-function",
]


def _compile(unit, obj, verbose, defines=()):
    src, extra = unit
    cmd = ["hipcc", *HIPCC_FLAGS, "-c", *defines, *extra, "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src} {' '.join(extra)}")
    if verbose:
        sys.stderr.write(res.stderr)
    return obj


PHASES_LIB = os.path.join(PKG, "libkvq_phases.so")


def build(verbose: bool = False, phase_timers: bool = False) -> str:
    """Compile every unit for gfx950 (in parallel) and link libkvq.so in-tree (with
    phase_timers: the profiling variant libkvq_phases.so)."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build_phases" if phase_timers else "_build")
    lib = PHASES_LIB if phase_timers else LIB
    defines = ["-DKVQ_PHASE_TIMERS"] if phase_timers else []
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, f"unit{i}.o") for i in range(len(UNITS))]
    workers = max(1, min(len(UNITS), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda a: _compile(*a, verbose, defines), [(u, o) for u, o in zip(UNITS, objs)]))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libkvq.so failed")
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, phase_timers="--phase-timers" in sys.argv[1:]))

"""Build libmoe_fp4.so (HIP, gfx950) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_fp4.so")
MEASURE_LIB = os.path.join(HERE, "libmoe_fp4_measure.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "route.hip", "router.hip", "decode.hip", "prefill.hip", "prefill_lds.hip", "mx8.hip", "shared.hip", "stack.hip"]

# Packed fp32 VALU ops are switched off for all device code (the host pass warns
# that it does not know the feature; that is harmless).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the sources build without warnings; the host pass's note that it does not
    # know the packed-fp32 feature is expected
    warn = [l for l in r.stderr.splitlines() if "warning" in l and "packed-fp32-ops" not in l]
    if warn:
        raise RuntimeError(f"compiler warnings: {' '.join(cmd)}\n" + "\n".join(warn))
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for cmd, r in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # the measurement companion (a plain streaming read), loaded by the benchmark only
    tmp = MEASURE_LIB + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "measure.hip")])
    os.replace(tmp, MEASURE_LIB)
    if verbose:
        print("built", LIB, "and", MEASURE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)

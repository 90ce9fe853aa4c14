"""Build the accumulation probe library of tests/test_gpu_accum.py (gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libaccum_probe.so")


def build(verbose: bool = False) -> str:
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", SO, os.path.join(HERE, "accum_probe.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(" ".join(cmd))
    return SO


if __name__ == "__main__":
    build(verbose=True)

"""Build libsscan.so in-tree with hipcc for gfx950 (no JIT, no torch extension)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsscan.so")
SOURCES = [os.path.join(CSRC, f) for f in ("sscan_api.hip", "sscan_kernels.hip", "sscan_bwd.hip", "sscan_ssd.hip")]
ARCH = "gfx950"

# Packed-FP32 VALU forms are kept out of the generated code; the host pass warns
# that it does not know the target feature, which is harmless.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *(extra or []), "-o", tmp, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libsscan.so in-tree with hipcc for gfx950 (no JIT, no torch extension).

Each translation unit is compiled to an object in a temporary directory, in
parallel, and the objects are linked into the shared library."""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsscan.so")
# debug build: every kernel fills its LDS with NaN before use (tests/test_gpu_debug.py)
POISON_LIB = os.path.join(HERE, "libsscan_poison.so")
SOURCES = [os.path.join(CSRC, f) for f in ("sscan_api.hip", "sscan_kernels.hip", "sscan_bwd.hip", "sscan_ssd.hip")]
ARCH = "gfx950"

# Packed-FP32 VALU forms are kept out of the generated code; the host pass warns
# that it does not know the target feature, which is harmless.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd: list[str]) -> str:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="sscan_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[hipcc(), *FLAGS, *(extra or []), "-c", "-o", obj, src] for src, obj in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=len(cmds)) as pool:
            logs = list(pool.map(_run, cmds))
        tmp = out + ".tmp"
        logs.append(_run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]))
    if verbose:
        print("\n".join(logs))
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    """The library and its LDS-poison debug build, both compiled from the same sources."""
    return [build(LIB, verbose=verbose), build(POISON_LIB, ["-DSSCAN_LDS_POISON=1"], verbose=verbose)]


if __name__ == "__main__":
    print(build_all(verbose=True))

"""Build libbitmm.so for gfx950 with hipcc, in-tree.

Every translation unit under ``csrc/`` is compiled in parallel into ``_build/`` and
linked into ``bit_matmul_amd/libbitmm.so``. The benchmark's measurement kernels
(``probe/probe.hip``: a streaming read and a matrix-core loop, not part of the library)
are linked into ``bit_matmul_amd/libbitmm_probe.so``. Run ``python -m bit_matmul_amd.build``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitmm.so")
PROBE_SRC = os.path.join(HERE, "probe", "probe.hip")
PROBE_LIB = os.path.join(HERE, "libbitmm_probe.so")
ARCH = "gfx950"

# Packed-FP32 VALU instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libbitmm)")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs) + 1, max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        probe_obj = ex.submit(_compile, PROBE_SRC)
        objs = list(ex.map(_compile, srcs))
        probe_obj = probe_obj.result()
    _link(objs, LIB)
    _link([probe_obj], PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources, and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

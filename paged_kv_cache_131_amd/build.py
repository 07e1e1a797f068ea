"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_131_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("pa_kernels.hip", "pa_prefill.hip", "pa_api.cpp")]
LIBRARY = os.path.join(HERE, "libpagedattn.so")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms stay off; hipcc's host pass warns that it does not
    # know the feature, which is harmless
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build_library(verbose: bool = False) -> str:
    tmp = LIBRARY + f".tmp{os.getpid()}"
    cmd = [hipcc(), *FLAGS, f"-I{os.path.join(ROOT, 'include')}", "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    log = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{log}")
    os.replace(tmp, LIBRARY)
    if verbose and log.strip():
        print(log, file=sys.stderr)
    return LIBRARY


if __name__ == "__main__":
    print(build_library(verbose=True))

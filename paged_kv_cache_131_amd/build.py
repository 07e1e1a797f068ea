"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_131_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# (source, extra flags). The prompt-phase kernel keeps its MFMA accumulators
# in ordinary VGPRs: its online-softmax rescale works on them between MFMAs,
# and the default accumulator registers would be copied out and back each step.
# Its direct-to-LDS loads name M0 as clobbered, which the compiler reports as a
# reserved register (nothing it generates there uses M0).
SOURCES = [
    (os.path.join(HERE, "csrc", "pa_kernels.hip"), []),
    (os.path.join(HERE, "csrc", "pa_prefill.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form", "-Wno-inline-asm"]),
    (os.path.join(HERE, "csrc", "pa_api.cpp"), []),
]
LIBRARY = os.path.join(HERE, "libpagedattn.so")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _run(cmd) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    log = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{log}")
    return log


def build_library(verbose: bool = False) -> str:
    """Compile each source to an object (in parallel), then link the shared
    library next to this file."""
    from concurrent.futures import ThreadPoolExecutor

    tmpdir = tempfile.mkdtemp(prefix="pa_build_")
    tmp = LIBRARY + f".tmp{os.getpid()}"
    try:
        inc = f"-I{os.path.join(ROOT, 'include')}"
        jobs = []
        for src, extra in SOURCES:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            jobs.append((obj, [hipcc(), *FLAGS, *extra, inc, "-c", "-o", obj, src]))
        with ThreadPoolExecutor(len(jobs)) as pool:
            logs = list(pool.map(lambda j: _run(j[1]), jobs))
        logs.append(_run([hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp, *(o for o, _ in jobs)]))
        os.replace(tmp, LIBRARY)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
        if os.path.exists(tmp):
            os.remove(tmp)
    log = "\n".join(x for x in logs if x.strip())
    if verbose and log:
        print(log, file=sys.stderr)
    return LIBRARY


if __name__ == "__main__":
    print(build_library(verbose=True))

"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_131_amd.build
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# (source, extra flags). The prompt-phase kernel keeps its MFMA accumulators
# in ordinary VGPRs: its online-softmax rescale works on them between MFMAs,
# and the default accumulator registers would be copied out and back each step.
# Its direct-to-LDS loads are inline assembly that sets M0, a register the
# compiler reserves and may not preserve across the statement (it warns;
# -Wno-inline-asm silences that). check_m0() verifies on every build that no
# instruction of that file's device code other than these loads and their
# own M0 setting reads or writes M0.
PREFILL_SOURCE = os.path.join(HERE, "csrc", "pa_prefill.hip")
SOURCES = [
    (os.path.join(HERE, "csrc", "pa_kernels.hip"), []),
    (PREFILL_SOURCE, ["-mllvm", "-amdgpu-mfma-vgpr-form", "-Wno-inline-asm"]),
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


LLVM_BIN = "/opt/rocm/llvm/bin"
# instructions that read or write M0 without naming it
IMPLICIT_M0 = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|s_ttracedata|ds_gws|ds_ordered_count|ds_append|ds_consume|"
                         r"ds_read_addtid|ds_write_addtid|v_interp|s_setreg|\w+_lds_|\w+_lds$|buffer_\w+ .*\blds\b)")


def m0_violations(disassembly: str) -> list:
    """Instructions of a gfx950 disassembly that touch M0 other than the
    pairs `s_mov_b32 m0, sN` + `global_load_lds_dwordx4` of the prompt-phase
    kernel's direct-to-LDS loads."""
    insts = []
    for line in disassembly.splitlines():
        text = line.split("//")[0].strip()
        if not text or text.endswith(":") or text.startswith(("Disassembly", "<")) or "file format" in text:
            continue
        insts.append(text)
    bad = []
    for i, text in enumerate(insts):
        mnem = text.split()[0]
        names_m0 = re.search(r"\bm0\b", text) is not None
        if names_m0:
            ok = (re.fullmatch(r"s_mov_b32 m0, s\d+", text) is not None and i + 1 < len(insts)
                  and insts[i + 1].split()[0] == "global_load_lds_dwordx4")
            if not ok:
                bad.append(text)
        elif IMPLICIT_M0.match(text):
            ok = mnem == "global_load_lds_dwordx4" and i > 0 and re.fullmatch(r"s_mov_b32 m0, s\d+", insts[i - 1])
            if not ok:
                bad.append(text)
    return bad


def check_m0(obj: str, tmpdir: str) -> int:
    """Disassemble the gfx950 code object inside `obj` (the prompt-phase
    kernel just compiled) and raise if any instruction besides the inline
    assembly's own M0 setting and direct-to-LDS loads touches M0. Returns
    the number of direct-to-LDS loads seen."""
    fatbin = os.path.join(tmpdir, "prefill.fatbin")
    code = os.path.join(tmpdir, "prefill.co")
    _run([os.path.join(LLVM_BIN, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}", obj,
          os.path.join(tmpdir, "discard.o")])
    _run([os.path.join(LLVM_BIN, "clang-offload-bundler"), "--type=o", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}",
          f"--input={fatbin}", f"--output={code}", "--unbundle"])
    res = subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "-d", f"--mcpu={ARCH}", code],
                         capture_output=True, text=True, check=True)
    loads = res.stdout.count("global_load_lds_dwordx4")
    bad = m0_violations(res.stdout)
    if bad or loads == 0:
        raise RuntimeError("pa_prefill.hip: compiler-generated code touches M0, which the direct-to-LDS inline "
                           f"assembly clobbers ({len(bad)} instructions, e.g. {bad[:3]}; {loads} loads)")
    return loads


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
        check_m0(jobs[[src for src, _ in SOURCES].index(PREFILL_SOURCE)][0], tmpdir)
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

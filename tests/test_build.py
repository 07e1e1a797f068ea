"""The build's M0 check: the prompt-phase kernel's direct-to-LDS loads are
inline assembly that sets M0, which the compiler reserves; the build fails
if any other instruction of that file's device code touches M0. CPU only."""

import os

import pytest

from paged_kv_cache_131_amd import build


def test_accepts_the_load_pairs():
    text = "\ts_mov_b32 m0, s3\n\tglobal_load_lds_dwordx4 v1, off\n\tv_add_f32 v0, v1, v2\n"
    assert build.m0_violations(text) == []


@pytest.mark.parametrize("planted", [
    "\ts_movrels_b32 s0, s1\n",                       # implicit M0 read
    "\tv_readlane_b32 s2, v0, m0\n",                  # explicit M0 operand
    "\ts_mov_b32 m0, s4\n\tv_add_f32 v0, v1, v2\n",   # M0 set for something else
    "\tglobal_load_lds_dwordx4 v1, off\n",            # a direct-to-LDS load not right after its M0
    "\tds_read_addtid_b32 v0\n",
])
def test_flags_other_uses(planted):
    text = "\ts_mov_b32 m0, s3\n\tglobal_load_lds_dwordx4 v1, off\n" + planted
    assert build.m0_violations(text)


def test_current_build_passes():
    # runs the real check on a fresh compile of the prompt-phase source
    import subprocess
    import tempfile

    with tempfile.TemporaryDirectory() as d:
        obj = os.path.join(d, "pf.o")
        flags = dict(build.SOURCES)[build.PREFILL_SOURCE]
        inc = f"-I{os.path.join(build.ROOT, 'include')}"
        subprocess.run([build.hipcc(), *build.FLAGS, *flags, inc, "-c", "-o", obj, build.PREFILL_SOURCE],
                       check=True, capture_output=True)
        assert build.check_m0(obj, d) > 0

"""Builds tests/host_checks.hip with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code (the device code is built as usual) and runs it without a GPU:
workspace layouts (regions aligned, disjoint, inside the total; every index
range the kernels reach fits its region; the dHidden split rule against its
slab bound for every completion count), and host-side refusal of bad
arguments by every entry point."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "preference_alignment_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.slow
def test_host_checks_under_sanitizers(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_checks")
    # sanitizers on the host side only; each -fsanitize= follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(ROOT, "tests", "host_checks.hip"), os.path.join(CSRC, "kernels_head.hip"),
                os.path.join(CSRC, "kernels_stream.hip")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([cc, *flags, *san, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    r = subprocess.run([cc, "--offload-arch=gfx950", *san, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout

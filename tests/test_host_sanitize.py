"""The C ABI's host code under the address and undefined-behaviour sanitizers (CPU only).

capi.cpp (argument validation, workspace layout, launch planning) is built with
g++ and -fsanitize=address,undefined against a minimal stand-in for the HIP
runtime header and fake kernel launchers (tests/host_check/).  The launchers
check each launch plan against its shape instead of launching.  A driver then
calls every entry point with valid, invalid and random arguments, using host
arrays of exactly the length the arguments imply.  Any out-of-bounds access,
overflow or failed check ends the run with a non-zero status.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CHECK = os.path.join(HERE, "host_check")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")


def _build(tmp_path, sources, out, includes=()):
    exe = str(tmp_path / out)
    cmd = ["g++", "-std=c++17", "-O1", "-g", *SAN, *[f"-I{i}" for i in includes], *sources, "-o", exe]
    proc = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stderr[-3000:]
    return exe


def test_sanitizers_are_active(tmp_path):
    """The toolchain's sanitizer runtime reports a planted heap overflow (so a
    clean run of the driver below means something)."""
    src = tmp_path / "planted.cpp"
    src.write_text("#include <vector>\nint main(int c, char **) { std::vector<int> v(4); return v.data()[3 + c]; }\n")
    exe = _build(tmp_path, [str(src)], "planted")
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert proc.returncode != 0 and "AddressSanitizer" in proc.stderr


def test_capi_host_code_under_sanitizers(tmp_path):
    sources = [os.path.join(ROOT, "lossless_draft_verification_verify_amd", "csrc", "capi.cpp"),
               os.path.join(CHECK, "fakes.cpp"), os.path.join(CHECK, "driver.cpp")]
    includes = [os.path.join(CHECK, "fake_hip"), os.path.join(ROOT, "include"),
                os.path.join(ROOT, "lossless_draft_verification_verify_amd", "csrc")]
    exe = _build(tmp_path, sources, "host_check", includes)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert proc.returncode == 0, (proc.stdout[-2000:], proc.stderr[-4000:])
    assert "0 failures" in proc.stdout, proc.stdout

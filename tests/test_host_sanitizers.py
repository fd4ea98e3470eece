"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library sources are compiled with both sanitizers on the host pass only
(the checks are about argument validation, layout arithmetic and the error
paths, which run on the CPU; the device code is built as usual, at -O1, and
never launched without a GPU), and linked with
tests/sanitize/validate_abi.cpp, which calls every entry point with failing,
extreme and (without a GPU) valid arguments.  Any sanitizer report aborts the
program; the test asserts a clean exit and the driver's own expectations.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_sequence_length_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "validate_abi.cpp")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not on PATH")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    objs = []
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [DRIVER]
    procs = []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = ["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, *lang, "-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for src, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"{src}:\n{out[-4000:]}"
    exe = str(tmp_path / "validate_abi")
    r = subprocess.run(["hipcc", "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " 0 failures" in r.stdout, r.stdout

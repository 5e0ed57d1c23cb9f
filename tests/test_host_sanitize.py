"""The descriptor's host code and the fp64 reference under the address and
undefined-behaviour sanitizers, on the CPU: tests/host_tree_check.cpp checks
tree validation, subtree ends, logical positions and visible-pair counts
against brute force on random preorder trees and windows, the rejection
codes of malformed trees, large trees, and calls the reference's attention,
backward, merge and sink functions; built here with g++/gcc (host code only)
with -fsanitize=address,undefined and run; any sanitizer report fails it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def test_host_code_under_sanitizers(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if not gxx or not gcc:
        pytest.skip("no host compiler")
    obj = str(tmp_path / "oracle.o")
    exe = str(tmp_path / "host_tree_check")
    subprocess.check_call([gcc, "-std=c99", "-c", os.path.join(ROOT, "oracle", "cpattn_oracle.c"), "-o", obj] + SAN)
    subprocess.check_call([gxx, "-std=c++17", os.path.join(ROOT, "tests", "host_tree_check.cpp"), obj, "-o", exe,
                           "-I" + os.path.join(ROOT, "include"), "-lm"] + SAN)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout)
    assert r.returncode == 0 and "host checks passed" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr

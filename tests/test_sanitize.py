"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two standalone drivers, each built with gcc/g++ -fsanitize=address,undefined
and run to completion: tests/sanitize/oracle_driver.c over the CPU oracle
(oracle/tms_oracle.c) and tests/sanitize/trie_build_driver.cpp over the
library's host-side catalog compiler (trie_masked_sparse_amd/csrc/
trie_build.cpp).  They are built separately: the oracle and the library
share no code.  Any out-of-bounds access, leak or undefined operation makes
the test program exit non-zero with the sanitizer's report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def _run(tmp_path, compiler, std, srcs, extra=()):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / "driver")
    subprocess.run([compiler, *SAN, f"-std={std}", *extra, *srcs, "-o", exe, *(["-lm"] if compiler == "gcc" else [])],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    return int(r.stdout.split()[1])


def test_oracle_under_sanitizers(tmp_path):
    n = _run(tmp_path, "gcc", "c11", [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                                      os.path.join(ROOT, "oracle", "tms_oracle.c")])
    assert n > 300


def test_host_trie_builder_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "trie_masked_sparse_amd", "csrc")
    n = _run(tmp_path, "g++", "c++17", [os.path.join(ROOT, "tests", "sanitize", "trie_build_driver.cpp"),
                                        os.path.join(csrc, "trie_build.cpp")], extra=[f"-I{csrc}"])
    assert n > 1000

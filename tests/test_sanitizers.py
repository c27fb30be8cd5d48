"""The C and C++ host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The oracle's C library and librescomp's host code (plan creation, validation,
layout arithmetic, argument checks) are rebuilt with both sanitizers, and the
CPU tests that drive them run again in a child process with the sanitizer
runtime preloaded. Any report (an out-of-bounds access, a use after free, an
overflowing shift, a value outside an enumeration ...) aborts that process.
"""
import os
import subprocess
import sys

import pytest

import oracle
from activation_residual_compression_amd import sanitize

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = ["tests/test_oracle_quant.py", "tests/test_oracle_nm_lr.py", "tests/test_oracle_ef.py",
                "tests/test_oracle_bs.py", "tests/test_oracle_layout.py", "tests/test_oracle_schedule.py"]


def _gcc_runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()


def _run_child(tests, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", "--capture=no"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = oracle.build(force=True, sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (os.path.isabs(asan) and os.path.isabs(ubsan)):
        pytest.skip("gcc sanitizer runtimes not installed")
    out = _run_child(ORACLE_TESTS, {"LD_PRELOAD": asan + ":" + ubsan, "ORACLE_LIB": lib})
    assert " passed" in out


def test_host_code_under_asan_and_ubsan(tmp_path):
    lib = sanitize.build(str(tmp_path / "san"))
    out = _run_child(["tests/test_abi.py"], {"LD_PRELOAD": sanitize.runtime(), "LIBRESCOMP_LIB": lib})
    assert " passed" in out

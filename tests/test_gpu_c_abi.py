"""The C ABI from a plain C program (tests/c_abi_roundtrip.c, built by
__graft_entry__.build()): every scheme, two steps, receiver bit-identical to the
sender, e plus the update of ahat equal to the residual, bad pointers rejected."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import __graft_entry__  # noqa: E402


def test_c_caller_round_trip():
    exe = __graft_entry__.C_ABI_TEST_BIN
    assert os.path.exists(exe), "%s is not built; run __graft_entry__.build()" % exe
    print("[gpu] c abi round trip", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_abi_roundtrip: all ok" in r.stdout
    for scheme in ("q1", "q2", "nm", "lowrank", "blocksel"):
        assert "%s: ok" % scheme in r.stdout

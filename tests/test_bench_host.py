"""Host logic of bench.py: when a committed profile still describes a kernel.

A profile records the hashes of the kernel sources it was taken with. The
roofline traffic and the contraction times may be read from it only while the
sources of that kernel (its own file plus the shared headers and the host
driver) are unchanged; a change to another kernel's file does not void it.
"""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_profile_freshness_is_per_kernel_source(tmp_path, monkeypatch):
    bench = _bench()
    from activation_residual_compression_amd.profsummary import source_hashes
    now = source_hashes()
    assert {"quant.hip", "lowrank.hip", "plan.cpp", "device_common.hpp"} <= set(now)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))

    def write(sources):
        (tmp_path / "p.json").write_text(json.dumps({"kernels": {}, "sources": sources}))

    q = "q_compress_kernel<unsigned short, 128, 2,"
    write(dict(now))
    assert bench._fresh_profile("p.json") is not None
    assert bench._fresh_profile("p.json", q) is not None
    assert bench._fresh_profile("p.json", "lr_") is not None

    write(dict(now, **{"lowrank.hip": "0" * 64}))           # another kernel's file changed
    assert bench._fresh_profile("p.json") is None
    assert bench._fresh_profile("p.json", q) is not None
    assert bench._fresh_profile("p.json", "lr_") is None

    write(dict(now, **{"plan.cpp": "0" * 64}))              # the host driver changed
    assert bench._fresh_profile("p.json", q) is None
    assert bench._fresh_profile("p.json", "lr_") is None

    write(dict(now, **{"quant.hip": "0" * 64}))
    assert bench._fresh_profile("p.json", q) is None
    assert bench._fresh_profile("p.json", "nm_compress_kernel<unsigned short,") is not None
    assert bench._fresh_profile("p.json", "unknown_kernel") is None
    assert bench._fresh_profile("missing.json", q) is None


def test_more_than_one_gpu_is_refused_before_touching_a_gpu():
    """The path has no inter-GPU step: --gpus N > 1 (or a launcher's
    WORLD_SIZE > 1) ends with exit status 2 and a message, before any GPU or
    library call."""
    import subprocess
    import sys
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                           text=True, timeout=120, env=dict(os.environ, **env))
        assert r.returncode == 2, (args, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr and r.stdout == ""

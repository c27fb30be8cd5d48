"""Build librescomp.so (HIP, gfx950) in place.

The kernels are compiled with contraction off (every fp32 operation rounds
once, fused multiply-adds are written explicitly), fp32 denormals kept, and
packed-fp32 instruction selection disabled. The compiler's per-kernel resource
report (registers, LDS, occupancy, scratch) is kept in lib/kernel_resources.json,
and a kernel that spills to scratch memory fails the build: every kernel here is
written to fit in registers, and a spill has turned a 350 us kernel into a
1900 us one.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "lib", "librescomp.so")
RESOURCES = os.path.join(HERE, "lib", "kernel_resources.json")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["quant.hip", "nm.hip", "lowrank.hip", "blocksel.hip", "checks.hip", "noalloc.hip", "probe.hip", "plan.cpp"]
ARCH = os.environ.get("RC_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE,
]
REPORT = ["-Rpass-analysis=kernel-resource-usage"]
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
           "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds_bytes",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill"}


def parse_resource_report(text: str) -> dict:
    """{kernel symbol: {field: int}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass-analysis", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = out.setdefault(body.split(":", 1)[1].strip(), {})
        elif cur is not None and ":" in body:
            key, val = body.rsplit(":", 1)
            key = key.strip()
            if key in _FIELDS:
                try:
                    cur[_FIELDS[key]] = int(val.strip())
                except ValueError:
                    pass
    return out


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *FLAGS, *REPORT, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-xhip")
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj, parse_resource_report(r.stderr)

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        results = list(ex.map(compile_one, SOURCES))
    objs = [o for o, _ in results]
    kernels = {}
    for _, rep in results:
        kernels.update(rep)
    import json
    with open(RESOURCES, "w") as f:
        json.dump({"arch": ARCH, "kernels": kernels}, f, indent=1, sort_keys=True)
    spills = {k: v for k, v in kernels.items() if v.get("scratch_bytes", 0) or v.get("vgpr_spill", 0)}
    if spills:
        raise RuntimeError("kernels spill to scratch memory: %s" % ", ".join(
            "%s (%d B/lane)" % (k, v.get("scratch_bytes", 0)) for k, v in sorted(spills.items())))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

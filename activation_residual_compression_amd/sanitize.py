"""CPU sanitizer build of librescomp's host code.

The plan, validation, layout and dispatch code is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (the
device code is built as usual and never runs on the CPU) into a library of its
own. Loading it needs the sanitizer runtime preloaded; the CPU tests do that in
a child process, with LIBRESCOMP_LIB naming the library (test_sanitizers.py).
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from activation_residual_compression_amd import build as B

HOST_SAN = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=all".split()
FLAGS = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"] + HOST_SAN


def runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (it carries the UB checks too)."""
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(B._hipcc())), "lib", "llvm",
                                         "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found next to hipcc")
    return hits[-1]


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    hipcc = B._hipcc()

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *FLAGS, "-I", B.CSRC, "-c", os.path.join(B.CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-xhip")
        subprocess.run(cmd, check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(one, B.SOURCES))
    out = os.path.join(out_dir, "librescomp.so")
    subprocess.run([hipcc, "--offload-arch=" + B.ARCH, "-shared", "-fPIC", "-shared-libsan", *HOST_SAN,
                    *objs, "-o", out], check=True, capture_output=True)
    return out

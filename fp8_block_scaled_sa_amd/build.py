"""Builds libdg_fp8.so (the gfx950 HIP library behind include/dg_fp8.h) in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "dg_fp8.hip")]
DEPS = SOURCES + [os.path.join(HERE, "csrc", "kernels.hpp"), os.path.join(HERE, "csrc", "quant.hpp"),
        os.path.join(HERE, "csrc", "moe.hpp"),
        os.path.join(ROOT, "include", "dg_fp8.h")]
LIBRARY = os.path.join(HERE, "libdg_fp8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def build(output: str = LIBRARY, extra_flags=()) -> str:
    """Compile every source into one shared library (always recompiles)."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra_flags, *SOURCES, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, output)
    return output


def is_stale(output: str = LIBRARY) -> bool:
    if not os.path.exists(output):
        return True
    t = os.path.getmtime(output)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build())

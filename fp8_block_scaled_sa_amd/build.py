"""Builds libdg_fp8.so (the gfx950 HIP library behind include/dg_fp8.h) in-tree,
and the same sources at -O1 -g as libdg_fp8_O1.so: a build with a different
instruction schedule and register allocation, which the tests compare with
the release build bit for bit (a race or a missing wait shows up as a
difference between the two)."""
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
DEBUG_LIBRARY = os.path.join(HERE, "libdg_fp8_O1.so")
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


def build_debug(output: str = DEBUG_LIBRARY) -> str:
    """The same library at -O1 with debug information (-O0 cannot place the
    inline-asm LDS-DMA operands in scalar registers)."""
    tmp = output + ".tmp%d" % os.getpid()
    flags = ["-O1", "-g"] + [f for f in FLAGS if f != "-O3"]
    subprocess.check_call([HIPCC, *flags, *SOURCES, "-o", tmp])
    os.replace(tmp, output)
    return output


def is_stale(output: str = LIBRARY) -> bool:
    if not os.path.exists(output):
        return True
    t = os.path.getmtime(output)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build())
    print(build_debug())

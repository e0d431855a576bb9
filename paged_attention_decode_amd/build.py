"""Ahead-of-time build of libpaged_decode.so for gfx950 with hipcc.

    python -m paged_attention_decode_amd.build

Compiles the HIP kernels and the host library in-tree (next to this file), so
the built library travels with the source tree.  Packed-fp32 instructions are
disabled for device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libpaged_decode.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("PD_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pd_host.cpp", "pd_cascade_host.cpp", "pd_partial.hip", "pd_merge.hip", "pd_cascade.hip",
           "pd_sparse.hip", "pd_mla.hip", "pd_probe.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + INCLUDE, "-I" + CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-fgpu-flush-denormals-to-zero",
          "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str, build_dir: str, extra_flags) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc()] + COMMON + list(extra_flags) + DEVICE + ["-c", path, "-o", obj]
    else:
        cmd = [hipcc()] + COMMON + list(extra_flags) + ["-x", "c++", "-c", path, "-o", obj]
    subprocess.check_call(cmd)
    return obj


def build(verbose: bool = False, out: str = OUT, extra_flags=(), build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link the shared library at `out`
    (`extra_flags` are added to each compile, e.g. -D tuning knobs)."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra_flags), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp]
                          + objs)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def dump_isa(src: str = "pd_partial.hip", out_dir: str = BUILD_DIR) -> str:
    """Write the gfx950 assembly of one source (for inspecting register use)."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, src + ".s")
    cmd = [hipcc()] + COMMON + DEVICE + ["--cuda-device-only", "-S", os.path.join(CSRC, src),
                                         "-o", out]
    subprocess.check_call(cmd)
    return out


if __name__ == "__main__":
    build(verbose=True)
    if len(sys.argv) > 1 and sys.argv[1] == "--isa":
        print(dump_isa())

"""Build the gfx950 HIP library (libmoe_gfx950.so) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_gfx950.so")
SOURCES = ["moe_api.hip", "route.hip", "dispatch.hip", "grouped_gemm.hip", "stream_gemm.hip", "mfma_gemm.hip", "combine.hip", "pack.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
    # no packed-fp32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wl,-z,defs",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source to an object in parallel, then link the library."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    compile_flags = [f for f in FLAGS if f not in ("-shared", "-Wl,-z,defs")]
    tmpdir = tempfile.mkdtemp(prefix="moe_build_")
    objs = []

    def one(src):
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *compile_flags, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    os.rmdir(tmpdir)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

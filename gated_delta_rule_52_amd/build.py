"""Build libkda.so (HIP kernels + C ABI) for gfx950 with hipcc.

Run as ``python -m gated_delta_rule_52_amd.build``.  The library is built in
the package directory so that it travels with the source tree.  Each source
compiles to its own object in parallel (every kernel file is self-contained:
no device code crosses files), then hipcc links them.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_recurrent.hip", "kda_chunk.hip", "kda_segments.hip", "kda_prep.hip",
           "kda_scan.hip", "kda_backward.hip", "kda_dplr.hip", "kda_dplr_chunk.hip", "kda_noalloc.hip",
           "kda_chunk_bwd.hip"]
# measured ceilings (streaming copy, matrix-core loop) for the benchmark's roofline figures: a library of
# their own, outside the operator's ABI
CEIL_LIB = os.path.join(HERE, "libkda_ceilings.so")
CEIL_SOURCES = ["kda_ceilings.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: without it the register allocator keeps them in AGPRs
    # and copies them back and forth around loops (a bf16 MFMA loop ran at half rate)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if p and (os.path.sep not in p or os.path.exists(p)):
            return p
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source into libkda.so and libkda_ceilings.so (always
    recompiles); returns the path of libkda.so."""
    jobs = jobs or min(len(SOURCES) + len(CEIL_SOURCES), os.cpu_count() or 1, 16)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
            return src, obj, r.returncode, r.stdout

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_one, SOURCES + CEIL_SOURCES))
        failed = False
        for src, _, rc, out in results:
            # hipcc's host pass does not know the packed-fp32 feature and says so: harmless
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or rc != 0):
                print(f"--- {src}\n" + "\n".join(lines), flush=True)
            failed |= rc != 0
        if failed:
            raise subprocess.CalledProcessError(1, "hipcc -c")
        objs = {src: o for src, o, _, _ in results}
        for lib, srcs in ((LIB, SOURCES), (CEIL_LIB, CEIL_SOURCES)):
            tmp = lib + ".tmp"
            cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[objs[s] for s in srcs]]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

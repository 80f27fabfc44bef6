"""Build libdcpmerge.so (and its measurement twin libdcpmerge_bench.so) for
gfx950 with hipcc (cross-compiles without a GPU).

    python -m lse_weighted_merge_dcp_amd.csrc.build

Objects go to csrc/_build/; the shared libraries land next to the Python
binding (lse_weighted_merge_dcp_amd/), where the binding loads them.

libdcpmerge.so exports exactly the calls of include/dcpmerge.h.
libdcpmerge_bench.so links the same kernel objects behind the dcpb_* calls of
csrc/dcpmerge_bench.h (timing events on the kernels' own dispatches) and
exports nothing else; only measurement code loads it.  A linker version
script fixes each library's exported names.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
SOURCES = ["api.cpp", "pack.hip", "combine.hip", "inplace.hip", "bench_api.cpp"]
LIB = os.path.join(PKG, "libdcpmerge.so")
BENCH_LIB = os.path.join(PKG, "libdcpmerge_bench.so")
# exported names of each library (everything else is local)
EXPORTS = {
    LIB: ["dcp_lse_pack_dim", "dcp_status_str", "dcp_pack", "dcp_unpack_combine", "dcp_lse_combine_inplace"],
    BENCH_LIB: ["dcpb_pack", "dcpb_unpack_combine", "dcpb_lse_combine_inplace", "dcpb_empty_kernel"],
}
OBJECTS = {
    LIB: ["api", "pack", "combine", "inplace"],
    BENCH_LIB: ["bench_api", "api", "pack", "combine", "inplace"],
}
ARCH = "gfx950"

# Packed fp32 instructions are switched off for every HIP source; the host
# pass warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["-O3", "-std=c++20", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wextra", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libdcpmerge needs ROCm's hipcc to build")


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(HERE, src), "-o", obj] + HIP_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)


def _link(lib: str, bdir: str, verbose: bool) -> None:
    script = os.path.join(bdir, os.path.basename(lib) + ".map")
    with open(script, "w") as f:
        f.write("{\n  global:\n%s  local: *;\n};\n" % "".join("    %s;\n" % n for n in EXPORTS[lib]))
    objs = [os.path.join(bdir, o + ".o") for o in OBJECTS[lib]]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-Wl,--version-script=" + script,
           "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libdcpmerge.so and
    libdcpmerge_bench.so (always rebuilds).  Returns libdcpmerge.so's path."""
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(5, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(SOURCES, objs)))
    for lib in (LIB, BENCH_LIB):
        _link(lib, bdir, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

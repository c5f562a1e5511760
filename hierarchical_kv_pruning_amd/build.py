"""Build libatlaskv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree next to this file so that it travels with the
source tree.  `python -m hierarchical_kv_pruning_amd.build` rebuilds it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libatlaskv.so")
SOURCES = ["atlaskv_api.hip", "hikvp_select.hip", "hikvp_seq.hip", "hikvp_tree.hip", "hikvp_flat.hip", "hikvp_shared.hip", "hikvp_folded.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off: only scalar/vector fp32 forms are used
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """Compile every source into one shared library at `out` (extra_flags:
    e.g. host-only sanitizer flags, each behind -Xarch_host)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

Plain C, -O2, no fast-math, no FMA contraction, no BLAS, no OpenMP: the
single-threaded reference that the GPU library is checked against.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hikvp_oracle.c")
LIB = os.path.join(HERE, "liboracle_hikvp.so")


SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def build(force: bool = True, out: str = LIB, sanitize: bool = False) -> str:
    """gcc build of the oracle at `out`; sanitize: an AddressSanitizer +
    UndefinedBehaviorSanitizer build of the same source (same -ffp-contract)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    tmp = out + ".tmp"
    opt = SANITIZE if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

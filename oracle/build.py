"""Build liboracle.so (the CPU oracle; test infrastructure only).

Plain gcc, OpenMP, no fast-math and no floating-point contraction, so that the
fp32 operations the oracle spells out (one fused multiply-add per term in the
fp32 router mode, separate fp32 multiply and add for the scale and biases) are
exactly the IEEE operations written in the source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall",
         "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False, src: str = None, out: str = None, extra=()) -> str:
    """Compile oracle.c (or `src`, e.g. a copy with a planted mistake for the
    pins' mutation check) into liboracle.so (or `out`)."""
    src = src or os.path.join(HERE, "oracle.c")
    out = out or os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc"] + FLAGS + list(extra) + [src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

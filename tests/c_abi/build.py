"""Build layer_c, a C program that runs the padding-free layer through
libxmoe's C ABI and the HIP runtime's C API only (test infrastructure: the
GPU test test_gpu_c_abi.py runs it).  Plain gcc, C11; links the in-tree
libxmoe.so through a relative run path, so the tree can move."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "padding_free_expert_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "layer_c")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "layer_c.c"), "-o", tmp,
           "-L", PKG, "-lxmoe", "-Wl,-rpath,$ORIGIN/../../padding_free_expert_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build tests/c/abi_from_c, a plain C caller of the library's ABI (test
infrastructure: it links the library and the fp64 oracle and checks one
against the other).  gcc only; the library and the oracle must be built
first.  Runtime search paths are relative to the binary, so the tree can
move."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_from_c.c")
BIN = os.path.join(HERE, "abi_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'include')}", "-o", BIN + ".tmp", SRC,
           f"-L{os.path.join(ROOT, 'row_wise_online_amd')}", "-los_softmax",
           f"-L{os.path.join(ROOT, 'oracle')}", "-loracle",
           f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../row_wise_online_amd:$ORIGIN/../../oracle:"
           f"{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

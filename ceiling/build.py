"""Build ``ceiling/libos_ceiling.so`` (gfx950) in-tree with the same hipcc
flags as the softmax library."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from row_wise_online_amd.build import ARCH, COMMON, HIPCC  # noqa: E402

LIB = os.path.join(HERE, "libos_ceiling.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ceiling.hip")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on ceiling.hip:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

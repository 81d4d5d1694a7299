"""Build the HIP library in-tree with hipcc for gfx950.

``python -m block_max_qk_amd.build`` compiles ``csrc/msa_index_score.hip``
into ``block_max_qk_amd/libmsa_index_score.so``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "msa_index_score.hip")
LIB = os.path.join(HERE, "libmsa_index_score.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def command(out: str = LIB):
    return [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"),
                              "-I", os.path.join(HERE, "csrc"), "-o", out, SRC]


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % out)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

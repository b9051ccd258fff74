"""Build libcsa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcsa.so")
SOURCES = ["api.hip", "compress.hip", "index_scores.hip", "topk.hip", "attention.hip", "index_backward.hip", "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def build(verbose=False):
    """Compile every source into libcsa.so (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(HERE, "..", "include")] + \
        [os.path.join(SRC, s) for s in SOURCES] + ["-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError("hipcc failed building libcsa.so")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))

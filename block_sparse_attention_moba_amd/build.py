"""Build libmoba.so (HIP for gfx950) in-tree with hipcc.

Each source compiles to its own object in parallel, then hipcc links the
shared library next to this file.  Usage: ``python -m
block_sparse_attention_moba_amd.build``.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libmoba.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic is kept off: scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# The attention kernels never see NaN inputs on their own arithmetic paths
# (masked logits are -inf, not NaN): without IEEE mode, fmaxf needs no
# quieting of its operands.  Matrix-core results go to ordinary vector
# registers, so the softmax reads the logits without copies out of the
# accumulation registers.
EXTRA = {"attn.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         # the gate's top-k network compares scores only (NaN inputs give no
         # defined selection): with NaNs ruled out, min / max / med3 need no
         # quieting instruction per score.  (IEEE mode stays on: with it off
         # as well, ROCm 7.2's compiler folds med3(max(-inf, a), b, -inf) to
         # med3(a, b, a) = a instead of min(a, b), breaking the list.)
         "gate.hip": ["-fno-honor-nans"]}


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmoba.so")
    return path


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [cc, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

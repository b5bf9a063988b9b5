"""Build libthdattn.so in-tree with hipcc for gfx950.

    python -m variable_length_packed_amd.build [--verbose]

Compiles every ``csrc/*.hip`` into one shared library next to this file.
"""
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libthdattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libthdattn.so")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # keep hipcc from forming packed fp32 ops on its own
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in VGPRs: the softmax / gradient VALU work reads them
        # directly instead of copying them out of AGPRs
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def build_library(verbose=False, extra_flags=()):
    """Compile csrc/*.hip into LIB_PATH.  Always recompiles."""
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc_path(), *compile_flags(), *extra_flags, "-shared", "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr:
        # hipcc's host pass warns about the device-only target feature
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose="--verbose" in sys.argv)
    print(LIB_PATH)

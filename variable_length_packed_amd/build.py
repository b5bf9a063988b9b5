"""Build libthdattn.so in-tree with hipcc for gfx950.

    python -m variable_length_packed_amd.build [--verbose]

Compiles every ``csrc/*.hip`` (one object each, under ``_build/``) and links
them into one shared library next to this file.
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


# Per-source machine-scheduler strategy, each measured on 16 causal
# sequences of 64-2048 tokens (h = 16, d = 128): the latency-oriented one ran
# the forward 1 % faster; the memory-clause one ran the dq pass 3-4 % faster
# (the latency-oriented one 2 %); neither helped the dk/dv pass.
PER_SOURCE_FLAGS = {
    "thd_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "thd_bwd_split.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
}


def compile_flags(source=None):
    """hipcc flags for one source (the common ones when source is None)."""
    flags = [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # keep hipcc from forming packed fp32 ops on its own
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]
    # MFMA results in VGPRs: the softmax / gradient VALU work reads them
    # directly instead of copying them out of AGPRs
    flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    if source is not None:
        flags += PER_SOURCE_FLAGS.get(os.path.basename(source), [])
    return flags


def build_library(verbose=False, extra_flags=()):
    """Compile csrc/*.hip into LIB_PATH (one object per source, in parallel,
    then one link).  Always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    hipcc = hipcc_path()
    objdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *compile_flags(src), *extra_flags, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return src, obj, res

    jobs = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, sources))
    for src, obj, res in results:
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} (exit {res.returncode})")
        if verbose and res.stderr:
            # hipcc's host pass warns about the device-only target feature
            lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
            if lines:
                sys.stderr.write("\n".join(lines) + "\n")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[obj for _, obj, _ in results]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def asan_runtime():
    """Path of the clang AddressSanitizer runtime that hipcc's host pass links
    against, or None."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc_path())))
    cands = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return cands[-1] if cands else None


def build_host_asan_library(out_path):
    """A copy of the library whose host code in thd_api.hip (argument checks,
    workspace sizes, status strings) is built with AddressSanitizer; the
    other sources' objects come from the last build_library run.  Device code
    is built as usual: the sanitizer flags are host-only."""
    objdir = os.path.join(PKG_DIR, "_build")
    # the objects of the current sources only (a removed source's object may
    # still sit in the build folder)
    others = [os.path.join(objdir, os.path.basename(src) + ".o")
              for src in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
              if os.path.basename(src) != "thd_api.hip"]
    if not others or not all(os.path.exists(o) for o in others):
        raise RuntimeError("build_library() first: its objects are linked in")
    hipcc = hipcc_path()
    src = os.path.join(CSRC, "thd_api.hip")
    obj = out_path + ".thd_api.o"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    res = subprocess.run([hipcc, *compile_flags(src), *san, "-c", "-o", obj, src],
                         capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed on thd_api.hip (host sanitizer build)")
    res = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                          "-Xarch_host", "-fsanitize=address", "-shared-libsan",
                          "-o", out_path, obj, *others], capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc link failed (host sanitizer build)")
    return out_path


if __name__ == "__main__":
    build_library(verbose="--verbose" in sys.argv)
    print(LIB_PATH)

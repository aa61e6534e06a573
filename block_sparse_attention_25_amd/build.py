"""Compile the HIP library (libbsa.so) in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "bsa.hip"), os.path.join(PKG, "csrc", "reblock.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, extra_flags=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (exit %d): %s" % (res.returncode, " ".join(cmd)))
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on
# the host code only: argument checks, geometry, workspace layout, launch
# set-up).  Each -fsanitize flag applies to the host pass alone, so the GPU
# code is built as usual.  Load it with the sanitizer runtime preloaded (see
# asan_runtime()) and BSA_LIBRARY pointing at it.
SANITIZE_FLAGS = [
    "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan",
]


def asan_runtime():
    """Path of the compiler's shared AddressSanitizer runtime, or None."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized(out_path: str) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + SANITIZE_FLAGS
    cmd = [hipcc, *flags, "-I", INCLUDE, *SRCS, "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (exit %d): %s\n%s" % (res.returncode, " ".join(cmd), res.stderr))
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libmoe.so, the HIP library behind the C ABI in include/moe.h (gfx950 only)."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "permute.hip", "experts.hip", "skinny.hip", "combine.hip", "backward.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source for gfx950 and link libmoe.so in the package directory."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        return obj

    n = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(n) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (device code
# built as usual, uninstrumented): the argument validation and error paths of
# the C ABI, for CPU runs.
SAN_LIB = os.path.join(PKG, "libmoe_san.so")
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O1",
    "-g",
    "-std=c++17",
    "-fPIC",
    "-fno-omit-frame-pointer",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime a host process preloads to load libmoe_san.so."""
    cc = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    for cand in (cc, "/opt/rocm/llvm/bin/clang++"):
        if os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("the AddressSanitizer runtime (libclang_rt.asan-x86_64.so) was not found")


def build_sanitized(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source, its host code with ASan + UBSan, and link libmoe_san.so."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *SAN_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized host compile failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    n = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(n) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

"""Build libpa.so (gfx950) in-tree with hipcc.

    python -m paged_kv_cache_188_amd.build
    python -m paged_kv_cache_188_amd.build --sanitize

Every source under csrc/ (HIP and host C++) is compiled to an object in parallel, then linked
into paged_kv_cache_188_amd/libpa.so.  The library is replaced atomically, so
a process that already loaded the previous build keeps a consistent copy.

--sanitize builds a second copy, _build/sanitize/libpa.so, whose HOST code
(the C ABI's argument validation, launch set-up and the block manager) is
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; device
code is built as usual.  A process loads it with PA_LIBRARY set to its path
and the sanitizer runtime preloaded (sanitizer_env() gives the variables);
tests/test_sanitized_host.py runs the host-side suites that way on the CPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpa.so")

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def sources():
    """HIP kernels and launchers (*.hip) and host-only C++ (*.cpp)."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer", "-g", "-shared-libsan"]
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libpa.so")


def _compile(src: str, verbose: bool, extra=(), out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature; that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    out_dir = SANITIZE_DIR if sanitize else BUILD_DIR
    lib_path = SANITIZE_LIB if sanitize else LIB_PATH
    extra = SANITIZE_HOST if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, out_dir), srcs))
    tmp = lib_path + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}", file=sys.stderr)
    return lib_path


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of hipcc's clang (it carries the
    UndefinedBehaviorSanitizer runtime too)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin",
                             "clang")
        res = subprocess.run([clang, "--print-runtime-dir"], capture_output=True, text=True)
        path = os.path.join(res.stdout.strip(), "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime of hipcc's clang not found")
    return path


def sanitizer_env() -> dict:
    """Environment for a process that loads the sanitized build."""
    return {"PA_LIBRARY": SANITIZE_LIB, "LD_PRELOAD": sanitizer_runtime(),
            "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])

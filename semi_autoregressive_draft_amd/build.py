"""Build libdspark.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m semi_autoregressive_draft_amd.build
    python -m semi_autoregressive_draft_amd.build --sanitize

Each .hip source is compiled to an object under _build/ in parallel, then
linked into semi_autoregressive_draft_amd/libdspark.so.

--sanitize builds libdspark_san.so with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (the device code is built as
usual), then runs the CPU tests of the C ABI against it: argument checks,
workspace sizing, status words and the no-allocation entry point's limits,
every host path that runs without a GPU.  The sanitizer runtime is preloaded
into the interpreter and the binding is pointed at the sanitized library
through DSPARK_LIB.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdspark.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no packed-fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# host-side sanitizers: every -fsanitize= carries -Xarch_host, so that the
# device code is built without them
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(PKG, "libdspark_san.so")
SAN_RUNTIME = "libclang_rt.asan-x86_64.so"


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    os.makedirs(SAN_BUILD if sanitize else BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = out + ".tmp"
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(link_san if sanitize else []), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def sanitizer_run(pytest_args=("tests/test_abi_cpu.py", "-q")) -> int:
    """Run CPU tests of the C ABI against libdspark_san.so; returns pytest's
    exit status (a sanitizer report aborts the run with a non-zero status)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    rt = subprocess.run([clang, f"-print-file-name={SAN_RUNTIME}"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        raise RuntimeError(f"sanitizer runtime {SAN_RUNTIME} not found")
    env = dict(os.environ, DSPARK_LIB=SAN_LIB, LD_PRELOAD=rt,
               # the interpreter's own allocations outlive it by design
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-m", "pytest", "-m", "not gpu", *pytest_args], cwd=ROOT,
                          env=env).returncode


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build(verbose=True, sanitize=True)
        sys.exit(sanitizer_run())
    build(verbose=True)
    sys.exit(0)

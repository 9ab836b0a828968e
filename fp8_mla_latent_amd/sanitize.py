"""Sanitizer build of the host code, and the CPU test suite run under it.

    python -m fp8_mla_latent_amd.sanitize

The library's host code (argument checks, split planning, workspace carving,
the shadow-file I/O of mla8_kvfile.hip) and the CPU oracle are rebuilt with
AddressSanitizer and UndefinedBehaviorSanitizer in a scratch copy of the
repository, and ``pytest -m "not gpu"`` runs there with the sanitizer runtime
preloaded into the Python process.  The device code is compiled as usual
(sanitizer flags go to the host pass only), and no test of that suite launches
a kernel.  Any report aborts the run with a non-zero exit status.

Both libraries are built with the ROCm clang so that one ASan runtime serves
the process (gcc's libasan next to clang's would conflict).  Nothing here runs
on a GPU; the normal in-tree libraries are left untouched.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LLVM = "/opt/rocm/llvm"

# host-pass-only sanitizer flags for hipcc: each -fsanitize= follows -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
ORACLE_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    hits = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found")
    return hits[-1]


def _copy_tree(dst: str) -> None:
    ignore = shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__", ".pytest_cache", "*.o")
    for d in ("fp8_mla_latent_amd", "oracle", "tests", "include"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d), ignore=ignore)
    for f in ("bench.py", "__graft_entry__.py"):
        shutil.copy2(os.path.join(ROOT, f), dst)
    os.makedirs(os.path.join(dst, "profiles"), exist_ok=True)
    for f in glob.glob(os.path.join(ROOT, "profiles", "*")):
        shutil.copy2(f, os.path.join(dst, "profiles"))


def build(dst: str) -> None:
    sys.path.insert(0, dst)
    from fp8_mla_latent_amd import build as b  # the copy's build module

    pkg = os.path.join(dst, "fp8_mla_latent_amd")
    src = [os.path.join(pkg, "csrc", os.path.basename(s)) for s in b.SRC]
    flags = [f if f != os.path.join(ROOT, "include") else os.path.join(dst, "include")
             for f in b.HIPCC_FLAGS]
    flags = [f if f != os.path.join(PKG, "csrc") else os.path.join(pkg, "csrc") for f in flags]
    subprocess.check_call([b.hipcc(), *flags, *HOST_SAN, *src, "-o",
                           os.path.join(pkg, "libmla8.so")])
    osrc = os.path.join(dst, "oracle", "mla8_oracle.c")
    ocflags = [f for f in ("-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           "-ffp-contract=off", "-fno-fast-math")]
    subprocess.check_call([os.path.join(LLVM, "bin", "clang"), *ocflags, *ORACLE_SAN,
                           "-o", os.path.join(dst, "oracle", "liboracle.so"), osrc, "-lm",
                           "-L" + os.path.join(LLVM, "lib"), "-Wl,-rpath," +
                           os.path.join(LLVM, "lib")])


def run(extra_args=()) -> int:
    dst = tempfile.mkdtemp(prefix="mla8_sanitize_")
    try:
        _copy_tree(dst)
        build(dst)
        env = dict(os.environ)
        env["LD_PRELOAD"] = asan_runtime()
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:detect_odr_violation=0"
        env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
        env["PYTHONDONTWRITEBYTECODE"] = "1"
        cmd = [sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-x", "-q",
               "-p", "no:cacheprovider", *extra_args]
        print("sanitizer run:", " ".join(cmd), flush=True)
        return subprocess.call(cmd, cwd=dst, env=env)
    finally:
        shutil.rmtree(dst, ignore_errors=True)


if __name__ == "__main__":
    sys.exit(run(sys.argv[1:]))

"""Host-code sanitizer run (CPU only; never on a GPU).

Builds a copy of the package whose host code is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (device code as usual), then
runs the host-only tests -- the ABI and planner tests and the owner planner's
parity tests -- against that library with the ASan runtime preloaded into
Python.  Any sanitizer report aborts the run with a non-zero exit status.

    python tests/sanitize_host.py [--keep DIR]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG_NAME = "matrix_optimizer_step_owned_amd"
sys.path.insert(0, os.path.join(ROOT, PKG_NAME))
import _build  # noqa: E402  (the package's own source list and compile flags)

SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan"]
TESTS = ["tests/test_abi_host.py", "tests/test_owners.py"]


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise SystemExit("no clang ASan runtime under /opt/rocm/llvm")
    return hits[-1]


def build(dst_root: str) -> str:
    pkg = os.path.join(dst_root, PKG_NAME)
    os.makedirs(os.path.join(pkg, "_b"), exist_ok=True)
    shutil.copy(os.path.join(ROOT, PKG_NAME, "__init__.py"), pkg)
    hipcc = _build._hipcc()
    flags = [f for f in _build.HIPCC_FLAGS]
    jobs, objs = [], []
    for src in _build.SOURCES:
        obj = os.path.join(pkg, "_b", src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([hipcc, *flags, *SANITIZE, "-c", os.path.join(_build.CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_build._run, jobs))
    lib = os.path.join(pkg, "libdmuon.so")
    _build._run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *SANITIZE, *objs, "-o", lib])
    return lib


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--keep", help="build into this directory and keep it")
    args = ap.parse_args()
    dst = args.keep or tempfile.mkdtemp(prefix="dmuon_sanitize_")
    lib = build(dst)
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([dst, ROOT] + ([env["PYTHONPATH"]] if env.get("PYTHONPATH") else []))
    env["LD_PRELOAD"] = asan_runtime()
    # Python's own allocations are not instrumented and its arenas look like
    # leaks; halt on the first real report
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    check = ("import " + PKG_NAME + " as m; assert m.LIB_PATH == " + repr(lib) + ", m.LIB_PATH")
    # and inside the pytest run: a test in the build directory that checks the
    # library every other test module imports
    probe = os.path.join(dst, "test_sanitized_library.py")
    with open(probe, "w") as f:
        f.write("import " + PKG_NAME + " as m\n\n\ndef test_sanitized_library_loaded():\n"
                "    assert m.LIB_PATH == " + repr(lib) + "\n")
    # run from the build directory, with pytest appending (not prepending)
    # the repository root to sys.path, so the sanitized package is the one
    # imported
    subprocess.run([sys.executable, "-c", check], env=env, cwd=dst, check=True)
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "--import-mode=append",
           "--rootdir", ROOT, "-m", "not gpu", *[os.path.join(ROOT, t) for t in TESTS], probe]
    rc = subprocess.run(cmd, env=env, cwd=dst).returncode
    print(f"sanitized library {lib}: pytest exit status {rc}")
    if not args.keep:
        shutil.rmtree(dst, ignore_errors=True)
    return rc


if __name__ == "__main__":
    sys.exit(main())

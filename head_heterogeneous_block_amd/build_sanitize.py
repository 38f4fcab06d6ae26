"""AddressSanitizer + UndefinedBehaviorSanitizer build of the library's host
code, and a run of the CPU test tier against it.

    python head_heterogeneous_block_amd/build_sanitize.py [pytest args]

builds libsparse_attn_san.so (host code instrumented; device code as in the
normal build) and runs ``pytest tests -m "not gpu"`` in a child process with
the sanitizer runtime preloaded and SA_SANITIZE=1, so the binding loads the
instrumented library.  Any sanitizer report aborts the child, which fails the
run.  Without a GPU every device call returns SA_ERR_NO_DEVICE, so this covers
the host logic: argument validation, schedules, budgets, calibration tables and
the debug checks' entry points.  Leak detection is off: the Python interpreter
and torch keep allocations alive until exit by design.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_LIB = os.path.join(HERE, "libsparse_attn_san.so")

# every sanitizer flag applies to the host side only
HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-g"]
LINK_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-shared-libsan"]


def runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too)."""
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                       check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"sanitizer runtime not found ({path!r})")
    return path


def main(argv: list[str]) -> int:
    sys.path.insert(0, HERE)
    import build  # noqa: E402

    build.build(verbose=True, sanitize=True)
    env = dict(os.environ)
    env["SA_SANITIZE"] = "1"
    env["LD_PRELOAD"] = runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "tests", "-m", "not gpu and not sanitize", "-q", "-p", "no:cacheprovider",
           *argv]
    print("running:", " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

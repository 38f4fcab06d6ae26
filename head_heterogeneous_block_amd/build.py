"""Build libsparse_attn.so for gfx950 with hipcc (in-tree).

Every HIP source is compiled for --offload-arch=gfx950 with packed fp32 vector
instructions disabled; objects go to ``_build/`` at the repository root and the
shared library next to this file.
"""

from __future__ import annotations

import concurrent.futures
import importlib.util
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["sa_api.cpp", "sa_select.hip", "sa_prefill.hip", "sa_prefill_wide.hip", "sa_decode.hip", "sa_calib.hip", "sa_peaks.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # inputs are finite: lets v_max/v_max3 take MFMA results without a
    # canonicalizing v_max per value (infinities, used as -inf masks, are kept)
    "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, obj: str, extra=()) -> None:
    lang = ["-x", "hip"]  # sa_api.cpp launches kernels through hip runtime: compile every file as HIP
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = False, sanitize: bool | None = None) -> str:
    """Compile every source and link the library; returns its path.  With
    ``sanitize`` (default: SA_SANITIZE=1 in the environment) the host code is
    built with AddressSanitizer and UndefinedBehaviorSanitizer into
    libsparse_attn_san.so instead (device code is unchanged); the binding loads
    that one when SA_SANITIZE=1 (see build_sanitize.py, which also runs the CPU
    tests under it)."""
    if sanitize is None:
        sanitize = os.environ.get("SA_SANITIZE") == "1"
    extra, link_extra, lib, sub = [], [], LIB, "_build"
    if sanitize:
        spec = importlib.util.spec_from_file_location("sa_build_sanitize", os.path.join(HERE, "build_sanitize.py"))
        san = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(san)
        extra, link_extra, lib, sub = san.HOST_FLAGS, san.LINK_FLAGS, san.SAN_LIB, os.path.join("_build", "san")
    out_dir = os.path.join(ROOT, sub)
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(out_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(lambda a: _compile(a[0], a[1], extra), zip(SOURCES, objs)))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)

"""Build libsparse_attn.so for gfx950 with hipcc (in-tree).

Every HIP source is compiled for --offload-arch=gfx950 with packed fp32 vector
instructions disabled; objects go to ``_build/`` at the repository root and the
shared library next to this file.
"""

from __future__ import annotations

import concurrent.futures
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


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"]  # sa_api.cpp launches kernels through hip runtime: compile every file as HIP
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(out_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

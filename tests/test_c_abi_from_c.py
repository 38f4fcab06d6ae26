"""The boundary used from plain C (no GPU needed).

include/sparse_attn.h is a C header: a C99 program that includes it compiles
with -pedantic -Werror, links against libsparse_attn.so and calls two host
entry points.  The schedule it prints equals the oracle's greedy LPT bit for
bit, and a bad argument comes back as a status code with the error text.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "head_heterogeneous_block_amd")
LIB = os.path.join(LIBDIR, "libsparse_attn.so")

PROGRAM = r"""
#include <stdio.h>
#include "sparse_attn.h"

int main(void) {
  const int64_t loads[9] = {7, 3, 9, 9, 1, 4, 4, 8, 2};
  int32_t bin_of[9], off[4], items[9];
  int64_t bin_load[3];
  int i;
  if (sa_version() < 10000) return 2;
  if (sa_lpt_schedule(loads, 9, 3, bin_of, off, items, bin_load) != SA_OK) return 3;
  for (i = 0; i < 9; ++i) printf("%d ", (int)bin_of[i]);
  printf("\n");
  for (i = 0; i < 4; ++i) printf("%d ", (int)off[i]);
  printf("\n");
  for (i = 0; i < 9; ++i) printf("%d ", (int)items[i]);
  printf("\n");
  for (i = 0; i < 3; ++i) printf("%lld ", (long long)bin_load[i]);
  printf("\n");
  /* a negative load: a status, and the reason in sa_last_error */
  {
    const int64_t bad[2] = {1, -1};
    sa_status st = sa_lpt_schedule(bad, 2, 1, bin_of, off, items, NULL);
    printf("%d %s\n", (int)st, sa_last_error());
  }
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_c_program_uses_the_library(tmp_path):
    src = tmp_path / "use_sparse_attn.c"
    exe = tmp_path / "use_sparse_attn"
    src.write_text(PROGRAM)
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                         os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", LIBDIR, "-lsparse_attn",
                         f"-Wl,-rpath,{LIBDIR}"], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stderr)
    lines = run.stdout.splitlines()
    got = [np.array(line.split(), dtype=np.int64) for line in lines[:4]]
    want = O.lpt_schedule([7, 3, 9, 9, 1, 4, 4, 8, 2], 3)
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g, np.asarray(w, dtype=np.int64))
    status, _, msg = lines[4].partition(" ")
    assert int(status) == -1 and "load" in msg, lines[4]

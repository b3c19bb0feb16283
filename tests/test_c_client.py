"""The boundary from plain C: the headers compile as strict C99 and as C++, a C program links
against liblbsa.so, takes the address of every declared entry point, and its call of the host
planner on the worked example of [P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 (requests of
1024, 5120 and 2048 tokens: tiles [2, 10, 4] over four workers, four tiles each) gives the oracle's
map word for word.  No GPU calls."""

import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from oracle.plan import ref_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "load_balanced_split_attn_amd")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _declared_functions():
    names = set()
    for hdr in sorted(os.listdir(INC)):
        if hdr.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(INC, hdr)).read(), flags=re.S)
            names |= set(re.findall(r"\b(attn_[a-z_]+)\s*\(", src))
    return sorted(names)


C_MAIN = r"""
#include <stdio.h>
#include "lbsa.h"
#include "lbsa_probe.h"

typedef void (*any_fn)(void);
static const any_fn entry_points[] = {
%(table)s
};

int main(void) {
  const int32_t lens[3] = {1024, 5120, 2048};
  int32_t map[256];
  int32_t words = 0;
  int rc;
  int i;
  /* every entry point resolved at link time */
  for (i = 0; i < (int)(sizeof(entry_points) / sizeof(entry_points[0])); ++i)
    if (!entry_points[i]) return 10;
  /* too small a buffer: LBSA_ERR_CAPACITY and the size needed */
  rc = attn_plan(lens, 3, 4, 512, map, 4, &words);
  if (rc != LBSA_ERR_CAPACITY || words <= 4) return 11;
  rc = attn_plan(lens, 3, 4, 512, map, 256, &words);
  if (rc != LBSA_OK) return 12;
  printf("words %%d\n", (int)words);
  for (i = 0; i < words; ++i) printf("%%d\n", (int)map[i]);
  printf("status %%s|%%s|%%s\n", attn_status_string(ATTN_OK), attn_status_string(ATTN_ERR_CAPACITY),
         attn_status_string(ATTN_ERR_INVALID));
  return 0;
}
"""


def _lib():
    path = os.path.join(PKG, "liblbsa.so")
    if not os.path.exists(path):
        pytest.fail("liblbsa.so is not built (python -m load_balanced_split_attn_amd.build)")
    return path


def test_headers_compile_as_c99_and_cpp(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "lbsa.h"\n#include "lbsa_probe.h"\nint lbsa_header_check;\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-I", INC,
                    str(src)], check=True)
    cpp = tmp_path / "h.cpp"
    cpp.write_text('#include "lbsa.h"\n#include "lbsa_probe.h"\nint lbsa_header_check;\n')
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-I", INC,
                    str(cpp)], check=True)


def test_c_program_plans_the_worked_example(tmp_path):
    lib = _lib()
    names = _declared_functions()
    assert "attn_plan" in names and "attn_splitkv" in names and "attn_combine" in names
    src = tmp_path / "client.c"
    src.write_text(C_MAIN % {"table": ",\n".join(f"  (any_fn){n}" for n in names)})
    exe = tmp_path / "client"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INC, str(src),
                    "-o", str(exe), "-L", os.path.dirname(lib), "-l:liblbsa.so",
                    "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.split("\n")
    words = int(out[0].split()[1])
    got = np.array([int(x) for x in out[1:1 + words]], dtype=np.int32)
    ref = ref_plan([1024, 5120, 2048], 4, 512)
    assert np.array_equal(got, ref)
    # budgets of the worked example: four tiles on each of the four workers
    assert got[5] == 16 and got[2] == 4
    status = out[1 + words].split(" ", 1)[1].split("|")
    assert len(status) == 3 and all(status) and len(set(status)) == 3

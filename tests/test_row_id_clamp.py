"""The range check of gathered row ids (csrc/row_ids.hpp), compiled for the host with g++ and run on
the CPU: the same constexpr functions decide, in the gather kernel and in the gathering GEMM loads,
whether an id lies in [0, rows) and which row an out-of-range id reads instead (the nearest one)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "hstu_sequential_transduction_attn_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include "row_ids.hpp"
using namespace hstu;
static_assert(row_id_in_range(0, 1) && !row_id_in_range(1, 1) && !row_id_in_range(-1, 1), "");
static_assert(clamp_row_id(-5, 10) == 0 && clamp_row_id(10, 10) == 9 && clamp_row_id(3, 10) == 3, "");
int main() {
  const long long ids[] = {-9223372036854775807LL - 1, -1, 0, 1, 6, 7, 8, 1000, 9223372036854775807LL};
  const long long rows[] = {1, 7, 8, 4294967297LL};
  for (long long r : rows)
    for (long long id : ids)
      printf("%lld %lld %d %lld\n", id, r, (int)row_id_in_range(id, r), (long long)clamp_row_id(id, r));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_clamp_of_row_ids_on_the_host(tmp_path):
    src = tmp_path / "clamp.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "clamp"
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    n = 0
    for line in out:
        if not line.strip():
            continue
        id_, rows, ok, got = (int(v) for v in line.split())
        assert ok == (0 <= id_ < rows), line
        assert got == min(max(id_, 0), rows - 1), line
        n += 1
    assert n == 36

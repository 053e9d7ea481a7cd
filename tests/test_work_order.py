"""The work order of the query-major attention kernels (csrc/work_order.hpp), compiled for the host with
g++ and run on the CPU: the map from workgroup index to (block rank, sequence-head pair) must visit every
item exactly once for every shape; when the pairs divide evenly among the 8 XCDs, every workgroup on XCD x
(index % 8 = x) works on a pair of that XCD (pair % 8 = x), and the backward's canonical row of an item is
its rank-major position.  The listed order of one small shape is compared with the groups the
header describes (first two pairs interleaved, then one pair at a time, then the last two interleaved)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "hstu_sequential_transduction_attn_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <vector>
#include "work_order.hpp"
using namespace hstu::attn;
int main(int argc, char **argv) {
  if (argc == 3) {   // list one shape's order
    const int HB = atoi(argv[1]), nqb = atoi(argv[2]);
    for (int i = 0; i < HB * nqb; ++i) {
      const WorkItem w = work_item(i, HB, nqb);
      printf("%d %d %d\n", i, w.rank, w.pair);
    }
    return 0;
  }
  int shapes = 0;
  for (int HB = 1; HB <= 200; ++HB)
    for (int nqb = 1; nqb <= 40; ++nqb) {
      std::vector<int> seen((size_t)HB * nqb, 0);
      for (int i = 0; i < HB * nqb; ++i) {
        const WorkItem w = work_item(i, HB, nqb);
        if (w.rank < 0 || w.rank >= nqb || w.pair < 0 || w.pair >= HB) { printf("RANGE %d %d %d\n", HB, nqb, i); return 1; }
        const int c = canonical_item(w, HB);
        if (c != w.rank * HB + w.pair) { printf("CANON %d %d %d\n", HB, nqb, i); return 1; }
        if (HB % 8 == 0 && w.pair % 8 != i % 8) { printf("XCD %d %d %d\n", HB, nqb, i); return 1; }
        if (seen[c]++) { printf("TWICE %d %d %d\n", HB, nqb, i); return 1; }
      }
      ++shapes;
    }
  printf("ok %d\n", shapes);
  return 0;
}
"""


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("work_order")
    src = d / "order.cpp"
    src.write_text(PROGRAM)
    out = d / "order"
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", CSRC, str(src), "-o", str(out)], check=True)
    return str(out)


def test_every_item_once_and_xcd_local(exe):
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.strip()
    assert out == f"ok {200 * 40}", out


def _order(exe, HB, nqb):
    lines = subprocess.run([exe, str(HB), str(nqb)], check=True, capture_output=True, text=True).stdout.split("\n")
    return [tuple(int(v) for v in ln.split()) for ln in lines if ln.strip()]


def test_groups_listed(exe):
    """HB = 40 pairs (5 per XCD), 3 blocks each: XCD 3 runs pairs 3, 11 interleaved (rank 0, the longest
    block, first), then 19 alone, then 27 and 35 interleaved."""
    order = _order(exe, 40, 3)
    xcd3 = [(r, p) for i, r, p in order if i % 8 == 3]
    assert xcd3 == [(0, 3), (0, 11), (1, 3), (1, 11), (2, 3), (2, 11),
                    (0, 19), (1, 19), (2, 19),
                    (0, 27), (0, 35), (1, 27), (1, 35), (2, 27), (2, 35)]


def test_few_pairs_keep_rank_major(exe):
    """HB not a multiple of 8, or at most 3 pairs per XCD: rank major (longest block first) over all pairs."""
    for HB, nqb in ((7, 4), (24, 5), (12, 3)):
        order = _order(exe, HB, nqb)
        assert [(r, p) for _, r, p in order] == [(i // HB, i % HB) for i in range(HB * nqb)]

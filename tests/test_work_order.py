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


def _expected_xcd_order(x, PX, nb):
    """The groups the header describes, for XCD x: g pairs at each end run together (rank by rank, the
    group's pairs in turn), every pair in between alone (rank by rank); g = 2 when PX nb >= 1024, else
    max(2, ceil(128 / nb))."""
    g = 2 if PX * nb >= 1024 else max(2, -(-128 // nb))
    if PX < 2 * g:
        groups = [list(range(PX))]
    else:
        groups = [list(range(g))] + [[p] for p in range(g, PX - g)] + [list(range(PX - g, PX))]
    return [(r, x + 8 * p) for grp in groups for r in range(nb) for p in grp]


@pytest.mark.parametrize("PX,nb", [(5, 64), (9, 32), (40, 8), (7, 3), (4, 64), (64, 72), (64, 32), (16, 64), (128, 8)])
def test_groups_listed(exe, PX, nb):
    """Each XCD's list of items follows the end-group rule (e.g. 5 pairs of 64 blocks: the first two
    interleaved, the middle one alone, the last two interleaved; 9 pairs of 32 blocks: groups of 4;
    64 pairs of 32 blocks, deep enough for groups of 2)."""
    order = _order(exe, 8 * PX, nb)
    for x in (0, 3, 7):
        assert [(r, p) for i, r, p in order if i % 8 == x] == _expected_xcd_order(x, PX, nb), (PX, nb, x)


def test_few_pairs_keep_rank_major(exe):
    """HB not a multiple of 8, or fewer than 2 g pairs per XCD: rank major (longest block first) over all
    pairs."""
    for HB, nqb in ((7, 4), (24, 5), (12, 3), (24, 64), (128, 8), (504, 4)):
        order = _order(exe, HB, nqb)
        assert [(r, p) for _, r, p in order] == [(i // HB, i % HB) for i in range(HB * nqb)]

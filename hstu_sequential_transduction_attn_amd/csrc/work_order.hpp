// Order of the work items of the attention kernels (the forward and the backward's dQ pass, query
// blocks; the backward's dK/dV pass, key blocks): item i (the workgroup index) -> (block rank, sequence-
// head pair), rank 0 being the pair's block with the most work (the last query block, the first key
// block).  Plain constexpr code, compiled for the device by the kernels and for the host by a test that
// checks the map is a bijection.
//
// Workgroups are handed to the chip's 8 XCDs round robin (workgroup i to XCD i % 8), and each XCD has its
// own L2.  Every query block of a (sequence, head) pair reads that pair's K and V from the first key
// tile on (every key block its Q and dO up to the last query tile), so the fewer pairs an XCD works on
// at a time, the more of those reads its L2 serves.  When the pairs divide evenly among the XCDs
// (HB = 8 PX), XCD x takes pairs x, x + 8, ..., x + 8 (PX - 1) and runs them in groups, longest block
// first (rank order) inside each group:
//   - the first two pairs together and the last two pairs together: a lone pair's longest blocks would
//     start late at the end (and set the kernel's end) and leave the XCD half filled at the start;
//   - every pair in between alone.
// With PX <= 3 the XCD runs all its pairs as one group, and when HB is not a multiple of 8 the items
// go rank major over all pairs: both are the order of a single group.
#pragma once

namespace hstu {
namespace attn {

struct WorkItem {
  int rank;   // 0: the pair's block with the most work
  int pair;   // sequence * num_heads + head
};

// item in [0, HB * nb); HB = number of (sequence, head) pairs, nb = blocks per pair
constexpr WorkItem work_item(int item, int HB, int nb) {
  const int PX = HB >> 3;
  if ((HB & 7) != 0 || PX <= 3) return WorkItem{item / HB, item % HB};
  const int x = item & 7, j = item >> 3;
  const int e0 = 2 * nb, e1 = (PX - 2) * nb;   // end of the first group, start of the last
  int rank = 0, pr = 0;
  if (j < e0) {
    rank = j / 2;
    pr = j % 2;
  } else if (j < e1) {
    pr = 2 + (j - e0) / nb;
    rank = (j - e0) % nb;
  } else {
    rank = (j - e1) / 2;
    pr = PX - 2 + (j - e1) % 2;
  }
  return WorkItem{rank, x + 8 * pr};
}

// The position of an item in rank-major order: the backward's dQ pass stores each workgroup's
// bias-gradient bins at this row, so that their reduction adds the rows in the same order whatever the
// work order.
constexpr int canonical_item(WorkItem w, int HB) { return w.rank * HB + w.pair; }

}  // namespace attn
}  // namespace hstu

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
//   - its first g pairs together and its last g pairs together: the groups at the ends fill the XCD's 64
//     workgroup slots at the start and let the last long blocks start early enough at the end (a lone
//     last pair's longest blocks would set the kernel's end).  With nb blocks per pair (the longest
//     2 nb key tiles, a pair about nb^2), an XCD's 64 slots each hold about PX nb / 128 longest blocks
//     of work: at 8 or more (PX nb >= 1024) the end is short against the whole and g = 2 keeps the most
//     locality; below that g = max(2, ceil(128 / nb)), so that the last group alone holds one longest
//     block's time of work per slot;
//   - every pair in between alone.
// With fewer than 2 g pairs per XCD, or pairs that do not divide by 8, the items go rank major over all
// pairs: the order of a single group.
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
  const int gt = (128 + nb - 1) / nb;
  const int g = (PX * nb >= 1024 || gt < 2) ? 2 : gt;   // pairs in each end group
  if ((HB & 7) != 0 || PX < 2 * g) return WorkItem{item / HB, item % HB};
  const int x = item & 7, j = item >> 3;
  const int e0 = g * nb, e1 = (PX - g) * nb;   // end of the first group, start of the last
  int rank = 0, pr = 0;
  if (j < e0) {
    rank = j / g;
    pr = j % g;
  } else if (j < e1) {
    pr = g + (j - e0) / nb;
    rank = (j - e0) % nb;
  } else {
    rank = (j - e1) / g;
    pr = PX - g + (j - e1) % g;
  }
  return WorkItem{rank, x + 8 * pr};
}

// The position of an item in rank-major order: the backward's dQ pass stores each workgroup's
// bias-gradient bins at this row, so that their reduction adds the rows in the same order whatever the
// work order.
constexpr int canonical_item(WorkItem w, int HB) { return w.rank * HB + w.pair; }

}  // namespace attn
}  // namespace hstu

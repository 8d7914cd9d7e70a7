// Host-side metadata region and the attention work-unit split (host only).
//
// The split decides how many work-groups the attention kernel runs and how
// many keys each reads, so it sets the kernel's HBM traffic together with
// k_attn.hip; the measured-traffic record of the attention kernel names this
// file and k_attn.hip.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "kvpool.h"

namespace er {

// A bump allocator over the pinned host metadata region (h) and its device
// mirror (d): offsets are 256-byte aligned and valid in both.
struct Meta {
  char* h = nullptr;
  char* d = nullptr;
  size_t used = 0, cap = 0;
  bool ok = true;
  void reset() { used = 0; ok = true; }
  template <class T>
  T* push(size_t n, size_t* off) {
    const size_t a = (used + 255) & ~(size_t)255;
    if (a + n * sizeof(T) > cap) { ok = false; *off = 0; return nullptr; }
    *off = a;
    used = a + n * sizeof(T);
    return (T*)(h + a);
  }
  template <class T>
  T* dev(size_t off) const { return (T*)(d + off); }
};

// Attention work units of the n items whose queries start at pos0[i] and
// number cnt[i], pushed into the metadata region as [n + 1] exclusive prefix
// sums of units per item followed by [n] blocks per unit of each item.  The
// unit length (unit_target) aims at ~768 work-groups over all KV heads -- one
// resident round of the attention kernel at three work-groups per CU -- but
// is at least 16 blocks (4 per wave of a work-group), and once the items
// alone give 768 work-groups no item is split below 1024 blocks.  From sweeps
// on MI355X at the rollout's batch and context pairs, against an aim of ~1024
// work-groups with no split from 512 items: attention 4 % faster at batch 96
// (2 units of 103 blocks each instead of 3: 128.0 vs 133.4 us), 2-6 % at
// batch 6-46, 1-2 % slower at batch 1 and 22, and the same at batch 204 (816
// items, not split either way; splitting them in two made the kernel 3 %
// faster but the combine cost more).  An aim of ~1536 with units from 8
// blocks was 6 % faster at batch 1 and 7 % slower at batch 11.  Earlier, with
// two resident work-groups per CU, ~1024 with 16 blocks at least had beaten
// ~256 with 8 by 12-15 % at batch 11-22.  An item of nblk blocks is cut into
// ceil(nblk/target) even units (so at most ceil(nblk/16) units, each over
// half the target), and an item that fits in one unit is not split (no
// combine for it).  Then the list of
// the items that were split ([n] entries, n_split used), and the most units
// of one item.  *o_rec gets the offset of one record per unit, eight int32
// each: item, split index | units of the item << 16, first block, blocks per
// unit, query count, first query position, first query row, block-table row
// (row0 and btrow per item), so that a work-group finds all of it in one load.
// Blocks per attention work unit for `total` key blocks over all items.
// The split's aim and floor: kAttnAimPairs (unit, KV head) pairs, units of
// at least kAttnMinUnitBlocks blocks, no split once the items alone give
// kAttnNoSplitPairs pairs.
constexpr int64_t kAttnAimPairs = 768, kAttnMinUnitBlocks = 16, kAttnNoSplitPairs = 768;
inline int64_t unit_target(int64_t total, int hkv) {
  return std::min<int64_t>(1024, std::max<int64_t>(kAttnMinUnitBlocks, (total * hkv + kAttnAimPairs - 1) / kAttnAimPairs));
}

inline size_t push_units(Meta& M, int n, int hkv, const int32_t* pos0, const int32_t* cnt, const int32_t* row0,
                         const int32_t* btrow, int* n_units, int* n_split, int* max_units, size_t* o_rec) {
  size_t off = 0;
  int32_t* us = M.push<int32_t>((size_t)3 * n + 1, &off);
  if (!us) return 0;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
  const int64_t target = (int64_t)n * hkv >= kAttnNoSplitPairs ? 1024 : unit_target(total, hkv);
  int32_t acc = 0;
  int ns = 0, mu = 0;
  for (int i = 0; i < n; ++i) {
    us[i] = acc;
    const int64_t nblk = (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
    const int64_t nu = std::max<int64_t>(1, (nblk + target - 1) / target);
    us[n + 1 + i] = (int32_t)((nblk + nu - 1) / nu);
    if (nu > 1) us[2 * n + 1 + ns++] = i;
    acc += (int32_t)nu;
    mu = std::max(mu, (int)nu);
  }
  us[n] = acc;
  *n_units = acc;
  *n_split = ns;
  *max_units = mu;
  int32_t* rec = M.push<int32_t>((size_t)8 * std::max(acc, 1), o_rec);
  if (!rec) return 0;
  for (int i = 0; i < n; ++i) {
    const int nu = us[i + 1] - us[i], bpu = us[n + 1 + i];
    for (int k = 0; k < nu; ++k) {
      int32_t* r = rec + (size_t)8 * (us[i] + k);
      r[0] = i;
      r[1] = k | (nu << 16);
      r[2] = k * bpu;
      r[3] = bpu;
      r[4] = cnt[i];
      r[5] = pos0[i];
      r[6] = row0[i];
      r[7] = btrow[i];
    }
  }
  return off;
}

// A fixed-shape split for replayed graphs: every item gets exactly U units
// (so the unit count n * U, the split list and the combine grid depend on n
// and U alone, not on the contexts).  Item i's units are ceil(nblk_i / U)
// blocks long; units that start past the item's last block read nothing and
// leave an empty partial (running max -inf, sum 0), which the combine weighs
// by zero.  With U = 1 no item is split.  The layout (unit table [3n + 1],
// then n * U records) is the one push_units writes.
// Units per item of a graph's fixed split, for n items of at most cap_blocks
// blocks: sized at half the capacity, the low end of a capacity class, so
// that units stay at the eager split's length where contexts sit (a class
// spans cap/2 .. cap), and never longer than the 1024 block ids one
// work-group of the attention kernel stages.
inline int graph_units_per_item(int n, int hkv, int cap_blocks) {
  const int64_t half = std::max<int64_t>(1, cap_blocks / 2);
  const int64_t target = unit_target((int64_t)n * half, hkv);
  const int64_t u = std::max<int64_t>((half + target - 1) / target, ((int64_t)cap_blocks + 1023) / 1024);
  return (int)std::max<int64_t>(1, u);
}
inline size_t push_units_fixed(Meta& M, int n, int U, const int32_t* pos0, const int32_t* cnt, const int32_t* row0,
                               const int32_t* btrow, size_t* o_rec) {
  size_t off = 0;
  int32_t* us = M.push<int32_t>((size_t)3 * n + 1, &off);
  if (!us) return 0;
  int32_t* rec = M.push<int32_t>((size_t)8 * n * U, o_rec);
  if (!rec) return 0;
  for (int i = 0; i <= n; ++i) us[i] = i * U;
  for (int i = 0; i < n; ++i) {
    const int64_t nblk = (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
    const int32_t bpu = (int32_t)std::max<int64_t>(1, (nblk + U - 1) / U);
    us[n + 1 + i] = bpu;
    us[2 * n + 1 + i] = i;
    for (int k = 0; k < U; ++k) {
      int32_t* r = rec + (size_t)8 * ((size_t)i * U + k);
      r[0] = i;
      r[1] = k | (U << 16);
      r[2] = k * bpu;
      r[3] = bpu;
      r[4] = cnt[i];
      r[5] = pos0[i];
      r[6] = row0[i];
      r[7] = btrow[i];
    }
  }
  return off;
}

}  // namespace er

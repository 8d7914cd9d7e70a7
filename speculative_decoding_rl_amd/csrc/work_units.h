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
// unit length aims at ~256 work-groups over all KV heads (one per compute
// unit: fewer, longer units keep each wave's block ring full, and a long
// sequence no longer sets the kernel time alone; from a sweep of 128 / 256 /
// 512 / 1024 / 2048 on MI355X at batch 1..128 and 4k/8k context) but never
// goes below 8 blocks; an item's units split its blocks evenly, and an item
// that fits in one unit is not split (no combine for it).  Then the list of
// the items that were split ([n] entries, n_split used), and the most units
// of one item.  *o_rec gets the offset of one record per unit, eight int32
// each: item, split index | units of the item << 16, first block, blocks per
// unit, query count, first query position, first query row, block-table row
// (row0 and btrow per item), so that a work-group finds all of it in one load.
inline size_t push_units(Meta& M, int n, int hkv, const int32_t* pos0, const int32_t* cnt, const int32_t* row0,
                         const int32_t* btrow, int* n_units, int* n_split, int* max_units, size_t* o_rec) {
  size_t off = 0;
  int32_t* us = M.push<int32_t>((size_t)3 * n + 1, &off);
  if (!us) return 0;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
  const int64_t target = std::min<int64_t>(1024, std::max<int64_t>(8, (total * hkv + 255) / 256));
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

}  // namespace er

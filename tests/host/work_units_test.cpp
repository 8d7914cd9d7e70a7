// Host unit test of the attention work-unit split (csrc/work_units.h), built
// with g++ and the address/undefined-behaviour sanitizers by
// tests/test_host_abi.py: on random batches the units cover every item's key
// blocks exactly once, the per-unit records agree with the unit table, and a
// metadata region that is too small fails cleanly.  Prefill-shaped batches
// too: one sequence's chunk of up to 4096 prompt tokens cut into items of
// qmax = 64 / (n_q_heads / n_kv_heads) queries at consecutive positions, for
// prompts of up to 15000 tokens filled chunk after chunk into one region (as
// er_prefill does, each fill starting from a reset region).  And the
// fixed-shape split of replayed graphs (push_units_fixed): every item's blocks
// covered exactly once by its U units, no unit over 1024 blocks.
#include <algorithm>
#include <cassert>
#include <cstdio>
#include <random>
#include <vector>

#include "../../speculative_decoding_rl_amd/csrc/work_units.h"

using namespace er;

// Split n items into the region and check every invariant; returns the number of units.
static int check_split(Meta& M, int n, int hkv, const std::vector<int32_t>& pos0, const std::vector<int32_t>& cnt,
                       const std::vector<int32_t>& row0, const std::vector<int32_t>& btrow) {
  int nu_tot = -1, ns = -1, mu = -1;
  size_t o_rec = 0;
  const size_t off = push_units(M, n, hkv, pos0.data(), cnt.data(), row0.data(), btrow.data(), &nu_tot, &ns, &mu,
                                &o_rec);
  assert(M.ok);
  assert(M.used <= M.cap);
  const int32_t* us = (const int32_t*)(M.h + off);
  const int32_t* rec = (const int32_t*)(M.h + o_rec);
  assert(us[0] == 0 && us[n] == nu_tot);
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
  // ~768 (unit, KV head) pairs of at least 16 blocks; no split below 1024 blocks once the items alone
  // give 768 pairs
  const bool many = (int64_t)n * hkv >= 768;
  const int64_t target = many ? 1024 : std::min<int64_t>(1024, std::max<int64_t>(16, (total * hkv + 767) / 768));
  int split_seen = 0, most = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t nblk = (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
    const int nu = us[i + 1] - us[i];
    const int bpu = us[n + 1 + i];
    assert(nu >= 1 && bpu >= 1);
    // the attention kernel stages one unit's block ids in LDS, at most 1024 of them
    assert(bpu <= 1024);
    // the units cover the blocks: the last one is non-empty and none runs past the end
    assert((int64_t)bpu * nu >= nblk && (int64_t)bpu * (nu - 1) < nblk);
    // an item that fits one unit is not split; a split item has at most ceil(nblk / 16) units (within
    // the ceil(nblk / 8) the partials area and the combine are sized by) of more than half the target
    assert((nblk <= target) == (nu == 1));
    assert(nu <= (nblk + 15) / 16 || nu == 1);
    if (nu > 1) assert(2 * (int64_t)bpu > target);
    if (nu > 1) {
      assert(us[2 * n + 1 + split_seen] == i);
      ++split_seen;
    }
    most = std::max(most, nu);
    for (int k = 0; k < nu; ++k) {
      const int32_t* r = rec + (size_t)8 * (us[i] + k);
      assert(r[0] == i && (r[1] & 0xFFFF) == k && (r[1] >> 16) == nu);
      assert(r[2] == k * bpu && r[3] == bpu);
      // every unit starts inside its item's blocks
      assert((int64_t)r[2] < nblk);
      assert(r[4] == cnt[i] && r[5] == pos0[i] && r[6] == row0[i] && r[7] == btrow[i]);
    }
  }
  assert(split_seen == ns && most == mu);
  // about 768 (unit, KV head) pairs once the target is neither floored nor capped
  if (!many && target > 16 && target < 1024) assert((int64_t)nu_tot * hkv <= 768 + (int64_t)n * hkv);
  if (many) assert(ns == 0 || mu >= 2);
  return nu_tot;
}

// The fixed-shape split of replayed graphs: U units per item, the item's
// blocks covered exactly once in unit order, units past the end empty, no
// unit longer than the 1024 block ids a work-group stages, and the layout of
// push_units (unit table, blocks per unit, split list, records).
static void check_fixed(Meta& M, int n, int hkv, int cap, const std::vector<int32_t>& pos0,
                        const std::vector<int32_t>& cnt, const std::vector<int32_t>& row0,
                        const std::vector<int32_t>& btrow) {
  const int U = graph_units_per_item(n, hkv, cap);
  assert(U >= 1 && U <= (cap + 15) / 16 + 1 && (int64_t)U * 1024 >= cap);
  size_t o_rec = 0;
  const size_t off = push_units_fixed(M, n, U, pos0.data(), cnt.data(), row0.data(), btrow.data(), &o_rec);
  assert(M.ok && M.used <= M.cap);
  const int32_t* us = (const int32_t*)(M.h + off);
  const int32_t* rec = (const int32_t*)(M.h + o_rec);
  for (int i = 0; i <= n; ++i) assert(us[i] == i * U);
  for (int i = 0; i < n; ++i) {
    const int64_t nblk = (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
    assert(nblk <= cap);
    const int bpu = us[n + 1 + i];
    assert(bpu >= 1 && bpu <= 1024);
    assert(us[2 * n + 1 + i] == i);
    std::vector<int> seen((size_t)nblk, 0);
    for (int k = 0; k < U; ++k) {
      const int32_t* r = rec + (size_t)8 * ((size_t)i * U + k);
      assert(r[0] == i && (r[1] & 0xFFFF) == k && (r[1] >> 16) == U);
      assert(r[2] == k * bpu && r[3] == bpu);
      assert(r[4] == cnt[i] && r[5] == pos0[i] && r[6] == row0[i] && r[7] == btrow[i]);
      for (int64_t b = r[2]; b < std::min<int64_t>(nblk, (int64_t)r[2] + bpu); ++b) ++seen[(size_t)b];
    }
    for (int64_t b = 0; b < nblk; ++b) assert(seen[(size_t)b] == 1);
  }
}

int main() {
  std::mt19937 rng(11);
  std::vector<char> buf((size_t)8 << 20);
  for (int it = 0; it < 400; ++it) {
    const int n = 1 + (int)(rng() % 300);
    const int hkv = 1 << (rng() % 4);
    std::vector<int32_t> pos0(n), cnt(n), row0(n), btrow(n);
    int32_t row = 0;
    for (int i = 0; i < n; ++i) {
      pos0[i] = (int32_t)(rng() % (it % 3 == 0 ? 64 : 20000));
      cnt[i] = 1 + (int32_t)(rng() % 9);
      row0[i] = row;
      row += cnt[i];
      btrow[i] = (int32_t)(rng() % 1000);
    }
    Meta M;
    M.h = buf.data();
    M.d = buf.data();
    M.cap = buf.size();
    M.reset();
    check_split(M, n, hkv, pos0, cnt, row0, btrow);
    // a region too small for the records: not ok, nothing written past it
    Meta S;
    std::vector<char> small(4 * (3 * (size_t)n + 1));  // the unit table fits, the records do not
    S.h = small.data();
    S.d = small.data();
    S.cap = small.size();
    S.reset();
    int a = 0, b = 0, c = 0;
    size_t o2 = 0;
    push_units(S, n, hkv, pos0.data(), cnt.data(), row0.data(), btrow.data(), &a, &b, &c, &o2);
    assert(!S.ok);
  }
  // prefill-shaped batches: chunks of one long prompt, filled one after another into one region of
  // the library's size (64 MiB), items of qmax queries at consecutive positions
  std::vector<char> region((size_t)64 << 20);
  const int prompts[] = {700, 2560, 4096, 9000, 15000, 15001};
  const int qmaxes[] = {9, 64};    // 64 / group size for the 7B shape (group 7) and for MHA
  const int chunks[] = {256, 4096};
  for (int plen : prompts)
    for (int qmax : qmaxes)
      for (int chunk : chunks)
        for (int hkv : {4, 8}) {
          int fills = 0;
          for (int c0 = 0; c0 < plen; c0 += chunk) {
            const int cn = std::min(chunk, plen - c0);
            const int n = (cn + qmax - 1) / qmax;
            std::vector<int32_t> pos0(n), cnt(n), row0(n), btrow(n, 3);
            for (int k = 0; k < n; ++k) {
              pos0[k] = c0 + k * qmax;
              cnt[k] = std::min(qmax, cn - k * qmax);
              row0[k] = k * qmax;
            }
            Meta M;
            M.h = region.data();
            M.d = region.data();
            M.cap = region.size();
            M.reset();
            // the rows of one chunk: positions c0 .. c0 + cn - 1, each item's queries inside the chunk
            assert(row0[n - 1] + cnt[n - 1] == cn);
            check_split(M, n, hkv, pos0, cnt, row0, btrow);
            ++fills;
          }
          assert(fills == (plen + chunk - 1) / chunk);
        }
  // fixed-shape splits: power-of-two batches and capacity classes, contexts up to the capacity
  for (int it = 0; it < 300; ++it) {
    const int n = 1 << (rng() % 5);
    const int hkv = 1 << (rng() % 4);
    const int cap = 16 << (rng() % 12);   // up to 32768 blocks (512k keys)
    const int q = 1 + (int)(rng() % 9);
    std::vector<int32_t> pos0(n), cnt(n, q), row0(n), btrow(n);
    for (int i = 0; i < n; ++i) {
      pos0[i] = (int32_t)(rng() % (cap * KV_BLOCK - q + 1));
      row0[i] = i * q;
      btrow[i] = i;
    }
    Meta M;
    M.h = buf.data();
    M.d = buf.data();
    M.cap = buf.size();
    M.reset();
    check_fixed(M, n, hkv, cap, pos0, cnt, row0, btrow);
  }
  std::printf("work_units ok\n");
  return 0;
}

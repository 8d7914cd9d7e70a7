// Host unit test of the attention work-unit split (csrc/work_units.h), built
// with g++ and the address/undefined-behaviour sanitizers by
// tests/test_host_abi.py: on random batches the units cover every item's key
// blocks exactly once, the per-unit records agree with the unit table, and a
// metadata region that is too small fails cleanly.
#include <algorithm>
#include <cassert>
#include <cstdio>
#include <random>
#include <vector>

#include "../../speculative_decoding_rl_amd/csrc/work_units.h"

using namespace er;

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
    int nu_tot = -1, ns = -1, mu = -1;
    size_t o_rec = 0;
    const size_t off = push_units(M, n, hkv, pos0.data(), cnt.data(), row0.data(), btrow.data(), &nu_tot, &ns, &mu,
                                  &o_rec);
    assert(M.ok);
    const int32_t* us = (const int32_t*)(M.h + off);
    const int32_t* rec = (const int32_t*)(M.h + o_rec);
    assert(us[0] == 0 && us[n] == nu_tot);
    int64_t total = 0;
    for (int i = 0; i < n; ++i) total += (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
    const int64_t target = std::min<int64_t>(1024, std::max<int64_t>(8, (total * hkv + 255) / 256));
    int split_seen = 0, most = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t nblk = (pos0[i] + cnt[i] + KV_BLOCK - 1) / KV_BLOCK;
      const int nu = us[i + 1] - us[i];
      const int bpu = us[n + 1 + i];
      assert(nu >= 1 && bpu >= 1);
      // the units cover the blocks: the last one is non-empty and none runs past the end
      assert((int64_t)bpu * nu >= nblk && (int64_t)bpu * (nu - 1) < nblk);
      // an item that fits one unit is not split; units hold at least min(nblk, 8) blocks
      assert((nblk <= target) == (nu == 1));
      assert(bpu >= std::min<int64_t>(nblk, 8));
      if (nu > 1) {
        assert(us[2 * n + 1 + split_seen] == i);
        ++split_seen;
      }
      most = std::max(most, nu);
      for (int k = 0; k < nu; ++k) {
        const int32_t* r = rec + (size_t)8 * (us[i] + k);
        assert(r[0] == i && (r[1] & 0xFFFF) == k && (r[1] >> 16) == nu);
        assert(r[2] == k * bpu && r[3] == bpu);
        assert(r[4] == cnt[i] && r[5] == pos0[i] && r[6] == row0[i] && r[7] == btrow[i]);
      }
    }
    assert(split_seen == ns && most == mu);
    // about 256 (unit, KV head) pairs once the target is neither floored nor capped
    if (target > 8 && target < 1024) assert((int64_t)nu_tot * hkv <= 256 + (int64_t)n * hkv);
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
  std::printf("work_units ok\n");
  return 0;
}

// Host unit test of the paged KV block pool and block tables (built with g++
// and the address/undefined-behaviour sanitizers by tests/test_host_abi.py).
#include <algorithm>
#include <cassert>
#include <cstdio>
#include <random>
#include <vector>

#include "../../speculative_decoding_rl_amd/csrc/kvpool.h"

using namespace er;

int main() {
  BlockPool pool;
  pool.init(64);
  assert(pool.total() == 64 && pool.free_count() == 64);

  // reserve / truncate / release round trip keeps every block accounted for
  std::mt19937 rng(7);
  std::vector<BlockTable> seqs(8);
  for (int it = 0; it < 2000; ++it) {
    BlockTable& t = seqs[rng() % seqs.size()];
    const int op = (int)(rng() % 3);
    if (op == 0) {
      const int64_t want = (int64_t)(rng() % 200);
      const int64_t before = pool.free_count();
      const size_t had = t.blocks.size();
      const bool ok = t.reserve(pool, want);
      if (ok) {
        assert((int64_t)t.blocks.size() * KV_BLOCK >= want);
      } else {
        assert(pool.free_count() == before && t.blocks.size() == had);  // all-or-nothing
      }
    } else if (op == 1) {
      const int64_t keep = (int64_t)(rng() % 120);
      const size_t had = t.blocks.size();
      t.truncate(pool, keep);
      assert(t.blocks.size() == std::min(had, (size_t)BlockTable::blocks_for(keep)));
    } else {
      t.release(pool);
      assert(t.blocks.empty());
    }
    int64_t held = 0;
    for (auto& s : seqs) held += (int64_t)s.blocks.size();
    assert(held + pool.free_count() == pool.total());
  }
  for (auto& s : seqs) s.release(pool);
  assert(pool.free_count() == pool.total());

  // shared prefix blocks: refcounted, freed by the last user
  BlockTable a, b;
  assert(a.reserve(pool, 40));  // 3 blocks
  for (int i = 0; i < 2; ++i) {  // b shares a's two full prompt blocks
    pool.incref(a.blocks[(size_t)i]);
    b.blocks.push_back(a.blocks[(size_t)i]);
  }
  assert(pool.refcount(a.blocks[0]) == 2 && pool.refcount(a.blocks[2]) == 1);
  const int64_t f0 = pool.free_count();
  a.release(pool);
  assert(pool.free_count() == f0 + 1);  // only a's private third block returns
  b.release(pool);
  assert(pool.free_count() == pool.total());
  std::printf("kvpool ok\n");
  return 0;
}

// Paged KV block pool and per-sequence block tables (host only).
//
// The drafter and the target share one KV store (EfficientRollout "关键模块"
// item 1): a sequence owns one block table; the drafter writes provisional
// entries for draft positions, the verify pass overwrites them with the
// target's, and after the acceptance decision the tail past the committed
// length is released (the discarded drafts of the TLT notes, section 1).
// Blocks hold 16 positions; prompt blocks can be shared between sequences of
// one group (reference-counted, released when the last user goes).
#pragma once

#include <cstdint>
#include <vector>

namespace er {

constexpr int KV_BLOCK = 16;

class BlockPool {
 public:
  void init(int64_t n) {
    free_.clear();
    free_.reserve((size_t)n);
    for (int64_t b = n - 1; b >= 0; --b) free_.push_back((int32_t)b);
    ref_.assign((size_t)n, 0);
    total_ = n;
  }
  int64_t total() const { return total_; }
  int64_t free_count() const { return (int64_t)free_.size(); }
  // Returns the block id, or -1 when the pool is empty.
  int32_t alloc() {
    if (free_.empty()) return -1;
    const int32_t b = free_.back();
    free_.pop_back();
    ref_[(size_t)b] = 1;
    return b;
  }
  void incref(int32_t b) { ++ref_[(size_t)b]; }
  void decref(int32_t b) {
    if (--ref_[(size_t)b] == 0) free_.push_back(b);
  }
  int32_t refcount(int32_t b) const { return ref_[(size_t)b]; }

 private:
  std::vector<int32_t> free_;
  std::vector<int32_t> ref_;
  int64_t total_ = 0;
};

struct BlockTable {
  std::vector<int32_t> blocks;

  static int64_t blocks_for(int64_t positions) { return (positions + KV_BLOCK - 1) / KV_BLOCK; }

  // Make room for positions [0, len).  On failure releases what this call took
  // and returns false (the table is unchanged).
  bool reserve(BlockPool& pool, int64_t len) {
    const size_t need = (size_t)blocks_for(len);
    const size_t had = blocks.size();
    while (blocks.size() < need) {
      const int32_t b = pool.alloc();
      if (b < 0) {
        while (blocks.size() > had) {
          pool.decref(blocks.back());
          blocks.pop_back();
        }
        return false;
      }
      blocks.push_back(b);
    }
    return true;
  }
  // Keep positions [0, len); release whole blocks past them.
  void truncate(BlockPool& pool, int64_t len) {
    const size_t keep = (size_t)blocks_for(len);
    while (blocks.size() > keep) {
      pool.decref(blocks.back());
      blocks.pop_back();
    }
  }
  void release(BlockPool& pool) { truncate(pool, 0); }
};

}  // namespace er

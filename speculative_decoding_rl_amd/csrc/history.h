// Model-free history drafter: drafts copied from earlier rollouts (host only).
//
// History Tree Dynamic RL page, section 1 (drafts taken from responses of
// earlier rollouts, high-reward pieces first, for later rollouts of the same
// prompt) and section 3.3 (a fixed-prefix history cache per prompt plus a
// global fallback; candidates at a fixed prefix length; reward-first updates).
// The rule in full: a record is one earlier rollout (prompt, response,
// reward); position i of its response is keyed by the L tokens before it in
// prompt + response and offers the record's tokens from i on.  Each prompt has
// its own map and one global map holds every prompt's keys; a key keeps the
// candidate of the highest reward, among equal rewards the one recorded last.
// A sequence's draft: the key of its last L tokens (prompt + generated, the
// last generated token being the unverified one) in its prompt's map, else in
// the global map; the first gamma tokens of that candidate, or none.
#pragma once

#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

namespace er {

struct TokenSeqHash {
  size_t operator()(const std::vector<int32_t>& v) const {
    uint64_t h = 1469598103934665603ull;  // FNV-1a over the 32-bit words
    for (int32_t t : v) {
      h ^= (uint32_t)t;
      h *= 1099511628211ull;
    }
    return (size_t)h;
  }
};

class HistoryCache {
 public:
  explicit HistoryCache(int prefix_len) : L_(prefix_len) {}
  int prefix_len() const { return L_; }
  int64_t records() const { return (int64_t)recs_.size(); }

  void add(const int32_t* prompt, int P, const int32_t* resp, int R, float reward) {
    const int32_t rid = (int32_t)recs_.size();
    std::vector<int32_t> toks(prompt, prompt + P);
    toks.insert(toks.end(), resp, resp + R);
    recs_.push_back(std::move(toks));
    const std::vector<int32_t>& t = recs_.back();
    Map& mine = per_prompt_[std::vector<int32_t>(prompt, prompt + P)];
    std::vector<int32_t> key((size_t)L_);
    for (int i = P; i < P + R; ++i) {
      if (i < L_) continue;
      std::memcpy(key.data(), t.data() + (i - L_), sizeof(int32_t) * (size_t)L_);
      put(mine, key, Entry{rid, i, reward});
      put(global_, key, Entry{rid, i, reward});
    }
  }

  // Draft for a sequence whose prompt is prompt[0, P) and whose tokens are
  // ctx[0, C) (prompt + generated); writes up to gamma tokens, returns the count.
  int propose(const int32_t* prompt, int P, const int32_t* ctx, int C, int gamma, int32_t* out) const {
    if (gamma < 1 || C < L_) return 0;
    const std::vector<int32_t> key(ctx + (C - L_), ctx + C);
    const Entry* e = nullptr;
    auto pm = per_prompt_.find(std::vector<int32_t>(prompt, prompt + P));
    if (pm != per_prompt_.end()) {
      auto it = pm->second.find(key);
      if (it != pm->second.end()) e = &it->second;
    }
    if (!e) {
      auto it = global_.find(key);
      if (it != global_.end()) e = &it->second;
    }
    if (!e) return 0;
    const std::vector<int32_t>& t = recs_[(size_t)e->rec];
    int k = 0;
    for (; k < gamma && e->pos + k < (int)t.size(); ++k) out[k] = t[(size_t)(e->pos + k)];
    return k;
  }

 private:
  struct Entry {
    int32_t rec, pos;
    float reward;
  };
  using Map = std::unordered_map<std::vector<int32_t>, Entry, TokenSeqHash>;
  static void put(Map& m, const std::vector<int32_t>& key, const Entry& e) {
    auto it = m.find(key);
    if (it == m.end()) m.emplace(key, e);
    else if (e.reward >= it->second.reward) it->second = e;
  }
  int L_;
  std::vector<std::vector<int32_t>> recs_;
  std::unordered_map<std::vector<int32_t>, Map, TokenSeqHash> per_prompt_;
  Map global_;
};

}  // namespace er

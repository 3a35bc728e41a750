// Tiered expert residency (host side).  The routed experts of a layer stay in host memory in
// the store's block layout (the cold tier: the pages keep them on SSD and read one fixed-
// stride block per expert, TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍
// 구조", and the Swiftlet article, section "같은 모델을 왜 이렇게 적은 메모리로 돌릴 수
// 있나"), and a fixed number of device slots caches the blocks in use.  Replacement is LFU
// with recency: the pages name a 16-slot LFU cache per layer and an LFU + recency pool.
//
// Policy of one call (the distinct experts named by the call, in order of first appearance):
//   - an expert already in a slot is a hit: its use count grows by one, its last use is now;
//   - a missing expert takes an empty slot (lowest index first), else evicts the slot not
//     used by this call with the smallest use count, then the oldest last use, then the lowest
//     index; it starts with count 1 and last use now (one block copy fills the slot).
// Counts live with the slot (an evicted expert starts again from 1); there is no ageing.
#pragma once
#include <cstdint>
#include <vector>

#include "bounds.h"

namespace qmoe {

struct CachePlan {
  std::vector<int32_t> slot_of;                // per id of the call
  std::vector<int32_t> fill_expert, fill_slot;  // blocks to copy
};

class ExpertCachePolicy {
 public:
  ExpertCachePolicy(int n_experts, int n_slots)
      : where_(n_experts, -1), slot_expert_(n_slots, -1), count_(n_slots, 0), last_(n_slots, 0),
        used_(n_slots, 0) {}

  int slots() const { return (int)slot_expert_.size(); }
  int64_t hits() const { return hits_; }
  int64_t misses() const { return misses_; }

  // Returns false (and changes nothing) when the call names an id outside [0, E) or more
  // distinct experts than there are slots.
  bool plan(const int32_t *ids, int n, CachePlan &p) {
    const int E = (int)where_.size();
    std::vector<int32_t> distinct;
    std::vector<char> seen(E, 0);
    for (int i = 0; i < n; ++i) {
      const int e = ids[i];
      if (e < 0 || e >= E) return false;
      if (!seen[e]) { seen[e] = 1; distinct.push_back(e); }
    }
    if ((int)distinct.size() > slots()) return false;
    ++tick_;
    for (int s = 0; s < slots(); ++s) used_[s] = 0;
    p.fill_expert.clear();
    p.fill_slot.clear();
    for (int e : distinct)                       // hits first: they pin their slots
      if (where_[e] >= 0) {
        const int s = where_[e];
        ++count_[s];
        last_[s] = tick_;
        used_[s] = 1;
        ++hits_;
      }
    for (int e : distinct) {
      if (where_[e] >= 0) continue;
      int v = -1;
      for (int s = 0; s < slots() && v < 0; ++s)
        if (slot_expert_[s] < 0) v = s;
      if (v < 0)
        for (int s = 0; s < slots(); ++s) {
          if (used_[s]) continue;
          if (v < 0 || count_[s] < count_[v] || (count_[s] == count_[v] && last_[s] < last_[v]))
            v = s;
        }
      if (slot_expert_[v] >= 0) where_[slot_expert_[v]] = -1;
      slot_expert_[v] = e;
      where_[e] = v;
      count_[v] = 1;
      last_[v] = tick_;
      used_[v] = 1;
      ++misses_;
      p.fill_expert.push_back(e);
      p.fill_slot.push_back(v);
    }
    p.slot_of.resize(n);
    for (int i = 0; i < n; ++i) p.slot_of[i] = where_[ids[i]];
    check(ids, n, p);
    return true;
  }

  // Invariants after a plan (bounds assertions of the debug build): slots and experts map one
  // to one, every id of the call has a slot that holds it, and each copy fills a distinct slot
  // with an expert of the call.
  void check(const int32_t *ids, int n, const CachePlan &p) const {
#ifdef QMOE_DEBUG_BOUNDS
    const int E = (int)where_.size();
    for (int e = 0; e < E; ++e) {
      const int s = where_[e];
      QMOE_BOUNDS(s >= -1 && s < slots());
      if (s >= 0) QMOE_BOUNDS(slot_expert_[s] == e);
    }
    for (int s = 0; s < slots(); ++s) {
      const int e = slot_expert_[s];
      QMOE_BOUNDS(e >= -1 && e < E);
      if (e >= 0) QMOE_BOUNDS(where_[e] == s && count_[s] >= 1 && last_[s] <= tick_);
    }
    for (int i = 0; i < n; ++i) {
      const int s = p.slot_of[i];
      QMOE_BOUNDS(s >= 0 && s < slots() && slot_expert_[s] == ids[i] && used_[s]);
    }
    QMOE_BOUNDS(p.fill_expert.size() == p.fill_slot.size());
    std::vector<char> filled(slots(), 0);
    for (size_t j = 0; j < p.fill_slot.size(); ++j) {
      const int s = p.fill_slot[j];
      QMOE_BOUNDS(s >= 0 && s < slots() && !filled[s] && slot_expert_[s] == p.fill_expert[j]);
      filled[s] = 1;
    }
#else
    (void)ids;
    (void)n;
    (void)p;
#endif
  }

 private:
  std::vector<int32_t> where_, slot_expert_;
  std::vector<int64_t> count_, last_;
  std::vector<char> used_;
  int64_t tick_ = 0, hits_ = 0, misses_ = 0;
};

}  // namespace qmoe

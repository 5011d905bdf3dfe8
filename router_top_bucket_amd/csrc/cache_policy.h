// Which device-cache slot each expert of a call uses, and which experts are
// kept there for later calls ("Run Kimi 3.1 locally on one GPU", sections
// "One GPU, three storage tiers" and "A drafter that leaves the answer
// unchanged").  The pages report that LRU alone misses every time once a
// block needs more experts than fit, and that admitting only experts with
// a minimum number of rows in the block helps; admit_min_rows is that
// threshold.  Host code only.
//
// Slots (numbered from 0 here; the device pool adds its own offset):
//   [0, n_transient)                       transient: hold an expert for one
//                                          call only, never looked up again
//   [n_transient, n_transient + n_cache)   cached: looked up by (layer, expert)
// A call plans its experts in the order given:
//   1. every cached expert is a hit and is stamped with the call's tick;
//   2. each other expert is a miss: when admission is on (admit_min_rows > 0)
//      and fewer than admit_min_rows rows of the call use it, it takes the
//      next transient slot (while there is one); otherwise it is admitted into
//      a cached slot: the lowest free one, else the least recently used one
//      (lowest slot on equal ticks) that no expert of this call holds.
// plan() fails (returns -1, nothing changed) when the call's experts do not
// fit: more misses than free-or-evictable cached slots plus transient slots.
#pragma once
#include <stdint.h>

#include <vector>

namespace moe {

class CachePolicy {
 public:
  CachePolicy(int n_layers, int n_routed, int n_cache, int n_transient, int admit_min_rows)
      : n_layers_(n_layers), n_routed_(n_routed), n_cache_(n_cache), n_transient_(n_transient),
        admit_(admit_min_rows), slot_of_((size_t)n_layers * n_routed, -1), key_of_(n_cache, -1),
        last_(n_cache, 0), pin_(n_cache, 0) {}

  int n_cache() const { return n_cache_; }
  int n_transient() const { return n_transient_; }

  // experts[0..n) routed expert ids of one call (distinct), rows[i] = rows of
  // the call using experts[i].  Writes slot[i] and hit[i] (1 hit, 0 miss) and
  // admitted[i] (1 if the miss now stays cached).  Returns the miss count.
  int plan(int layer, const int32_t *experts, const int32_t *rows, int n, int32_t *slot, int32_t *hit,
           int32_t *admitted) {
    if (layer < 0 || layer >= n_layers_) return -1;
    // feasibility first, so a failed plan changes nothing
    int misses = 0, bypass = 0, held = 0;
    for (int i = 0; i < n; ++i) {
      const int e = experts[i];
      if (e < 0 || e >= n_routed_) return -1;
      if (slot_of_[key(layer, e)] >= 0) {
        ++held;
      } else {
        ++misses;
        if (admit_ > 0 && rows[i] < admit_ && bypass < n_transient_) ++bypass;
      }
    }
    // admitted misses need cached slots not held by this call's hits; those
    // beyond them take the transient slots the bypassed ones left
    if (misses - bypass > (n_cache_ - held) + (n_transient_ - bypass)) return -1;
    ++tick_;
    for (int i = 0; i < n; ++i) {
      slot[i] = -1;
      hit[i] = admitted[i] = 0;
      const int s = slot_of_[key(layer, experts[i])];
      if (s >= 0) {
        last_[s] = pin_[s] = tick_;
        slot[i] = n_transient_ + s;
        hit[i] = 1;
      }
    }
    int nt = 0;  // transient slots taken
    if (admit_ > 0)
      for (int i = 0; i < n; ++i)
        if (!hit[i] && rows[i] < admit_ && nt < n_transient_) slot[i] = nt++;
    for (int i = 0; i < n; ++i) {
      if (slot[i] >= 0) continue;
      const int v = victim();
      if (v < 0) {  // every cached slot is held by this call
        slot[i] = nt++;
        continue;
      }
      const size_t k = key(layer, experts[i]);
      if (key_of_[v] >= 0) slot_of_[key_of_[v]] = -1;
      key_of_[v] = (int64_t)k;
      slot_of_[k] = v;
      last_[v] = pin_[v] = tick_;
      slot[i] = n_transient_ + v;
      admitted[i] = 1;
    }
    return misses;
  }

  // Drops (layer, expert) from the cache if it is there (its slot becomes
  // free): for an expert whose upload could not be enqueued.
  void forget(int layer, int e) {
    if (layer < 0 || layer >= n_layers_ || e < 0 || e >= n_routed_) return;
    const size_t k = key(layer, e);
    const int s = slot_of_[k];
    if (s < 0) return;
    slot_of_[k] = -1;
    key_of_[s] = -1;
  }

 private:
  size_t key(int layer, int e) const { return (size_t)layer * n_routed_ + e; }
  // lowest free cached slot, else the least recently used one not held by
  // this call (lowest index on equal ticks); -1 if every slot is held
  int victim() const {
    int best = -1;
    for (int s = 0; s < n_cache_; ++s) {
      if (key_of_[s] < 0) return s;
      if (pin_[s] == tick_) continue;
      if (best < 0 || last_[s] < last_[best]) best = s;
    }
    return best;
  }

  int n_layers_, n_routed_, n_cache_, n_transient_, admit_;
  std::vector<int32_t> slot_of_;  // (layer, expert) -> cached slot or -1
  std::vector<int64_t> key_of_;   // cached slot -> key or -1
  std::vector<int64_t> last_;     // cached slot -> tick of its last use
  std::vector<int64_t> pin_;      // cached slot -> tick of the call holding it
  int64_t tick_ = 0;
};

}  // namespace moe

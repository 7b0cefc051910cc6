// Host bookkeeping of a model's KV blocks and of the content-addressed prefix cache over them.
// Plain C++ (no HIP): the library applies the table writes and block copies it returns on the
// device, and a CPU test drives the same code against a brute-force model of block contents.
//
// Kipp Roadmap, status v0.0.3: pooled sessions share one model-owned slab through a pool of
// 32-token blocks addressed by content, published when a session finishes and verified by
// comparing tokens. Here a block is
//   free     - holds nothing;
//   private  - mapped by exactly one session, which writes it;
//   cached   - holds the K/V of one whole 32-position block of a known token prefix; any number
//              of sessions map it read-only; when none does it stays cached (a later prefix can
//              still hit it) but may be evicted, least recently used first, when a block is
//              needed and none is free.
// The key of a cached block is its 32 token ids and its parent: the cached block holding the
// previous 32 positions of the same prefix (none for the first block), at the generation the
// parent had when the child was published. A chain of keys therefore names the whole prefix. A
// parent that is evicted and published again gets a new generation, which leaves its old
// children unreachable until they are evicted in turn. Lookups compare the stored tokens and
// parent, so a hash collision cannot produce a false hit.
#pragma once

#include <cstdint>
#include <cstring>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

namespace gqa {

class KvPool {
 public:
  static constexpr int kTok = 32;
  enum State : uint8_t { FREE = 0, PRIVATE = 1, CACHED = 2 };

  explicit KvPool(int n) : b_(n) {
    for (int i = 0; i < n; ++i) free_.insert(i);
  }

  int size() const { return (int)b_.size(); }
  int free_count() const { return (int)free_.size(); }
  int evictable_count() const { return (int)lru_.size(); }
  int available() const { return free_count() + evictable_count(); }   // blocks a caller can take
  int cached_count() const { return cached_; }
  State state(int i) const { return b_[i].st; }
  int refs(int i) const { return b_[i].ref; }
  uint64_t lookups = 0, hits = 0, evictions = 0;

  // Take block i as private: it must be free or cached and unmapped. False otherwise.
  bool take(int i) {
    if (i < 0 || i >= size()) return false;
    Blk& x = b_[i];
    if (x.st == CACHED && x.ref == 0) {
      drop_cached(i);
      ++evictions;
    } else if (x.st != FREE) {
      return false;
    }
    free_.erase(i);
    x.st = PRIVATE;
    x.ref = 1;
    return true;
  }

  // The lowest-numbered free block, else the least recently used unmapped cached block, taken
  // as private; -1 if neither exists.
  int take_any() {
    int i = -1;
    if (!free_.empty()) {
      i = *free_.begin();
    } else if (!lru_.empty()) {
      i = lru_.begin()->second;
    } else {
      return -1;
    }
    take(i);
    return i;
  }

  // Drop one mapping of block i: a private block becomes free; a cached block stays cached and
  // becomes evictable when its last mapping goes.
  void unref(int i) {
    Blk& x = b_[i];
    if (x.st == PRIVATE) {
      x.st = FREE;
      x.ref = 0;
      free_.insert(i);
    } else if (x.st == CACHED && x.ref > 0) {
      if (--x.ref == 0) {
        x.stamp = ++clock_;
        lru_.insert({x.stamp, i});
      }
    }
  }

  // The cached block holding toks[0..32) after `parent` (-1: the first block of a prefix),
  // mapped once more; -1 if none.
  int acquire(int parent, const int32_t* toks) {
    ++lookups;
    const int i = find(parent, toks);
    if (i < 0) return -1;
    ++hits;
    Blk& x = b_[i];
    if (x.ref == 0) lru_.erase({x.stamp, i});
    ++x.ref;
    x.stamp = ++clock_;
    return i;
  }

  // Publish private block i, which holds toks[0..32) after `parent` (a cached block, or -1): it
  // becomes cached and stays mapped by its owner. If an equal block is already cached, i stays
  // private and that block is returned (not mapped), so the caller's chain continues from it.
  int publish(int i, int parent, const int32_t* toks) {
    if (b_[i].st != PRIVATE) return -1;
    if (parent >= 0 && b_[parent].st != CACHED) return -1;
    const int dup = find(parent, toks);
    if (dup >= 0) return dup;
    Blk& x = b_[i];
    x.st = CACHED;
    x.gen = ++gen_;
    x.parent = parent;
    x.pgen = parent >= 0 ? b_[parent].gen : 0;
    std::memcpy(x.toks, toks, sizeof(x.toks));
    x.key = key(parent, x.pgen, toks);
    x.stamp = ++clock_;
    index_.insert({x.key, i});
    ++cached_;
    return i;
  }

  // Consistency of the free set, the eviction order and the index with the block states
  // (for tests).
  bool consistent() const {
    int nfree = 0, nlru = 0, ncached = 0;
    for (int i = 0; i < size(); ++i) {
      const Blk& x = b_[i];
      const bool in_free = free_.count(i) != 0, in_lru = lru_.count({x.stamp, i}) != 0;
      if (in_free != (x.st == FREE)) return false;
      if (x.st == FREE && x.ref != 0) return false;
      if (x.st == PRIVATE && x.ref != 1) return false;
      if (x.st == CACHED) {
        ++ncached;
        if (in_lru != (x.ref == 0)) return false;
        bool indexed = false;
        auto r = index_.equal_range(x.key);
        for (auto it = r.first; it != r.second; ++it) indexed |= it->second == i;
        if (!indexed) return false;
      }
      nfree += in_free;
      nlru += in_lru;
    }
    return nfree == free_count() && nlru == evictable_count() && ncached == cached_ &&
           (int)index_.size() == cached_;
  }

 private:
  struct Blk {
    State st = FREE;
    int32_t ref = 0;
    uint32_t gen = 0;      // generation of this block's current cached content
    int32_t parent = -1;
    uint32_t pgen = 0;     // parent's generation when this block was published
    uint64_t key = 0;
    uint64_t stamp = 0;    // last use, for the eviction order
    int32_t toks[kTok] = {};
  };

  static uint64_t mix(uint64_t z) {   // SplitMix64 finaliser (Steele, Lea and Flood, 2014)
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  static uint64_t key(int parent, uint32_t pgen, const int32_t* toks) {
    uint64_t h = mix(((uint64_t)(uint32_t)parent << 32) | pgen);
    for (int t = 0; t < kTok; ++t) h = mix(h ^ (uint32_t)toks[t]);
    return h;
  }
  int find(int parent, const int32_t* toks) const {
    const uint32_t pgen = parent >= 0 ? b_[parent].gen : 0;
    if (parent >= 0 && b_[parent].st != CACHED) return -1;
    auto r = index_.equal_range(key(parent, pgen, toks));
    for (auto it = r.first; it != r.second; ++it) {
      const Blk& x = b_[it->second];
      if (x.st == CACHED && x.parent == parent && x.pgen == pgen && std::memcmp(x.toks, toks, sizeof(x.toks)) == 0)
        return it->second;
    }
    return -1;
  }
  // Remove unmapped cached block i from the index and the eviction order; it becomes free.
  void drop_cached(int i) {
    Blk& x = b_[i];
    lru_.erase({x.stamp, i});
    auto r = index_.equal_range(x.key);
    for (auto it = r.first; it != r.second; ++it)
      if (it->second == i) {
        index_.erase(it);
        break;
      }
    --cached_;
    x.st = FREE;
    x.ref = 0;
    free_.insert(i);
  }

  std::vector<Blk> b_;
  std::set<int> free_;
  std::set<std::pair<uint64_t, int>> lru_;        // (last use, block) of unmapped cached blocks
  std::unordered_multimap<uint64_t, int> index_;  // key -> cached block
  uint64_t clock_ = 0;
  uint32_t gen_ = 0;
  int cached_ = 0;
};

// One pooled session's block list over a KvPool. Blocks are mapped on demand: a block index is
// allocated when a position in it is first written; a prefix evaluation first maps the cached
// blocks matching its leading whole blocks of ids. Writing into a cached block replaces it with a
// private copy (copy on write) when positions before the write in that block must be kept, or
// with a fresh private block otherwise. The device side applies `TableWrite`s to the session's
// table and `BlockCopy`s to every layer's K and V pools, in order, before the evaluation.
struct TableWrite {
  int32_t idx, val;
};
struct BlockCopy {
  int32_t src, dst;
};

class PooledSeq {
 public:
  static constexpr int kTok = KvPool::kTok;
  PooledSeq(KvPool& pool, int max_pos)
      : pool_(&pool), blocks((max_pos + kTok - 1) / kTok, -1), toks(max_pos, -1) {}

  std::vector<int32_t> blocks;   // physical block per block index, -1 if unmapped
  std::vector<int32_t> toks;     // token id per position, -1 if not known on the host

  // At position 0: map the cached blocks that hold ids' leading whole blocks, keeping at least
  // one id to evaluate (blocks still mapped at those indices are dropped). Returns the number of
  // positions mapped (a multiple of 32).
  int map_prefix(const int32_t* ids, int n, std::vector<TableWrite>& tw) {
    int parent = -1, k = 0;
    for (int j = 0; j < (n - 1) / kTok; ++j) {
      const int b = pool_->acquire(parent, ids + j * kTok);
      if (b < 0) break;
      if (blocks[j] >= 0) pool_->unref(blocks[j]);   // left mapped by a truncation to 0
      blocks[j] = b;
      tw.push_back({j, b});
      parent = b;
      ++k;
    }
    record(0, ids, k * kTok);
    return k * kTok;
  }

  // Make every block covering positions [p0, p1) mapped and private. False, with nothing
  // changed, if the pool has too few blocks.
  bool prepare_write(int p0, int p1, std::vector<TableWrite>& tw, std::vector<BlockCopy>& cp) {
    if (p1 <= p0) return true;
    const int j0 = p0 / kTok, j1 = (p1 - 1) / kTok;
    int need = 0;
    for (int j = j0; j <= j1; ++j)
      need += blocks[j] < 0 || pool_->state(blocks[j]) == KvPool::CACHED;
    if (need > pool_->available()) return false;
    for (int j = j0; j <= j1; ++j) {
      const int b = blocks[j];
      if (b >= 0 && pool_->state(b) != KvPool::CACHED) continue;
      const int nb = pool_->take_any();   // cannot fail (counted above) nor evict b (mapped)
      if (b >= 0) {
        if (j * kTok < p0) cp.push_back({b, nb});   // keep positions [32 j, p0)
        pool_->unref(b);
      }
      blocks[j] = nb;
      tw.push_back({j, nb});
    }
    return true;
  }

  // Token ids of positions [p0, p0 + n) (ids == nullptr: not known on the host).
  void record(int p0, const int32_t* ids, int n) {
    for (int i = 0; i < n; ++i) toks[p0 + i] = ids ? ids[i] : -1;
  }

  // Publish the whole blocks below position `pos` whose tokens are all known, in order, stopping
  // at the first that is not.
  void publish(int pos) {
    int parent = -1;
    for (int j = 0; j < pos / kTok; ++j) {
      const int b = blocks[j];
      if (b < 0) return;
      if (pool_->state(b) == KvPool::CACHED) {
        parent = b;
        continue;
      }
      for (int t = 0; t < kTok; ++t)
        if (toks[j * kTok + t] < 0) return;
      const int r = pool_->publish(b, parent, &toks[j * kTok]);
      if (r < 0) return;
      parent = r;
    }
  }

  // End of a request: publish, then drop every mapping.
  void finish(int pos) {
    publish(pos);
    release();
  }

  void release() {
    for (int32_t& b : blocks)
      if (b >= 0) {
        pool_->unref(b);
        b = -1;
      }
  }

 private:
  KvPool* pool_;
};

}  // namespace gqa

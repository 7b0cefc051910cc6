// Randomised check of the KV block pool and of pooled sessions' block lists against a
// brute-force model of what every block holds. Each written slot stores a fingerprint of the
// whole token prefix ending at its position; a session is correct when every position below its
// own position reads its own prefix's fingerprint through its block list, whichever blocks it
// shares, copies or gets from the cache. Built with g++ and the host sanitizers by
// tests/test_kv_pool_host.py; exit status 0 and a final "ok" line mean every check passed.
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <random>
#include <vector>

#include "kv_pool.h"

using gqa::BlockCopy;
using gqa::KvPool;
using gqa::PooledSeq;
using gqa::TableWrite;

static uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                       \
    }                                                                     \
  } while (0)

constexpr int kT = 32;

struct Sim {
  int nblocks;
  KvPool pool;
  std::vector<std::vector<uint64_t>> content;   // [block][slot] fingerprint, 0 = never written
  explicit Sim(int n) : nblocks(n), pool(n), content(n, std::vector<uint64_t>(kT, 0)) {}
};

struct Sess {
  std::unique_ptr<PooledSeq> seq;
  int pos = 0, max_pos = 0;
  std::vector<int32_t> tok;     // true ids, known or not to the pool
  std::vector<uint64_t> fp;     // fingerprint of tok[0..p]
  std::vector<int32_t> table;   // the device copy of the block list (0 where unmapped)
};

static void set_tokens(Sess& s, int p0, const std::vector<int32_t>& ids) {
  for (size_t i = 0; i < ids.size(); ++i) {
    const int p = p0 + (int)i;
    s.tok[p] = ids[i];
    s.fp[p] = mix((p ? s.fp[p - 1] : 0x5eedull) ^ (uint64_t)(uint32_t)ids[i]);
  }
}

static void apply(Sim& sim, Sess& s, const std::vector<TableWrite>& tw, const std::vector<BlockCopy>& cp) {
  for (const BlockCopy& c : cp) sim.content[c.dst] = sim.content[c.src];
  for (const TableWrite& w : tw) s.table[w.idx] = w.val;
}

static void write_positions(Sim& sim, Sess& s, int p0, int p1) {
  for (int p = p0; p < p1; ++p) sim.content[s.table[p / kT]][p % kT] = s.fp[p];
}

// Every session reads its own prefix; reference counts match the sessions' mappings.
static void check_all(Sim& sim, std::vector<Sess>& ss) {
  CHECK(sim.pool.consistent());
  std::vector<int> maps(sim.nblocks, 0);
  for (Sess& s : ss) {
    if (!s.seq) continue;
    for (size_t j = 0; j < s.seq->blocks.size(); ++j) {
      const int b = s.seq->blocks[j];
      if (b < 0) continue;
      ++maps[b];
      CHECK(s.table[j] == b);
    }
    for (int p = 0; p < s.pos; ++p) {
      const int b = s.seq->blocks[p / kT];
      CHECK(b >= 0);
      CHECK(sim.content[b][p % kT] == s.fp[p]);
    }
  }
  for (int b = 0; b < sim.nblocks; ++b) {
    switch (sim.pool.state(b)) {
      case KvPool::FREE: CHECK(maps[b] == 0); break;
      case KvPool::PRIVATE: CHECK(maps[b] == 1); break;
      case KvPool::CACHED: CHECK(maps[b] == sim.pool.refs(b)); break;
    }
  }
}

int main(int argc, char** argv) {
  const int steps = argc > 1 ? std::atoi(argv[1]) : 200000;
  std::mt19937_64 rng(20251202);
  auto rnd = [&](int n) { return (int)(rng() % (uint64_t)n); };
  Sim sim(28);
  std::vector<Sess> ss(4);
  // three base prompts; prompts are their prefixes, some with one token changed
  std::vector<std::vector<int32_t>> base(3, std::vector<int32_t>(200));
  for (auto& b : base)
    for (auto& t : b) t = rnd(50);
  long hits = 0, copies = 0, ooms = 0, publishes = 0, prefills = 0;
  for (int step = 0; step < steps; ++step) {
    const int si = rnd((int)ss.size());
    Sess& s = ss[si];
    const int op = rnd(10);
    if (!s.seq) {   // create
      s.max_pos = 256;
      s.seq.reset(new PooledSeq(sim.pool, s.max_pos));
      s.pos = 0;
      s.tok.assign(s.max_pos, -1);
      s.fp.assign(s.max_pos, 0);
      s.table.assign(s.max_pos / kT, 0);
    } else if (op <= 2) {   // prefill a prompt (at position 0 the cache is consulted)
      const auto& b = base[rnd(3)];
      std::vector<int32_t> ids(b.begin(), b.begin() + 1 + rnd(200));
      if (rnd(3) == 0) ids[rnd((int)ids.size())] = 50 + rnd(5);
      if (s.pos + (int)ids.size() > s.max_pos) continue;
      std::vector<TableWrite> tw;
      std::vector<BlockCopy> cp;
      int reuse = 0;
      const std::vector<int32_t> before = s.seq->blocks;
      if (s.pos == 0) {
        reuse = s.seq->map_prefix(ids.data(), (int)ids.size(), tw);
        CHECK(reuse % kT == 0 && reuse < (int)ids.size());
        set_tokens(s, 0, ids);
        apply(sim, s, tw, {});
        for (int p = 0; p < reuse; ++p) CHECK(sim.content[s.seq->blocks[p / kT]][p % kT] == s.fp[p]);   // a hit holds this prefix
        hits += reuse / kT;
        tw.clear();
      }
      const int p0 = s.pos + reuse, p1 = s.pos + (int)ids.size();
      if (!s.seq->prepare_write(p0, p1, tw, cp)) {
        ++ooms;
        if (reuse) s.seq->release();
        for (size_t j = 0; j < before.size(); ++j) CHECK(reuse || s.seq->blocks[j] == before[j]);
        if (reuse) for (auto& t : s.table) t = 0;
        check_all(sim, ss);
        continue;
      }
      s.seq->record(p0, ids.data() + reuse, p1 - p0);
      set_tokens(s, s.pos, ids);
      copies += (long)cp.size();
      apply(sim, s, tw, cp);
      write_positions(sim, s, p0, p1);
      s.pos = p1;
      ++prefills;
    } else if (op <= 5) {   // append one token, known to the host or not
      if (s.pos + 1 > s.max_pos) continue;
      std::vector<TableWrite> tw;
      std::vector<BlockCopy> cp;
      const int32_t id = rnd(55);
      const bool known = rnd(4) != 0;
      const std::vector<int32_t> before = s.seq->blocks;
      if (!s.seq->prepare_write(s.pos, s.pos + 1, tw, cp)) {
        ++ooms;
        CHECK(s.seq->blocks == before);
        check_all(sim, ss);
        continue;
      }
      s.seq->record(s.pos, known ? &id : nullptr, 1);
      set_tokens(s, s.pos, {id});
      copies += (long)cp.size();
      apply(sim, s, tw, cp);
      write_positions(sim, s, s.pos, s.pos + 1);
      ++s.pos;
    } else if (op == 6) {   // truncate
      s.pos = rnd(s.pos + 1);
    } else if (op == 7) {
      s.seq->publish(s.pos);
      ++publishes;
    } else if (op == 8) {   // reset: the end of a request
      s.seq->finish(s.pos);
      s.pos = 0;
      ++publishes;
    } else {                // destroy
      s.seq->finish(s.pos);
      s.seq.reset();
      s.pos = 0;
      ++publishes;
    }
    check_all(sim, ss);
  }
  std::printf("steps %d prefills %ld hit_blocks %ld copies %ld ooms %ld publishes %ld lookups %llu evictions %llu\n",
              steps, prefills, hits, copies, ooms, publishes, (unsigned long long)sim.pool.lookups,
              (unsigned long long)sim.pool.evictions);
  CHECK(hits > 100 && copies > 10 && ooms > 10 && sim.pool.evictions > 10);
  std::printf("ok\n");
  return 0;
}

// Randomized run of the host pool for AddressSanitizer / UndefinedBehavior-
// Sanitizer builds (test infrastructure; built and run by
// tests/test_pool_sanitizers.py).  Every C entry point of the pool is driven
// with random but valid calls -- prefix-cached adds, appends (single and
// batched, including ones that must fail for lack of space), forks, frees,
// block caching, transfer pins, copy completion, table queries -- and the
// pool's own invariant check runs after every call.  A call that fails for
// lack of space must leave the whole pool unchanged.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <string>
#include <vector>

#include "internal.hpp"
#include "pagedattn.h"

// The error helpers live in the library's device-call layer, which this
// host-only program does not link.
namespace pa {
int fail(int code, const char*, ...) { return code; }
void clear_error() {}
}  // namespace pa

namespace {

int64_t g_no_space = 0, g_hits = 0, g_copies = 0;

[[noreturn]] void die(const char* what, int seed, int step) {
  std::fprintf(stderr, "pool_fuzz: %s (seed %d, step %d)\n", what, seed, step);
  std::exit(1);
}

struct Snapshot {
  std::vector<int32_t> free_order, refs;
  std::vector<int32_t> tables;
  std::vector<int32_t> lens;
  bool operator==(const Snapshot& o) const {
    return free_order == o.free_order && refs == o.refs && tables == o.tables && lens == o.lens;
  }
};

Snapshot snapshot(pa_pool* p, int32_t nb, const std::vector<int64_t>& live) {
  Snapshot s;
  int32_t n = 0;
  s.free_order.assign((size_t)nb, -1);
  pa_pool_free_order(p, s.free_order.data(), nb, &n);
  s.free_order.resize((size_t)n);
  for (int32_t b = 0; b < nb; ++b) {
    int32_t r = 0;
    pa_pool_refcount(p, b, &r);
    s.refs.push_back(r);
  }
  if (!live.empty()) {
    const int32_t W = nb;
    s.tables.assign(live.size() * (size_t)W, -1);
    s.lens.assign(live.size(), 0);
    pa_pool_block_table(p, live.data(), (int32_t)live.size(), s.tables.data(), W, s.lens.data());
  }
  return s;
}

void run(int seed) {
  std::mt19937_64 rng((uint64_t)seed * 7919 + 13);
  auto pick = [&](int64_t n) { return (int64_t)(rng() % (uint64_t)n); };
  const int32_t bs_choices[] = {1, 2, 4, 16};
  const int32_t B = bs_choices[pick(4)];
  const int32_t nb = 8 + (int32_t)pick(56);
  std::vector<int32_t> order((size_t)nb);
  for (int32_t i = 0; i < nb; ++i) order[(size_t)i] = i;
  for (int32_t i = nb - 1; i > 0; --i) std::swap(order[(size_t)i], order[(size_t)pick(i + 1)]);
  pa_pool* p = nullptr;
  if (pa_pool_create(nb, B, order.data(), &p) != PA_OK) die("create", seed, -1);

  std::vector<int64_t> live;
  std::map<int64_t, std::vector<int32_t>> toks, history;
  std::vector<int64_t> transfers;
  int64_t next_id = 0, next_t = 0;
  int32_t next_tok = 0;
  for (int step = 0; step < 1500; ++step) {
    const int64_t r = pick(100);
    if (live.empty() || r < 10) {
      // a new sequence, half the time with a prompt that repeats another's
      std::vector<int32_t> prompt;
      if (pick(2) && !history.empty()) {
        auto it = history.begin();
        std::advance(it, pick((int64_t)history.size()));
        prompt = it->second;
        prompt.resize((size_t)pick((int64_t)prompt.size() + 1));
      }
      int64_t hit = -1;
      if (pa_pool_add_seq_cached(p, next_id, prompt.data(), (int64_t)prompt.size(), &hit) != PA_OK)
        die("add_seq_cached", seed, step);
      if (hit < 0 || hit > (int64_t)prompt.size() || hit % B) die("hit length", seed, step);
      g_hits += hit > 0;
      prompt.resize((size_t)hit);
      toks[next_id] = prompt;
      live.push_back(next_id++);
    } else if (r < 45) {
      const int64_t s = live[(size_t)pick((int64_t)live.size())];
      const int32_t n = 1 + (int32_t)pick(3 * B + 5);
      std::vector<int64_t> slots((size_t)n);
      int32_t pair[2];
      const Snapshot before = snapshot(p, nb, live);
      const int rc = pa_pool_append(p, s, n, slots.data(), pair);
      if (rc == PA_ERR_NO_SPACE) {
        ++g_no_space;
        if (!(snapshot(p, nb, live) == before)) die("NO_SPACE changed the pool", seed, step);
      } else if (rc != PA_OK) {
        die("append", seed, step);
      } else {
        for (int64_t sl : slots)
          if (sl < 0 || sl >= (int64_t)nb * B) die("slot out of range", seed, step);
        g_copies += pair[0] >= 0;
        for (int32_t i = 0; i < n; ++i) toks[s].push_back(next_tok++);
      }
    } else if (r < 52) {
      std::vector<int64_t> ids;
      std::vector<int32_t> ns;
      for (int64_t s : live)
        if (pick(2)) {
          ids.push_back(s);
          ns.push_back(1 + (int32_t)pick(4));
        }
      int32_t total = 0;
      for (int32_t n : ns) total += n;
      std::vector<int64_t> slots((size_t)total + 1);
      std::vector<int32_t> pairs(2 * ids.size() + 2);
      int32_t done = -1;
      const int rc = pa_pool_append_batch(p, ids.data(), ns.data(), (int32_t)ids.size(), slots.data(),
                                          pairs.data(), &done);
      if (rc != PA_OK && rc != PA_ERR_NO_SPACE) die("append_batch", seed, step);
      for (int32_t i = 0; i < done; ++i)
        for (int32_t k = 0; k < ns[(size_t)i]; ++k) toks[ids[(size_t)i]].push_back(next_tok++);
    } else if (r < 58) {
      const int64_t s = live[(size_t)pick((int64_t)live.size())];
      if (pa_pool_fork(p, s, next_id) != PA_OK) die("fork", seed, step);
      toks[next_id] = toks[s];
      live.push_back(next_id++);
    } else if (r < 66) {
      const size_t i = (size_t)pick((int64_t)live.size());
      const int64_t s = live[i];
      if (pa_pool_free_seq(p, s) != PA_OK) die("free_seq", seed, step);
      history[s] = toks[s];
      toks.erase(s);
      live.erase(live.begin() + (long)i);
    } else if (r < 74) {
      const int64_t s = live[(size_t)pick((int64_t)live.size())];
      const auto& t = toks[s];
      const int64_t n = pick((int64_t)t.size() + 1);
      const int rc = pa_pool_cache_blocks(p, s, t.data(), n);
      if (rc != PA_OK && rc != PA_ERR_INVALID) die("cache_blocks", seed, step);
    } else if (r < 80) {
      const int64_t s = live[(size_t)pick((int64_t)live.size())];
      int32_t n = 0;
      std::vector<int32_t> blocks((size_t)nb);
      if (pa_pool_pin(p, s, next_t, blocks.data(), nb, &n) != PA_OK) die("pin", seed, step);
      transfers.push_back(next_t++);
    } else if (r < 85 && !transfers.empty()) {
      const size_t i = (size_t)pick((int64_t)transfers.size());
      if (pa_pool_unpin(p, transfers[i]) != PA_OK) die("unpin", seed, step);
      transfers.erase(transfers.begin() + (long)i);
    } else if (r < 93) {
      if (pa_pool_copies_done(p) != PA_OK) die("copies_done", seed, step);
    } else {
      // queries, including the kernel-block view and the statistics
      std::vector<int32_t> table(live.size() * (size_t)nb * B);
      std::vector<int32_t> lens(live.size());
      if (pa_pool_kernel_block_table(p, live.data(), (int32_t)live.size(), 1, table.data(), nb * B, lens.data()) !=
          PA_OK)
        die("kernel_block_table", seed, step);
      int64_t st[5];
      if (pa_pool_stats(p, st, 5) != PA_OK || st[0] + st[1] != nb || st[4] < 0) die("stats", seed, step);
      int32_t pins = 0, pend = 0, hashed = 0;
      uint64_t h = 0;
      for (int32_t b = 0; b < nb; ++b)
        if (pa_pool_block_state(p, b, &pins, &pend, &h, &hashed) != PA_OK) die("block_state", seed, step);
      // out-of-range and unknown ids are rejected, not undefined
      int32_t x = 0;
      if (pa_pool_refcount(p, nb, &x) != PA_ERR_INVALID) die("refcount range", seed, step);
      if (pa_pool_free_seq(p, next_id + 1000) != PA_ERR_INVALID) die("unknown free", seed, step);
    }
    if (pa_pool_check(p) != PA_OK) die("check", seed, step);
  }
  if (pa_pool_copies_done(p) != PA_OK) die("final copies_done", seed, -1);
  for (int64_t t : transfers)
    if (pa_pool_unpin(p, t) != PA_OK) die("final unpin", seed, -1);
  for (int64_t s : live)
    if (pa_pool_free_seq(p, s) != PA_OK) die("final free", seed, -1);
  if (pa_pool_check(p) != PA_OK) die("final check", seed, -1);
  int32_t nfree = 0;
  pa_pool_num_free(p, &nfree);
  if (nfree != nb) die("blocks leaked", seed, -1);
  pa_pool_destroy(p);
}

}  // namespace

int main(int argc, char** argv) {
  const int first = argc > 1 ? std::atoi(argv[1]) : 0;
  const int count = argc > 2 ? std::atoi(argv[2]) : 20;
  for (int seed = first; seed < first + count; ++seed) run(seed);
  std::printf("pool_fuzz ok: %d seeds, %lld prefix hits, %lld copies, %lld appends refused for space\n", count,
              (long long)g_hits, (long long)g_copies, (long long)g_no_space);
  return 0;
}

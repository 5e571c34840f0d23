// Host-only stress driver for the block allocator (built with g++ and the
// address / undefined-behaviour sanitizers by tests/test_allocator_asan.py).
// Random growth (plain and copy-on-write), forks, prefix publish / match and
// releases through the C ABI; after every step each block's reference count
// must equal the number of tables holding it, and held + free = pool.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pkv.h"

int main() {
  const int32_t nb = 64, nseq = 8, maxb = 64;
  std::mt19937 rng(12345);
  pkv_allocator* a = nullptr;
  if (pkv_allocator_create(nb, nullptr, &a) != PKV_OK) return 2;
  std::map<int32_t, std::vector<int32_t>> tables;
  std::vector<int32_t> row(maxb);
  for (int step = 0; step < 20000; ++step) {
    const int op = rng() % 100;
    const int32_t s = rng() % nseq;
    if (op < 45) {
      int64_t cur = 0;
      if (tables.count(s)) {
        // length is not tracked here: grow by a random amount past the table
        cur = (int64_t)tables[s].size() * PKV_BLOCK_SIZE;
      }
      const int64_t want = cur + (rng() % 40) - 20;
      int32_t n = 0, cs = -1, cd = -1;
      int32_t st = (op & 1) ? pkv_allocator_reserve_cow(a, s, want < 0 ? 0 : want, row.data(), maxb,
                                                        &n, &cs, &cd)
                            : pkv_allocator_reserve(a, s, want < 0 ? 0 : want, row.data(), maxb, &n);
      if (st == PKV_OK) tables[s].assign(row.begin(), row.begin() + n);
      else if (st != PKV_ERR_NO_BLOCKS && st != PKV_ERR_SHARED && st != PKV_ERR_INVALID_ARG) return 3;
    } else if (op < 60) {
      const int32_t d = rng() % nseq;
      if (pkv_allocator_fork(a, s, d) == PKV_OK) tables[d] = tables[s];
    } else if (op < 72) {
      std::vector<uint64_t> h(rng() % 6);
      for (auto& x : h) x = rng() % 8;
      (void)pkv_allocator_publish_prefix(a, s, h.data(), (int32_t)h.size());
    } else if (op < 84) {
      std::vector<uint64_t> h(rng() % 6);
      for (auto& x : h) x = rng() % 8;
      int32_t m = 0;
      if (pkv_allocator_match_prefix(a, s, h.data(), (int32_t)h.size(), &m) == PKV_OK) {
        // the matched blocks are the table now (rows of a matched sequence start empty)
        int32_t n = 0;
        if (pkv_allocator_reserve(a, s, (int64_t)m * PKV_BLOCK_SIZE, row.data(), maxb, &n) != PKV_OK)
          return 4;
        tables[s].assign(row.begin(), row.begin() + n);
      }
    } else {
      if (pkv_allocator_release(a, s) != PKV_OK) return 5;
      tables.erase(s);
    }
    std::vector<int32_t> held(nb, 0);
    for (auto& kv : tables)
      for (int32_t b : kv.second) {
        if (b < 0 || b >= nb) return 6;
        held[b] += 1;
      }
    int32_t free_n = 0, distinct = 0;
    if (pkv_allocator_free_count(a, &free_n) != PKV_OK) return 7;
    for (int32_t b = 0; b < nb; ++b) {
      int32_t r = -1;
      if (pkv_allocator_refcount(a, b, &r) != PKV_OK || r != held[b]) {
        std::fprintf(stderr, "step %d block %d refcount %d held %d\n", step, b, r, held[b]);
        return 8;
      }
      distinct += held[b] > 0;
    }
    if (distinct + free_n != nb) return 9;
  }
  pkv_allocator_destroy(a);
  std::printf("allocator stress ok\n");
  return 0;
}

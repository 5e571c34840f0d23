// Host block allocator: the on-demand allocate_block of [P1] "Long-context
// inference engineering truths 2026 ..." section 2.2.  A sequence's table grows
// by one physical block exactly when a token opens a new logical block, so
// each sequence wastes at most block_size - 1 slots (section 2.1's bound).
//
// Prefix sharing ([P2] "Unlocking long context ..." section 3.1: blocks of a
// shared prefix are reused, with copy-on-write): every block carries the
// number of tables that hold it, and returns to the free list when the last
// one lets go.  A sequence can be forked (the copy shares every block), and
// full blocks can be published under caller-computed prefix hashes so that a
// new sequence with the same prefix takes them over ([P1] section 5's prefix
// cache).  A write into a partly filled block that another table also holds
// first moves this sequence onto a fresh block, whose contents the caller
// copies (pkv_copy_blocks).
//
// KV offload ([P3] www.mhpn.cn/news/2466452 section 4.2; [P1] section 4): a
// host tier of num_host_slots block slots (a pinned host pool the caller owns
// and copies with pkv_copy_blocks).  The page table records, per logical
// block of a sequence, where it lives (a device block id, or PKV_OFFLOADED in
// the table and a host slot) and the last step that read it.  Offloading
// frees device blocks and hands out host slots; paging in (the prefetch)
// takes device blocks back; both return the copy pairs the caller issues, on
// whatever stream overlaps them with compute.
#include <algorithm>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_allocator {
  int32_t num_blocks;
  std::deque<int32_t> free_list;                    // front = next to hand out
  struct Seq {
    std::vector<int32_t> table;       // device id, or PKV_OFFLOADED
    std::vector<int32_t> host;        // host slot of an offloaded block, else -1
    std::vector<int64_t> last;        // last step that read the block, -1 never
    int64_t len = 0;
    void push(int32_t b) {
      table.push_back(b);
      host.push_back(-1);
      last.push_back(-1);
    }
    bool any_offloaded() const {
      return std::any_of(host.begin(), host.end(), [](int32_t h) { return h >= 0; });
    }
  };
  std::unordered_map<int32_t, Seq> seqs;
  std::vector<int32_t> refs;                        // tables holding each block
  std::unordered_map<uint64_t, int32_t> by_hash;    // published prefix blocks
  std::unordered_map<int32_t, uint64_t> hash_of;    // the inverse, for unpublishing
  int32_t num_host_slots = 0;
  std::deque<int32_t> host_free;                    // front = next to hand out

  // One table lets go of block b; the block is free again when none holds it.
  void drop(int32_t b) {
    if (--refs[b] > 0) return;
    auto h = hash_of.find(b);
    if (h != hash_of.end()) {
      by_hash.erase(h->second);
      hash_of.erase(h);
    }
    free_list.push_back(b);
  }
};

extern "C" int32_t pkv_allocator_create(int32_t num_blocks, const int32_t* free_order,
                                        pkv_allocator** out) {
  if (!out || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  auto* a = new (std::nothrow) pkv_allocator;
  if (!a) return PKV_ERR_INVALID_ARG;
  a->num_blocks = num_blocks;
  a->refs.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return PKV_ERR_INVALID_ARG;
      }
      seen[b] = 1;
      a->free_list.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_list.push_back(i);
  }
  *out = a;
  return PKV_OK;
}

namespace {

// Growth of `seq` to new_len, optionally with copy-on-write of a shared last
// block (cow != nullptr).  All-or-nothing.
int32_t grow(pkv_allocator* a, int32_t seq, int64_t new_len, int32_t* table_row,
             int32_t max_blocks, int32_t* num_blocks_out, int32_t* cow) {
  if (!a || seq < 0 || new_len < 0) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  const int64_t old_len = it == a->seqs.end() ? 0 : it->second.len;
  const int64_t have = it == a->seqs.end() ? 0 : (int64_t)it->second.table.size();
  if (new_len < old_len) return PKV_ERR_INVALID_ARG;
  const int64_t need = (new_len + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
  const int64_t add = need > have ? need - have : 0;
  if (table_row && need > max_blocks) return PKV_ERR_INVALID_ARG;
  const bool writes_tail = new_len > old_len && old_len % PKV_BLOCK_SIZE != 0;
  // the growth writes into the partly filled last block: in host memory?
  if (writes_tail && it->second.host.back() >= 0) return PKV_ERR_OFFLOADED;
  // ... or shared?
  const bool shared_tail = writes_tail && a->refs[it->second.table.back()] > 1;
  if (shared_tail && !cow) return PKV_ERR_SHARED;
  const int64_t take = add + (shared_tail ? 1 : 0);
  if (take > (int64_t)a->free_list.size()) return PKV_ERR_NO_BLOCKS;
  pkv_allocator::Seq& s = a->seqs[seq];
  if (cow) cow[0] = cow[1] = -1;
  if (shared_tail) {                      // the fresh block is taken first
    const int32_t old_b = s.table.back(), new_b = a->free_list.front();
    a->free_list.pop_front();
    a->refs[new_b] = 1;
    a->refs[old_b] -= 1;                  // still held by another table
    s.table.back() = new_b;
    cow[0] = old_b;
    cow[1] = new_b;
  }
  for (int64_t i = 0; i < add; ++i) {
    const int32_t b = a->free_list.front();
    a->free_list.pop_front();
    a->refs[b] = 1;
    s.push(b);
  }
  s.len = new_len;
  if (table_row)
    for (size_t j = 0; j < s.table.size(); ++j) table_row[j] = s.table[j];
  if (num_blocks_out) *num_blocks_out = (int32_t)s.table.size();
  return PKV_OK;
}

}  // namespace

extern "C" int32_t pkv_allocator_reserve(pkv_allocator* a, int32_t seq, int64_t new_len,
                                         int32_t* table_row, int32_t max_blocks,
                                         int32_t* num_blocks_out) {
  return grow(a, seq, new_len, table_row, max_blocks, num_blocks_out, nullptr);
}

extern "C" int32_t pkv_allocator_reserve_cow(pkv_allocator* a, int32_t seq, int64_t new_len,
                                             int32_t* table_row, int32_t max_blocks,
                                             int32_t* num_blocks_out, int32_t* cow_src,
                                             int32_t* cow_dst) {
  if (!cow_src || !cow_dst) return PKV_ERR_INVALID_ARG;
  int32_t cow[2] = {-1, -1};
  const int32_t st = grow(a, seq, new_len, table_row, max_blocks, num_blocks_out, cow);
  if (st == PKV_OK) {
    *cow_src = cow[0];
    *cow_dst = cow[1];
  }
  return st;
}

extern "C" int32_t pkv_allocator_fork(pkv_allocator* a, int32_t src_seq, int32_t dst_seq) {
  if (!a || src_seq < 0 || dst_seq < 0 || src_seq == dst_seq) return PKV_ERR_INVALID_ARG;
  auto src = a->seqs.find(src_seq);
  if (src == a->seqs.end() || a->seqs.count(dst_seq)) return PKV_ERR_INVALID_ARG;
  if (src->second.any_offloaded()) return PKV_ERR_OFFLOADED;   // host slots are not shared
  pkv_allocator::Seq copy = src->second;
  std::fill(copy.last.begin(), copy.last.end(), -1);
  for (int32_t b : copy.table) a->refs[b] += 1;
  a->seqs.emplace(dst_seq, std::move(copy));
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_publish_prefix(pkv_allocator* a, int32_t seq,
                                                const uint64_t* block_hashes, int32_t n_full) {
  if (!a || seq < 0 || n_full < 0 || (n_full > 0 && !block_hashes)) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return n_full == 0 ? PKV_OK : PKV_ERR_INVALID_ARG;
  if ((int64_t)n_full * PKV_BLOCK_SIZE > it->second.len) return PKV_ERR_INVALID_ARG;
  for (int32_t j = 0; j < n_full; ++j) {
    const int32_t b = it->second.table[j];
    if (b < 0) continue;                                  // in host memory: not shareable
    if (a->by_hash.count(block_hashes[j]) || a->hash_of.count(b)) continue;   // first one stays
    a->by_hash.emplace(block_hashes[j], b);
    a->hash_of.emplace(b, block_hashes[j]);
  }
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_match_prefix(pkv_allocator* a, int32_t seq,
                                              const uint64_t* block_hashes, int32_t n,
                                              int32_t* matched) {
  if (!a || seq < 0 || n < 0 || !matched || (n > 0 && !block_hashes)) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it != a->seqs.end() && (it->second.len != 0 || !it->second.table.empty()))
    return PKV_ERR_INVALID_ARG;
  pkv_allocator::Seq& s = a->seqs[seq];
  int32_t j = 0;
  for (; j < n; ++j) {
    auto h = a->by_hash.find(block_hashes[j]);
    if (h == a->by_hash.end()) break;
    a->refs[h->second] += 1;
    s.push(h->second);
  }
  s.len = (int64_t)j * PKV_BLOCK_SIZE;
  *matched = j;
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_refcount(const pkv_allocator* a, int32_t block, int32_t* out) {
  if (!a || !out || block < 0 || block >= a->num_blocks) return PKV_ERR_INVALID_ARG;
  *out = a->refs[block];
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_release(pkv_allocator* a, int32_t seq) {
  if (!a || seq < 0) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_OK;
  const pkv_allocator::Seq& s = it->second;
  for (size_t j = 0; j < s.table.size(); ++j) {
    if (s.host[j] >= 0) a->host_free.push_back(s.host[j]);
    else a->drop(s.table[j]);
  }
  a->seqs.erase(it);
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_waste_slots(const pkv_allocator* a, int32_t seq, int64_t* out) {
  if (!a || !out) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  *out = it == a->seqs.end()
             ? 0
             : (int64_t)it->second.table.size() * PKV_BLOCK_SIZE - it->second.len;
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_free_count(const pkv_allocator* a, int32_t* out) {
  if (!a || !out) return PKV_ERR_INVALID_ARG;
  *out = (int32_t)a->free_list.size();
  return PKV_OK;
}

// ---- host tier (KV offload) ----------------------------------------------

extern "C" int32_t pkv_allocator_set_host_slots(pkv_allocator* a, int32_t num_host_slots) {
  if (!a || num_host_slots < 0 || a->num_host_slots != 0) return PKV_ERR_INVALID_ARG;
  a->num_host_slots = num_host_slots;
  for (int32_t i = 0; i < num_host_slots; ++i) a->host_free.push_back(i);
  return PKV_OK;
}

namespace {

// The sequence and the clamped range [first, first + count) of its blocks.
pkv_allocator::Seq* range_of(pkv_allocator* a, int32_t seq, int32_t first, int32_t count,
                             int32_t* lo, int32_t* hi) {
  if (!a || seq < 0 || first < 0 || count < 0) return nullptr;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return nullptr;
  const int64_t n = (int64_t)it->second.table.size();
  *lo = (int32_t)std::min<int64_t>(first, n);
  *hi = (int32_t)std::min<int64_t>((int64_t)first + count, n);
  return &it->second;
}

}  // namespace

extern "C" int32_t pkv_allocator_offload(pkv_allocator* a, int32_t seq, int32_t first_block,
                                         int32_t count, int32_t* dev_ids, int32_t* host_slots,
                                         int32_t* n_pairs) {
  int32_t lo = 0, hi = 0;
  pkv_allocator::Seq* s = range_of(a, seq, first_block, count, &lo, &hi);
  if (!s || !n_pairs || (hi > lo && (!dev_ids || !host_slots))) return PKV_ERR_INVALID_ARG;
  int32_t moving = 0;
  for (int32_t j = lo; j < hi; ++j) {
    if (s->host[j] >= 0) continue;                      // already in host memory
    if (a->refs[s->table[j]] > 1) return PKV_ERR_SHARED;
    ++moving;
  }
  if (moving > (int32_t)a->host_free.size()) return PKV_ERR_NO_BLOCKS;
  int32_t k = 0;
  for (int32_t j = lo; j < hi; ++j) {
    if (s->host[j] >= 0) continue;
    const int32_t slot = a->host_free.front();
    a->host_free.pop_front();
    dev_ids[k] = s->table[j];
    host_slots[k] = slot;
    ++k;
    a->drop(s->table[j]);                               // back to the free list
    s->table[j] = PKV_OFFLOADED;
    s->host[j] = slot;
  }
  *n_pairs = k;
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_page_in(pkv_allocator* a, int32_t seq, int32_t first_block,
                                         int32_t count, int32_t* host_slots, int32_t* dev_ids,
                                         int32_t* n_pairs) {
  int32_t lo = 0, hi = 0;
  pkv_allocator::Seq* s = range_of(a, seq, first_block, count, &lo, &hi);
  if (!s || !n_pairs || (hi > lo && (!dev_ids || !host_slots))) return PKV_ERR_INVALID_ARG;
  int32_t moving = 0;
  for (int32_t j = lo; j < hi; ++j) moving += s->host[j] >= 0;
  if (moving > (int32_t)a->free_list.size()) return PKV_ERR_NO_BLOCKS;
  int32_t k = 0;
  for (int32_t j = lo; j < hi; ++j) {
    if (s->host[j] < 0) continue;
    const int32_t b = a->free_list.front();
    a->free_list.pop_front();
    a->refs[b] = 1;
    host_slots[k] = s->host[j];
    dev_ids[k] = b;
    ++k;
    a->host_free.push_back(s->host[j]);
    s->table[j] = b;
    s->host[j] = -1;
  }
  *n_pairs = k;
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_touch(pkv_allocator* a, int32_t seq, int32_t first_block,
                                       int32_t count, int64_t step) {
  int32_t lo = 0, hi = 0;
  pkv_allocator::Seq* s = range_of(a, seq, first_block, count, &lo, &hi);
  if (!s) return PKV_ERR_INVALID_ARG;
  for (int32_t j = lo; j < hi; ++j) s->last[j] = step;
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_block_state(const pkv_allocator* a, int32_t seq, int32_t block,
                                             int32_t* device_id, int32_t* host_slot,
                                             int64_t* last_access) {
  if (!a || !device_id || !host_slot || !last_access) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end() || block < 0 || block >= (int64_t)it->second.table.size())
    return PKV_ERR_INVALID_ARG;
  *device_id = it->second.table[block];
  *host_slot = it->second.host[block];
  *last_access = it->second.last[block];
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_table(const pkv_allocator* a, int32_t seq, int32_t* table_row,
                                       int32_t max_blocks, int32_t* num_blocks_out) {
  if (!a || !num_blocks_out || max_blocks < 0 || (max_blocks > 0 && !table_row))
    return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    *num_blocks_out = 0;
    return PKV_OK;
  }
  const std::vector<int32_t>& t = it->second.table;
  if ((int64_t)t.size() > max_blocks) return PKV_ERR_INVALID_ARG;
  std::copy(t.begin(), t.end(), table_row);
  *num_blocks_out = (int32_t)t.size();
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_host_free_count(const pkv_allocator* a, int32_t* out) {
  if (!a || !out) return PKV_ERR_INVALID_ARG;
  *out = (int32_t)a->host_free.size();
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_coldest(const pkv_allocator* a, int32_t max_n, int32_t* seqs,
                                         int32_t* blocks, int32_t* n) {
  if (!a || !n || max_n < 0 || (max_n > 0 && (!seqs || !blocks))) return PKV_ERR_INVALID_ARG;
  struct C {
    int64_t last;
    int32_t seq, block;
  };
  std::vector<C> cand;
  for (const auto& kv : a->seqs) {
    const pkv_allocator::Seq& s = kv.second;
    const int64_t full = s.len / PKV_BLOCK_SIZE;         // blocks no write will touch again
    for (int64_t j = 0; j < full && j < (int64_t)s.table.size(); ++j)
      if (s.host[j] < 0 && a->refs[s.table[j]] == 1) cand.push_back({s.last[j], kv.first, (int32_t)j});
  }
  const size_t k = std::min<size_t>(cand.size(), (size_t)max_n);
  std::partial_sort(cand.begin(), cand.begin() + k, cand.end(), [](const C& x, const C& y) {
    if (x.last != y.last) return x.last < y.last;
    if (x.seq != y.seq) return x.seq < y.seq;
    return x.block < y.block;
  });
  for (size_t i = 0; i < k; ++i) {
    seqs[i] = cand[i].seq;
    blocks[i] = cand[i].block;
  }
  *n = (int32_t)k;
  return PKV_OK;
}

extern "C" void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

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
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_allocator {
  int32_t num_blocks;
  std::deque<int32_t> free_list;                    // front = next to hand out
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
  };
  std::unordered_map<int32_t, Seq> seqs;
  std::vector<int32_t> refs;                        // tables holding each block
  std::unordered_map<uint64_t, int32_t> by_hash;    // published prefix blocks
  std::unordered_map<int32_t, uint64_t> hash_of;    // the inverse, for unpublishing

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
  // the growth writes into the partly filled last block: is it shared?
  const bool shared_tail = new_len > old_len && old_len % PKV_BLOCK_SIZE != 0 &&
                           a->refs[it->second.table.back()] > 1;
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
    s.table.push_back(b);
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
  pkv_allocator::Seq copy = src->second;
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
    s.table.push_back(h->second);
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
  for (int32_t b : it->second.table) a->drop(b);
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

extern "C" void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

// Host block allocator: the on-demand allocate_block of [P1] "Long-context
// inference engineering truths 2026 ..." section 2.2.  A sequence's table grows
// by one physical block exactly when a token opens a new logical block, so
// each sequence wastes at most block_size - 1 slots (section 2.1's bound).
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
};

extern "C" int32_t pkv_allocator_create(int32_t num_blocks, const int32_t* free_order,
                                        pkv_allocator** out) {
  if (!out || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  auto* a = new (std::nothrow) pkv_allocator;
  if (!a) return PKV_ERR_INVALID_ARG;
  a->num_blocks = num_blocks;
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

extern "C" int32_t pkv_allocator_reserve(pkv_allocator* a, int32_t seq, int64_t new_len,
                                         int32_t* table_row, int32_t max_blocks,
                                         int32_t* num_blocks_out) {
  if (!a || seq < 0 || new_len < 0) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  const int64_t old_len = it == a->seqs.end() ? 0 : it->second.len;
  const int64_t have = it == a->seqs.end() ? 0 : (int64_t)it->second.table.size();
  if (new_len < old_len) return PKV_ERR_INVALID_ARG;
  const int64_t need = (new_len + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
  const int64_t add = need > have ? need - have : 0;
  if (table_row && need > max_blocks) return PKV_ERR_INVALID_ARG;
  if (add > (int64_t)a->free_list.size()) return PKV_ERR_NO_BLOCKS;
  pkv_allocator::Seq& s = a->seqs[seq];
  for (int64_t i = 0; i < add; ++i) {
    s.table.push_back(a->free_list.front());
    a->free_list.pop_front();
  }
  s.len = new_len;
  if (table_row)
    for (size_t j = 0; j < s.table.size(); ++j) table_row[j] = s.table[j];
  if (num_blocks_out) *num_blocks_out = (int32_t)s.table.size();
  return PKV_OK;
}

extern "C" int32_t pkv_allocator_release(pkv_allocator* a, int32_t seq) {
  if (!a || seq < 0) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_OK;
  for (int32_t b : it->second.table) a->free_list.push_back(b);
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

// Host block manager: free list, per-block reference counts, per-sequence
// block tables and copy-on-write ("What is PagedAttention" (tecyfy), How it
// works; "pagedattention vllm" glossary, Memory Management > Block
// Allocation and Copy-on-Write Sharing > Reference Counting / Divergence
// Handling).  Deterministic policy: take blocks from the front of the free
// list, return freed blocks to its front in table order.
#include <deque>
#include <new>
#include <vector>

#include "pkv.h"

struct pkv_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;              // front = next block handed out
  std::vector<int32_t> refcount;              // per physical block
  std::vector<std::vector<int32_t>> tables;   // per sequence id
  std::vector<int32_t> length;                // per sequence id, -1 = absent
};

namespace {

bool seq_ok(const pkv_block_manager* bm, int32_t seq) {
  return bm && seq >= 0 && seq < (int32_t)bm->length.size();
}

bool live(const pkv_block_manager* bm, int32_t seq) {
  return seq_ok(bm, seq) && bm->length[seq] >= 0;
}

int32_t take(pkv_block_manager* bm) {
  const int32_t b = bm->free_list.front();
  bm->free_list.pop_front();
  bm->refcount[b] = 1;
  return b;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                                 const int32_t* free_order) {
  if (num_blocks < 0 || block_size <= 0 || max_seqs < 0) return nullptr;
  try {
    auto* bm = new pkv_block_manager;
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->refcount.assign(num_blocks, 0);
    bm->tables.resize(max_seqs);
    bm->length.assign(max_seqs, -1);
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order ? free_order[i] : i;
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return nullptr;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
    return bm;
  } catch (...) {
    return nullptr;
  }
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_seq(pkv_block_manager* bm, int32_t seq) {
  if (!bm) return PKV_ERR_NULL;
  if (!seq_ok(bm, seq) || bm->length[seq] >= 0) return PKV_ERR_STATE;
  bm->tables[seq].clear();
  bm->length[seq] = 0;
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t child) {
  if (!bm) return PKV_ERR_NULL;
  if (!live(bm, parent) || !seq_ok(bm, child) || bm->length[child] >= 0) return PKV_ERR_STATE;
  try {
    bm->tables[child] = bm->tables[parent];
  } catch (...) {
    return PKV_ERR_STATE;
  }
  bm->length[child] = bm->length[parent];
  for (int32_t b : bm->tables[child])
    if (b >= 0) ++bm->refcount[b];
  return PKV_OK;
}

int pkv_bm_fork_batch(pkv_block_manager* bm, const int32_t* parents, const int32_t* children,
                      int32_t n, int32_t* num_done) {
  if (!bm || !num_done || (n > 0 && (!parents || !children))) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int st = pkv_bm_fork(bm, parents[i], children[i]);
    if (st != PKV_OK) return st;
    *num_done = i + 1;
  }
  return PKV_OK;
}

int pkv_bm_free_batch(pkv_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* num_done) {
  if (!bm || !num_done || (n > 0 && !seqs)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int st = pkv_bm_free_seq(bm, seqs[i]);
    if (st != PKV_OK) return st;
    *num_done = i + 1;
  }
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int32_t seq, int32_t* slot, int32_t* cow_src,
                  int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PKV_ERR_NULL;
  if (!live(bm, seq)) return PKV_ERR_STATE;
  std::vector<int32_t>& table = bm->tables[seq];
  const int32_t t = bm->length[seq], B = bm->block_size;
  *cow_src = -1;
  *cow_dst = -1;
  if (t % B == 0) {
    if (bm->free_list.empty()) return PKV_ERR_NO_BLOCKS;
    try {
      table.reserve(table.size() + 1);
    } catch (...) {
      return PKV_ERR_STATE;
    }
    table.push_back(take(bm));
  } else {
    const int32_t last = table.back();
    if (bm->refcount[last] > 1) {
      if (bm->free_list.empty()) return PKV_ERR_NO_BLOCKS;
      const int32_t copy = take(bm);
      --bm->refcount[last];
      table.back() = copy;
      *cow_src = last;
      *cow_dst = copy;
    }
  }
  bm->length[seq] = t + 1;
  *slot = table[t / B] * B + t % B;
  return PKV_OK;
}

int pkv_bm_append_batch(pkv_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* slots,
                        int32_t* pairs, int32_t pairs_cap, int32_t* num_pairs, int32_t* num_done) {
  if (!bm || (n > 0 && (!seqs || !slots)) || !num_pairs || !num_done) return PKV_ERR_NULL;
  if (n < 0 || pairs_cap < 0 || (pairs_cap > 0 && !pairs)) return PKV_ERR_SHAPE;
  *num_pairs = 0;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    // A copy might be needed; refuse before changing anything if there is no room.
    if (*num_pairs >= pairs_cap && live(bm, seqs[i]) && bm->length[seqs[i]] % bm->block_size != 0 &&
        bm->refcount[bm->tables[seqs[i]].back()] > 1)
      return PKV_ERR_CAPACITY;
    int32_t src, dst;
    const int st = pkv_bm_append(bm, seqs[i], &slots[i], &src, &dst);
    if (st != PKV_OK) return st;
    if (src >= 0) {
      pairs[2 * *num_pairs] = src;
      pairs[2 * *num_pairs + 1] = dst;
      ++*num_pairs;
    }
    *num_done = i + 1;
  }
  return PKV_OK;
}

int pkv_bm_free_seq(pkv_block_manager* bm, int32_t seq) {
  if (!bm) return PKV_ERR_NULL;
  if (!live(bm, seq)) return PKV_ERR_STATE;
  for (int32_t b : bm->tables[seq])
    if (b >= 0 && bm->refcount[b] <= 0) return PKV_ERR_STATE;
  for (int32_t b : bm->tables[seq]) {
    if (b >= 0 && --bm->refcount[b] == 0) bm->free_list.push_front(b);
  }
  bm->tables[seq].clear();
  bm->length[seq] = -1;
  return PKV_OK;
}

int pkv_bm_move_seq(pkv_block_manager* from, pkv_block_manager* to, int32_t seq, int32_t* pairs,
                    int32_t pairs_cap, int32_t* num_pairs) {
  if (!from || !to || !num_pairs) return PKV_ERR_NULL;
  *num_pairs = 0;
  if (from == to || !live(from, seq) || !seq_ok(to, seq) || to->length[seq] >= 0 ||
      to->block_size != from->block_size)
    return PKV_ERR_STATE;
  const std::vector<int32_t>& table = from->tables[seq];
  int32_t n = 0;
  for (int32_t b : table) n += b >= 0;
  if (n > pairs_cap) return PKV_ERR_CAPACITY;
  if (n > 0 && !pairs) return PKV_ERR_NULL;
  if ((int64_t)to->free_list.size() < n) return PKV_ERR_NO_BLOCKS;
  for (int32_t b : table)
    if (b >= 0 && from->refcount[b] <= 0) return PKV_ERR_STATE;
  std::vector<int32_t> moved;
  try {
    moved.reserve(table.size());
  } catch (...) {
    return PKV_ERR_STATE;
  }
  for (int32_t b : table) {
    if (b < 0) {
      moved.push_back(-1);
      continue;
    }
    const int32_t nb = take(to);
    pairs[2 * *num_pairs] = b;
    pairs[2 * *num_pairs + 1] = nb;
    ++*num_pairs;
    moved.push_back(nb);
  }
  to->tables[seq].swap(moved);
  to->length[seq] = from->length[seq];
  return pkv_bm_free_seq(from, seq);
}

int pkv_bm_slide_window(pkv_block_manager* bm, int32_t seq, int32_t window) {
  if (!bm) return PKV_ERR_NULL;
  if (!live(bm, seq) || window <= 0) return PKV_ERR_STATE;
  auto& table = bm->tables[seq];
  const int64_t first = (int64_t)bm->length[seq] - window;   // first attended token
  const int64_t n = first > 0 ? first / bm->block_size : 0;  // blocks wholly before it
  for (int64_t i = 0; i < n && i < (int64_t)table.size(); ++i)
    if (table[i] >= 0 && bm->refcount[table[i]] <= 0) return PKV_ERR_STATE;
  int released = 0;
  for (int64_t i = 0; i < n && i < (int64_t)table.size(); ++i) {
    const int32_t b = table[i];
    if (b < 0) continue;
    if (--bm->refcount[b] == 0) bm->free_list.push_front(b);
    table[i] = -1;
    ++released;
  }
  return released;
}

int pkv_bm_seq_len(const pkv_block_manager* bm, int32_t seq) {
  if (!bm) return PKV_ERR_NULL;
  if (!live(bm, seq)) return PKV_ERR_STATE;
  return bm->length[seq];
}

int pkv_bm_block_table(const pkv_block_manager* bm, int32_t seq, int32_t* out, int32_t cap) {
  if (!bm) return PKV_ERR_NULL;
  if (!live(bm, seq)) return PKV_ERR_STATE;
  const auto& t = bm->tables[seq];
  if ((int32_t)t.size() > cap) return PKV_ERR_CAPACITY;
  if (!t.empty() && !out) return PKV_ERR_NULL;
  for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
  return (int)t.size();
}

int pkv_bm_export(const pkv_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* tables,
                  int32_t max_blocks, int32_t* context_lens) {
  if (!bm || (n > 0 && (!seqs || !tables || !context_lens))) return PKV_ERR_NULL;
  if (n < 0 || max_blocks < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    if (!live(bm, seqs[i])) return PKV_ERR_STATE;
    if ((int32_t)bm->tables[seqs[i]].size() > max_blocks) return PKV_ERR_CAPACITY;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& t = bm->tables[seqs[i]];
    int32_t* row = tables + (size_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < (int32_t)t.size() ? t[j] : -1;
    context_lens[i] = bm->length[seqs[i]];
  }
  return PKV_OK;
}

int pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (!bm) return PKV_ERR_NULL;
  if (block < 0 || block >= bm->num_blocks) return PKV_ERR_STATE;
  return bm->refcount[block];
}

int pkv_bm_num_free(const pkv_block_manager* bm) {
  if (!bm) return PKV_ERR_NULL;
  return (int)bm->free_list.size();
}

int pkv_bm_free_list(const pkv_block_manager* bm, int32_t* out, int32_t cap) {
  if (!bm) return PKV_ERR_NULL;
  if ((int32_t)bm->free_list.size() > cap) return PKV_ERR_CAPACITY;
  if (!bm->free_list.empty() && !out) return PKV_ERR_NULL;
  int32_t i = 0;
  for (int32_t b : bm->free_list) out[i++] = b;
  return i;
}

}  // extern "C"

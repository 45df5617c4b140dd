// Host block allocator: FIFO free list, refcounted fork/free, copy-on-write of a
// shared partially filled last block.
//
// [CB] "Batching Continuo y PagedAttention", section "PagedAttention: Memoria
// virtual para la KV cache": blocks are handed out on demand and returned when
// the request ends.  [IPX] iplexlaw.co.kr commentary, section "Dos respuestas a
// una entrada": refcounted sharing with copy-on-write of a block that still has
// room.  [OS] "PagedAttention: gestionar la KV cache como memoria de un sistema
// operativo", section "Cómo funciona por dentro": a block is requested only when
// the last one is full.
//
// Every public call validates first and mutates only after all checks pass, so a
// failing call leaves the allocator exactly as it was.
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

struct pkv_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  std::deque<int32_t> free_list;           // front = next block handed out
  std::vector<int32_t> ref;                // refcount per physical block
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 0;

  // Blocks taken by appending n tokens to s (one for every token that starts a
  // block, plus one for the copy when the first token lands in a shared block).
  int64_t needed(const Seq& s, int64_t n) const {
    if (n <= 0) return 0;
    const int64_t bs = block_size;
    int64_t need = 0;
    const int64_t off = s.len % bs;
    if (off != 0 && ref[s.table.back()] > 1) need += 1;
    // tokens at positions len .. len+n-1 that start a block
    const int64_t first = s.len, last = s.len + n - 1;
    const int64_t starts_upto_last = last / bs + 1;               // block starts <= last
    const int64_t starts_before_first = (first + bs - 1) / bs;    // block starts < first
    need += starts_upto_last - starts_before_first;
    return need;
  }

  // Caller has checked needed() <= free_list.size().
  void append(Seq& s, int64_t n, int64_t* slots, int32_t* cow, int32_t* n_cow) {
    const int64_t bs = block_size;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t off = s.len % bs;
      if (off == 0) {
        const int32_t b = free_list.front();
        free_list.pop_front();
        ref[b] = 1;
        s.table.push_back(b);
      } else if (ref[s.table.back()] > 1) {
        const int32_t old = s.table.back();
        const int32_t b = free_list.front();
        free_list.pop_front();
        ref[old] -= 1;
        ref[b] = 1;
        s.table.back() = b;
        cow[2 * *n_cow] = old;
        cow[2 * *n_cow + 1] = b;
        *n_cow += 1;
      }
      slots[i] = static_cast<int64_t>(s.table.back()) * bs + off;
      s.len += 1;
    }
  }
};

extern "C" {

pkv_status pkv_allocator_create(int32_t num_blocks, int32_t block_size,
                                const int32_t* initial_free_order, pkv_allocator** out) {
  if (!out) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_allocator_create: out is NULL");
  if (num_blocks <= 0) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_allocator_create: num_blocks must be > 0");
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return pkv_fail(PKV_ERR_UNSUPPORTED, "pkv_allocator_create: block_size must be 8, 16 or 32");
  std::vector<int32_t> order(num_blocks);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b])
        return pkv_fail(PKV_ERR_INVALID_ARG,
                        "pkv_allocator_create: initial_free_order is not a permutation of [0, num_blocks)");
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  pkv_allocator* a = new (std::nothrow) pkv_allocator();
  if (!a) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_allocator_create: out of host memory");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->free_list.assign(order.begin(), order.end());
  a->ref.assign(num_blocks, 0);
  *out = a;
  return PKV_OK;
}

void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

int32_t pkv_allocator_block_size(const pkv_allocator* a) { return a ? a->block_size : 0; }

int32_t pkv_allocator_num_free(const pkv_allocator* a) {
  return a ? static_cast<int32_t>(a->free_list.size()) : -1;
}

int32_t pkv_allocator_num_blocks(const pkv_allocator* a) { return a ? a->num_blocks : -1; }

pkv_status pkv_seq_create(pkv_allocator* a, int64_t* seq_id) {
  if (!a || !seq_id) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_create: NULL argument");
  const int64_t id = a->next_id++;
  a->seqs.emplace(id, pkv_allocator::Seq{});
  *seq_id = id;
  return PKV_OK;
}

pkv_status pkv_seq_blocks_needed(const pkv_allocator* a, int64_t seq, int32_t n_tokens,
                                 int32_t* needed) {
  if (!a || !needed) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_blocks_needed: NULL argument");
  if (n_tokens < 0) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_blocks_needed: n_tokens < 0");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_seq_blocks_needed: unknown sequence");
  *needed = static_cast<int32_t>(a->needed(it->second, n_tokens));
  return PKV_OK;
}

pkv_status pkv_seq_append_slots(pkv_allocator* a, int64_t seq, int32_t n_tokens,
                                int64_t* slots_out, int32_t* cow_src_dst_out,
                                int32_t* n_cow_out) {
  if (!a || !cow_src_dst_out || !n_cow_out || (n_tokens > 0 && !slots_out))
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_slots: NULL argument");
  if (n_tokens < 0) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_slots: n_tokens < 0");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_seq_append_slots: unknown sequence");
  if (a->needed(it->second, n_tokens) > static_cast<int64_t>(a->free_list.size()))
    return pkv_fail(PKV_ERR_OUT_OF_BLOCKS, "pkv_seq_append_slots: not enough free blocks");
  *n_cow_out = 0;
  a->append(it->second, n_tokens, slots_out, cow_src_dst_out, n_cow_out);
  return PKV_OK;
}

pkv_status pkv_seq_append_slots_batch(pkv_allocator* a, const int64_t* seqs,
                                      const int32_t* n_tokens, int32_t count,
                                      int64_t* slots_out, int32_t* cow_src_dst_out,
                                      int32_t* n_cow_out) {
  if (!a || !n_cow_out || count < 0 || (count > 0 && (!seqs || !n_tokens || !cow_src_dst_out)))
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_slots_batch: bad argument");
  std::vector<pkv_allocator::Seq*> ptrs(count);
  std::unordered_map<int64_t, int> dup;
  int64_t need = 0, total = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (n_tokens[i] < 0) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_slots_batch: n_tokens < 0");
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end())
      return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_seq_append_slots_batch: unknown sequence");
    if (dup[seqs[i]]++) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_slots_batch: repeated sequence");
    ptrs[i] = &it->second;
    need += a->needed(it->second, n_tokens[i]);
    total += n_tokens[i];
  }
  if (total > 0 && !slots_out) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_slots_batch: slots_out is NULL");
  if (need > static_cast<int64_t>(a->free_list.size()))
    return pkv_fail(PKV_ERR_OUT_OF_BLOCKS, "pkv_seq_append_slots_batch: not enough free blocks");
  *n_cow_out = 0;
  int64_t pos = 0;
  for (int32_t i = 0; i < count; ++i) {
    a->append(*ptrs[i], n_tokens[i], slots_out + pos, cow_src_dst_out, n_cow_out);
    pos += n_tokens[i];
  }
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_allocator* a, int64_t parent, int64_t* child) {
  if (!a || !child) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_fork: NULL argument");
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_seq_fork: unknown sequence");
  pkv_allocator::Seq copy = it->second;
  for (int32_t b : copy.table) a->ref[b] += 1;
  const int64_t id = a->next_id++;
  a->seqs.emplace(id, std::move(copy));
  *child = id;
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_allocator* a, int64_t seq) {
  if (!a) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_free: NULL allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_seq_free: unknown sequence");
  for (int32_t b : it->second.table) {
    if (--a->ref[b] == 0) a->free_list.push_back(b);
  }
  a->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_seq_block_table(const pkv_allocator* a, int64_t seq, int32_t* out, int32_t cap,
                               int32_t* n_blocks, int32_t* n_tokens) {
  if (!a || !n_blocks || !n_tokens || cap < 0 || (cap > 0 && !out))
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_block_table: bad argument");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_seq_block_table: unknown sequence");
  const auto& t = it->second.table;
  if (static_cast<int64_t>(t.size()) > cap)
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_seq_block_table: cap smaller than the table");
  for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
  *n_blocks = static_cast<int32_t>(t.size());
  *n_tokens = static_cast<int32_t>(it->second.len);
  return PKV_OK;
}

pkv_status pkv_block_tables(const pkv_allocator* a, const int64_t* seqs, int32_t count,
                            int32_t max_blocks, int32_t* tables_out, int32_t* context_lens_out) {
  if (!a || count < 0 || max_blocks < 0 ||
      (count > 0 && (!seqs || !context_lens_out || (max_blocks > 0 && !tables_out))))
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_block_tables: bad argument");
  for (int32_t i = 0; i < count; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_block_tables: unknown sequence");
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks)
      return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_block_tables: a table is longer than max_blocks");
  }
  for (int32_t i = 0; i < count; ++i) {
    const auto& s = a->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    size_t j = 0;
    for (; j < s.table.size(); ++j) row[j] = s.table[j];
    for (; j < static_cast<size_t>(max_blocks); ++j) row[j] = 0;
    context_lens_out[i] = static_cast<int32_t>(s.len);
  }
  return PKV_OK;
}

pkv_status pkv_block_refcount(const pkv_allocator* a, int32_t block, int32_t* rc) {
  if (!a || !rc) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_block_refcount: NULL argument");
  if (block < 0 || block >= a->num_blocks)
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_block_refcount: block out of range");
  *rc = a->ref[block];
  return PKV_OK;
}

}  // extern "C"

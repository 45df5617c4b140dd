// Internal declarations shared by the library's translation units.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/pkv.h"

// Record `msg` as this thread's last error and return `st`.
pkv_status pkv_fail(pkv_status st, const char* msg);
pkv_status pkv_failf(pkv_status st, const char* fmt, ...);

// Decode with every argument validated here (pkv_api.cpp): the body of
// pkv_attention_decode, _planned and _append (and of the allocation-free
// variant, pkv_noalloc.hip); `fn` names the entry point in error messages.
// With build_plan the plan is built at the start of the workspace.
pkv_status pkv_decode_impl(const char* fn, float* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale,
                           pkv_dtype dtype, const void* plan, size_t plan_bytes_given, void* workspace,
                           size_t workspace_bytes, bool build_plan, void* stream, const void* new_k = nullptr,
                           const void* new_v = nullptr, const int64_t* new_slots = nullptr);

// Kernel launchers (pkv_kernels.hip).  Arguments are already validated; each
// returns hipSuccess or the launch error as an int.
int pkv_launch_append(void* k_cache, void* v_cache, const void* k, const void* v,
                      const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                      int32_t num_kv_heads, int32_t row_bytes, int32_t block_size, void* stream);
int pkv_launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst, int32_t num_pairs,
                           int32_t num_blocks, int64_t block_bytes, void* stream);
// Block copies between two pools (device pointers; a host pool by its mapped address).
int pkv_launch_swap_blocks(void* k_dst, void* v_dst, int32_t dst_blocks, const void* k_src, const void* v_src,
                           int32_t src_blocks, const int32_t* src_dst, int32_t num_pairs, int64_t block_bytes,
                           void* stream);

// Context partitions of the decode work split (multiples of 16 tokens): 1024
// tokens for the VALU kernel; for the MFMA group kernels (which read Hq/Hkv
// heads per tile and gain more from long units than from balance) the largest
// of 4096, 2048 and 1024 tokens that still gives a full round of workgroups --
// four per CU on 256 CUs (the wide kernels: as many as fit, two for bf16 and
// three for float32) -- for the call's sizes, so that a batch of few
// sequences or KV heads gets shorter units instead of idle CUs.
constexpr int32_t kMinPartTokens = 1024;
constexpr int32_t kMaxPartTokens = 4096;
constexpr int64_t kMfmaRoundWorkgroups = 1024;
constexpr int32_t kMaxMfmaGroup = 16;
// Whether decode of these heads runs on a matrix-core group kernel -- bf16 or
// float32, two or more query heads per KV head (a group of more than 16 in
// 16-row slices), any block size (the matrix-core kernels walk contexts in
// 16-key tiles).
inline bool pkv_uses_mfma(int dtype, int32_t num_heads, int32_t num_kv_heads, int32_t block_size) {
  const int32_t group = num_heads / num_kv_heads;
  (void)block_size;
  return (dtype == PKV_BF16 || dtype == PKV_F32) && group >= 2;
}
// Whether a group of 17..64 query heads per KV head runs on a wide group
// kernel (one workgroup for all its 16-row slices, K/V staged once in LDS;
// two (bf16) or three (float32) workgroups per CU) instead of one workgroup
// per slice.
inline bool pkv_wide_group(int dtype, int32_t num_heads, int32_t num_kv_heads) {
  const int32_t group = num_heads / num_kv_heads;
  return (dtype == PKV_BF16 || dtype == PKV_F32) && group > kMaxMfmaGroup && group <= 4 * kMaxMfmaGroup;
}
inline int32_t pkv_part_tokens(int dtype, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t block_size, int32_t max_context_len) {
  if (!pkv_uses_mfma(dtype, num_heads, num_kv_heads, block_size)) return kMinPartTokens;
  // workgroups per partition of every context: (sequence, KV head), and per
  // 16-row slice unless the wide kernel takes all slices in one
  const bool wide = pkv_wide_group(dtype, num_heads, num_kv_heads);
  const int64_t groups = static_cast<int64_t>(num_seqs > 0 ? num_seqs : 0) * num_kv_heads *
                         (wide ? 1 : (num_heads / num_kv_heads + kMaxMfmaGroup - 1) / kMaxMfmaGroup);
  const int64_t round = wide ? (dtype == PKV_F32 ? 3 : 2) * kMfmaRoundWorkgroups / 4 : kMfmaRoundWorkgroups;
  for (int32_t p = kMaxPartTokens; p > kMinPartTokens; p /= 2) {
    const int64_t parts = (static_cast<int64_t>(max_context_len) + p - 1) / p;
    if (groups * (parts < 1 ? 1 : parts) >= round) return p;
  }
  return kMinPartTokens;
}

// Sizes of the decode plan and of the split-context partials.
namespace pkv_ws {
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
// Partial-result slots per (sequence, head): enough for the smallest partition.
inline int32_t num_partitions(int32_t max_context_len) {
  const int32_t np = (max_context_len + kMinPartTokens - 1) / kMinPartTokens;
  return np < 1 ? 1 : np;
}
// Header and (s, p) per unit: at most num_partitions per sequence, or one
// rowless unit.
constexpr size_t kPlanHdrWords = 8;
inline size_t plan_bytes(int32_t num_seqs, int32_t max_context_len) {
  return (kPlanHdrWords + 2 * static_cast<size_t>(num_seqs) * (num_partitions(max_context_len) + 1)) *
         sizeof(int32_t);
}
// Partials of the split contexts: (max, sum) pairs, accumulators, then one
// merge ticket (8 bytes) per (sequence, head).
inline size_t partial_acc_offset(int32_t num_seqs, int32_t num_heads, int32_t max_context_len) {
  const size_t units = static_cast<size_t>(num_seqs) * num_heads * num_partitions(max_context_len);
  return align256(units * 2 * sizeof(float));
}
inline size_t ticket_offset(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len) {
  const size_t units = static_cast<size_t>(num_seqs) * num_heads * num_partitions(max_context_len);
  return partial_acc_offset(num_seqs, num_heads, max_context_len) + align256(units * head_dim * sizeof(float));
}
inline size_t partial_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len) {
  if (num_partitions(max_context_len) <= 1) return 0;
  return ticket_offset(num_seqs, num_heads, head_dim, max_context_len) +
         static_cast<size_t>(num_seqs) * num_heads * sizeof(uint64_t);
}
}  // namespace pkv_ws

struct pkv_decode_args {
  float* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* plan; // unit list built by the plan kernel
  float* part_ml;      // [S][Hq][NP][2]  (running max in log2 units, sum)
  float* part_acc;     // [S][Hq][NP][d]
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_blocks;
  int32_t block_size;      // tokens per block: 8, 16 or 32
  int32_t max_context_len;
  int32_t num_partitions;  // NP = ceil(max_context_len / kMinPartTokens): partial slots per row
  int32_t part_tokens;     // tokens per partition for this launch
  float scale_log2;        // scale * log2(e)
  int dtype;               // pkv_dtype
  // Shared-prefix decode (null / 0 otherwise).  seq_start[s] (a multiple of 16)
  // is the first token of sequence s that its own plan units cover; tokens
  // before it belong to its group's shared-prefix units, which write partial
  // slots 0 .. ceil(seq_start[s] / prefix_part_tokens) - 1 of each row, so the
  // sequence's own units write the slots after those.
  const int32_t* seq_start;
  const int32_t* shared_plan;  // header + (first sequence, members, partition, prefix tokens) per unit
  int32_t prefix_part_tokens;
  // Decode with the step's cache write (null otherwise): sequence s's token
  // ctx-1 is new_k/new_v row s ([S][Hkv][d]); the decode kernels store it at
  // new_slots[s] and use it from there on the fly (-1: no new token).
  const void* new_k;
  const void* new_v;
  const int64_t* new_slots;
  // Partition merge inside the decode launch, set whenever a row can have
  // more than one partial.  One ticket per (sequence, head) row -- for the
  // MFMA group kernel per (sequence, KV head), at its first query head's row
  // (pkvd::ticket_arrive: (merge_epoch << 24) | units arrived); the unit that
  // arrives last merges the row and sets the word back to 0.  merge_epoch is
  // nonzero, below 2^40 and new for every call (the two launches of a
  // shared-prefix decode share one: a row's units in both count together).
  uint64_t* merge_tickets;
  uint64_t merge_epoch;
};
// Decode: the VALU kernel, or for query-head groups of 2 or more heads the
// MFMA group kernel (bf16: pkv_mfma.hip, float32: pkv_decode_f32.hip); split
// contexts are merged inside the launch.
int pkv_launch_decode(const pkv_decode_args& a, void* stream);
int pkv_launch_decode_group(const pkv_decode_args& a, void* stream);
int pkv_launch_decode_group_f32(const pkv_decode_args& a, void* stream);
int pkv_launch_plan(int32_t* plan, const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                    int32_t block_size, int32_t max_context_len, int32_t part_tokens, void* stream,
                    const int32_t* seq_start = nullptr);

// Shared-prefix decode (pkv_mfma.hip): one kernel plans the groups' common
// leading blocks (fills seq_start and the shared plan) and then the sequences'
// own units from those starts; then one launch decodes the shared units and
// one (pkv_launch_decode) the own units, on one merge epoch.  Tokens per
// shared-prefix partition:
constexpr int32_t kPrefixPartTokens = 1024;
int pkv_launch_shared_plans(const pkv_decode_args& a, const int32_t* group_start, int32_t num_groups,
                            int32_t* seq_start, int32_t* shared_plan, int32_t* plan, void* stream);
// The shared-prefix units on the matrix cores: bf16 pools (pkv_mfma.hip) and
// float32 pools (pkv_decode_f32.hip).  A row is merged by its last unit, in
// this launch or in the own units' launch after it.
int pkv_launch_shared_units(const pkv_decode_args& a, void* stream);
int pkv_launch_shared_units_f32(const pkv_decode_args& a, void* stream);

// Causal chunked-prefill attention (pkv_mfma.hip).
struct pkv_prefill_args {
  float* out;                     // [num_query_tokens][Hq][d]
  const void* q;                  // [num_query_tokens][Hq][d]
  const int32_t* query_start_loc; // [num_seqs + 1]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_query_tokens;
  int32_t max_query_len;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_blocks;
  int32_t block_size;             // 8, 16 or 32
  int32_t max_context_len;
  // The kernel exponentiates scores times scale_log2 > 0; the scale's sign
  // goes into the query: q_mode 0 uses q, 1 uses -q (scale < 0: the scores
  // scale * q.k = |scale| * (-q).k, exactly), 2 uses q = 0 (scale 0: every
  // visible key weighs the same).
  float scale_log2;
  int32_t q_mode;
};
// Query rows (token, head of a KV group) per prefill workgroup: the bf16
// kernel, and the float32 one.
constexpr int32_t kPrefillRowsPerWg = 128;
constexpr int32_t kPrefillF32RowsPerWg = 64;
int pkv_launch_prefill(const pkv_prefill_args& a, void* stream);
int pkv_launch_prefill_f32(const pkv_prefill_args& a, void* stream);

// C ABI entry points: argument validation, workspace layout and dispatch to the
// kernel launchers.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>

#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;


bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

pkv_status check_common(const char* fn, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        pkv_dtype dtype) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: block_size must be 8, 16 or 32 (got %d)", fn, block_size);
  if (head_dim != 64 && head_dim != 128)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn, head_dim);
  if (num_kv_heads <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_kv_heads must be > 0", fn);
  return PKV_OK;
}

pkv_status hip_status(const char* fn, int err) {
  if (err == hipSuccess) return PKV_OK;
  return pkv_failf(PKV_ERR_HIP, "%s: kernel launch failed: %s", fn,
                   hipGetErrorString(static_cast<hipError_t>(err)));
}

using pkv_ws::align256;
using pkv_ws::num_partitions;
using pkv_ws::kPlanHdrWords;
using pkv_ws::plan_bytes;
using pkv_ws::partial_bytes;

// Shared-prefix decode buffers.  The plan buffer holds the shared plan (a
// header, then 4 ints per shared unit), seq_start and the plan of the
// sequences' own units, in that order; the partial buffer holds the partials
// (prefix slots ahead of each sequence's own) and one merge ticket per
// (sequence, head).  The self-planning call puts the plan at the start of its
// workspace and the partials after it.
struct SharedLayout {
  int32_t prefix_slots, slots;
  size_t shared_plan, seq_start, plan, plan_total;   // within the plan buffer
  size_t part_ml, part_acc, tickets, part_total;     // within the partial buffer
  size_t total() const { return align256(plan_total) + part_total; }
};
SharedLayout shared_layout(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len) {
  SharedLayout l{};
  l.prefix_slots = (max_context_len + kPrefixPartTokens - 1) / kPrefixPartTokens;
  if (l.prefix_slots < 1) l.prefix_slots = 1;
  l.slots = l.prefix_slots + num_partitions(max_context_len);
  const size_t S = static_cast<size_t>(num_seqs);
  l.shared_plan = 0;
  l.seq_start = align256((kPlanHdrWords + 4 * S * l.prefix_slots) * sizeof(int32_t));
  l.plan = l.seq_start + align256(S * sizeof(int32_t));
  l.plan_total = l.plan + plan_bytes(num_seqs, max_context_len);
  const size_t units = S * num_heads * l.slots;
  l.part_ml = 0;
  l.part_acc = align256(units * 2 * sizeof(float));
  l.tickets = l.part_acc + align256(units * head_dim * sizeof(float));
  l.part_total = l.tickets + S * num_heads * sizeof(uint64_t);
  return l;
}

// Whether shared-prefix decode reads shared blocks on the matrix cores for
// these heads (bf16 or float32, 1..16 query heads per KV head, any supported
// block size); other shapes run plain decode.
bool shared_applies(pkv_dtype dtype, int32_t num_heads, int32_t num_kv_heads) {
  const int32_t group = num_kv_heads > 0 ? num_heads / num_kv_heads : 0;
  return (dtype == PKV_BF16 || dtype == PKV_F32) && group >= 1 && group <= kMaxMfmaGroup;
}

// The checks every shared-prefix call makes on its sizes.
pkv_status check_shared(const char* fn, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                        int32_t max_context_len, pkv_dtype dtype) {
  pkv_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_seqs < 0", fn);
  if (num_heads <= 0 || num_heads % num_kv_heads != 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                     fn, num_heads, num_kv_heads);
  if (num_blocks <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0", fn);
  if (max_blocks_per_seq <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: max_blocks_per_seq must be > 0", fn);
  if (max_context_len < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: max_context_len < 0", fn);
  const SharedLayout l = shared_layout(num_seqs, num_heads, head_dim, max_context_len);
  const int64_t grid = static_cast<int64_t>(num_seqs) * num_heads * (l.prefix_slots + num_partitions(max_context_len));
  if (grid > 0x7FFFFFFF || static_cast<int64_t>(num_seqs) * l.slots > 0x3FFFFFFF)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: launch grid too large", fn);
  return PKV_OK;
}

// The kernel arguments of a shared-prefix decode over a plan buffer and a
// partial buffer laid out by shared_layout.
pkv_decode_args shared_args(const SharedLayout& l, float* out, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                            float scale, pkv_dtype dtype, const char* plan, char* part) {
  pkv_decode_args a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.plan = reinterpret_cast<const int32_t*>(plan + l.plan);
  a.part_ml = part ? reinterpret_cast<float*>(part + l.part_ml) : nullptr;
  a.part_acc = part ? reinterpret_cast<float*>(part + l.part_acc) : nullptr;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_context_len = max_context_len;
  a.num_partitions = l.slots;
  a.part_tokens = pkv_part_tokens(dtype, num_seqs, num_heads, num_kv_heads, block_size, max_context_len);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dtype = dtype;
  a.seq_start = reinterpret_cast<const int32_t*>(plan + l.seq_start);
  a.shared_plan = reinterpret_cast<const int32_t*>(plan + l.shared_plan);
  a.prefix_part_tokens = kPrefixPartTokens;
  return a;
}
}  // namespace

// Merge-ticket epochs: 40-bit, nonzero, a new one for every decode launch.  The
// sequence starts at a random point so that a workspace holding another
// process's tickets cannot match.
static uint64_t next_merge_epoch() {
  static std::atomic<uint64_t> next{[] {
    std::random_device rd;
    const uint64_t t = static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count());
    return (static_cast<uint64_t>(rd()) << 32) ^ rd() ^ (t * 0x9E3779B97F4A7C15ull);
  }()};
  for (;;) {
    const uint64_t e = next.fetch_add(1, std::memory_order_relaxed) & 0xFFFFFFFFFFull;
    if (e != 0) return e;
  }
}

pkv_status pkv_fail(pkv_status st, const char* msg) {
  g_last_error = msg;
  return st;
}

pkv_status pkv_failf(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

pkv_status pkv_append(void* k_cache, void* v_cache, const void* k, const void* v,
                      const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_append";
  pkv_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_tokens < 0", fn);
  if (num_blocks <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0", fn);
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k || !v || !slot_mapping)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k) || !aligned16(v))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: cache and row pointers must be 16-byte aligned", fn);
  const int32_t row_bytes = head_dim * elem_bytes(dtype);
  return hip_status(fn, pkv_launch_append(k_cache, v_cache, k, v, slot_mapping, num_tokens,
                                          num_blocks, num_kv_heads, row_bytes, block_size, stream));
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst,
                           int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, pkv_dtype dtype,
                           void* stream) {
  const char* fn = "pkv_copy_blocks";
  pkv_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_pairs < 0", fn);
  if (num_blocks <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0", fn);
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: cache pointers must be 16-byte aligned", fn);
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  return hip_status(fn, pkv_launch_copy_blocks(k_cache, v_cache, src_dst, num_pairs, num_blocks,
                                               block_bytes, stream));
}

// Whether a kernel may dereference `p` as is: device (or managed) memory, or
// pinned host memory that the runtime maps at the same virtual address on the
// device.  Pageable host memory and pinned memory mapped elsewhere are refused.
static bool device_accessible(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) return true;
  if (attr.type == hipMemoryTypeHost) return attr.devicePointer && attr.devicePointer == attr.hostPointer;
  return false;
}

pkv_status pkv_swap_blocks(void* dst_k_cache, void* dst_v_cache, int32_t dst_num_blocks, const void* src_k_cache,
                           const void* src_v_cache, int32_t src_num_blocks, const int32_t* src_dst,
                           int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_swap_blocks";
  pkv_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_pairs < 0", fn);
  if (dst_num_blocks <= 0 || src_num_blocks <= 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: block counts must be > 0", fn);
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k_cache || !dst_v_cache || !src_k_cache || !src_v_cache || !src_dst)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(dst_k_cache) || !aligned16(dst_v_cache) || !aligned16(src_k_cache) || !aligned16(src_v_cache))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: pool pointers must be 16-byte aligned", fn);
  if (!device_accessible(dst_k_cache) || !device_accessible(dst_v_cache) || !device_accessible(src_k_cache) ||
      !device_accessible(src_v_cache))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: pools must be device memory or pinned host memory", fn);
  if (!device_accessible(src_dst))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: src_dst must be device memory or pinned host memory", fn);
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  return hip_status(fn, pkv_launch_swap_blocks(dst_k_cache, dst_v_cache, dst_num_blocks, src_k_cache, src_v_cache,
                                               src_num_blocks, src_dst, num_pairs, block_bytes, stream));
}

size_t pkv_decode_plan_bytes(int32_t num_seqs, int32_t max_context_len) {
  if (num_seqs <= 0 || max_context_len < 0) return 0;
  return plan_bytes(num_seqs, max_context_len);
}

pkv_status pkv_decode_plan(void* plan, size_t plan_bytes_given, const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t max_context_len, pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_decode_plan";
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: block_size must be 8, 16 or 32 (got %d)", fn, block_size);
  if (dtype != PKV_F32 && dtype != PKV_BF16) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads != 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn,
                     num_heads, num_kv_heads);
  if (num_seqs == 0) return PKV_OK;
  if (!plan || !context_lens) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (reinterpret_cast<uintptr_t>(plan) & 15u) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan must be 16-byte aligned", fn);
  if (static_cast<int64_t>(num_seqs) * (num_partitions(max_context_len) + 1) > 0x3FFFFFFF)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: too many work units", fn);
  const size_t need = plan_bytes(num_seqs, max_context_len);
  if (plan_bytes_given < need)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan buffer of %zu bytes is smaller than the %zu needed", fn,
                     plan_bytes_given, need);
  return hip_status(fn, pkv_launch_plan(static_cast<int32_t*>(plan), context_lens, num_seqs, max_blocks_per_seq,
                                        block_size, max_context_len,
                                        pkv_part_tokens(dtype, num_seqs, num_heads, num_kv_heads, block_size, max_context_len), stream));
}

size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                     int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  return align256(plan_bytes(num_seqs, max_context_len)) +
         partial_bytes(num_seqs, num_heads, head_dim, max_context_len);
}

}  // extern "C"

pkv_status pkv_decode_impl(const char* fn, float* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale,
                           pkv_dtype dtype, const void* plan, size_t plan_bytes_given, void* workspace,
                           size_t workspace_bytes, bool build_plan, void* stream, const void* new_k,
                           const void* new_v, const int64_t* new_slots) {
  pkv_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_seqs < 0", fn);
  if (num_heads <= 0 || num_heads % num_kv_heads != 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                     fn, num_heads, num_kv_heads);
  if (num_blocks <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0", fn);
  if (max_blocks_per_seq <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: max_blocks_per_seq must be > 0", fn);
  if (max_context_len < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: max_context_len < 0", fn);
  if (!std::isfinite(scale)) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: out, q and cache pointers must be 16-byte aligned", fn);
  if (new_slots && (!new_k || !new_v || !aligned16(new_k) || !aligned16(new_v)))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: k and v must be 16-byte aligned device pointers", fn);
  const int32_t np = num_partitions(max_context_len);
  const int64_t grid = static_cast<int64_t>(num_seqs) * num_heads * np;
  if (grid > 0x7FFFFFFF || static_cast<int64_t>(num_seqs) * (np + 1) > 0x3FFFFFFF)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: launch grid too large", fn);
  const int32_t part_tokens = pkv_part_tokens(dtype, num_seqs, num_heads, num_kv_heads, block_size, max_context_len);
  const size_t pb = plan_bytes(num_seqs, max_context_len);
  const size_t part = partial_bytes(num_seqs, num_heads, head_dim, max_context_len);
  const size_t need = (build_plan ? align256(pb) : 0) + part;
  if (workspace_bytes < need)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                     workspace_bytes, need);
  if (need > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace must be a 256-byte aligned device buffer", fn);
  char* ws = static_cast<char*>(workspace);
  if (build_plan) {
    plan = ws;
    ws += align256(pb);
    const int err = pkv_launch_plan(static_cast<int32_t*>(const_cast<void*>(plan)), context_lens, num_seqs,
                                    max_blocks_per_seq, block_size, max_context_len, part_tokens, stream);
    if (err) return hip_status(fn, err);
  } else {
    if (!plan) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan is NULL", fn);
    if (plan_bytes_given < pb)
      return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan of %zu bytes is smaller than the %zu these sizes need", fn,
                       plan_bytes_given, pb);
  }
  pkv_decode_args a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.plan = static_cast<const int32_t*>(plan);
  a.part_ml = part ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_acc = part ? reinterpret_cast<float*>(ws + pkv_ws::partial_acc_offset(num_seqs, num_heads, max_context_len))
                    : nullptr;
  if (part && part_tokens < max_context_len) {
    // a context can be split: its rows are merged inside the decode launch
    a.merge_tickets = reinterpret_cast<uint64_t*>(ws + pkv_ws::ticket_offset(num_seqs, num_heads, head_dim,
                                                                             max_context_len));
    a.merge_epoch = next_merge_epoch();
  }
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_context_len = max_context_len;
  a.num_partitions = np;
  a.part_tokens = part_tokens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dtype = dtype;
  a.new_k = new_k;
  a.new_v = new_v;
  a.new_slots = new_slots;
  return hip_status(fn, pkv_launch_decode(a, stream));
}

extern "C" {

pkv_status pkv_attention_decode_append(float* out, const void* q, const void* k, const void* v,
                                       const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_context_len, float scale, pkv_dtype dtype, const void* plan,
                                       size_t plan_bytes_given, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  const char* fn = "pkv_attention_decode_append";
  if (num_seqs > 0 && !slot_mapping) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: slot_mapping is NULL", fn);
  return pkv_decode_impl(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, dtype, plan,
                     plan_bytes_given, workspace, workspace_bytes, plan == nullptr, stream, k, v, slot_mapping);
}

pkv_status pkv_attention_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_context_len, float scale, pkv_dtype dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return pkv_decode_impl("pkv_attention_decode", out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, dtype, nullptr, 0, workspace, workspace_bytes, true, stream);
}

pkv_status pkv_attention_decode_planned(float* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, int32_t max_context_len, float scale,
                                        pkv_dtype dtype, const void* plan, size_t plan_bytes_given,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return pkv_decode_impl("pkv_attention_decode_planned", out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, dtype, plan, plan_bytes_given, workspace, workspace_bytes, false,
                     stream);
}

size_t pkv_attention_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                                   int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  const size_t plain = pkv_attention_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len);
  const size_t shared = shared_layout(num_seqs, num_heads, head_dim, max_context_len).total();
  return shared > plain ? shared : plain;
}

size_t pkv_decode_shared_plan_bytes(int32_t num_seqs, int32_t max_context_len) {
  if (num_seqs <= 0 || max_context_len < 0) return 0;
  return shared_layout(num_seqs, 1, 1, max_context_len).plan_total;
}

pkv_status pkv_decode_shared_plan(void* plan, size_t plan_bytes_given, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                  const int32_t* group_start, int32_t num_groups, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t block_size, int32_t max_context_len, pkv_dtype dtype,
                                  void* stream) {
  const char* fn = "pkv_decode_shared_plan";
  if (num_groups < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_groups < 0", fn);
  if (num_groups > num_seqs && num_seqs >= 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: more groups than sequences", fn);
  // head_dim does not enter the plan: any supported value passes the checks
  pkv_status st = check_shared(fn, num_seqs, num_heads, num_kv_heads, 128, block_size, 1, max_blocks_per_seq,
                               max_context_len, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!plan || !block_tables || !context_lens || (num_groups > 0 && !group_start))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (reinterpret_cast<uintptr_t>(plan) & 255u)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan must be 256-byte aligned", fn);
  const SharedLayout l = shared_layout(num_seqs, num_heads, 128, max_context_len);
  if (plan_bytes_given < l.plan_total)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan buffer of %zu bytes is smaller than the %zu needed", fn,
                     plan_bytes_given, l.plan_total);
  char* pb = static_cast<char*>(plan);
  if (!shared_applies(dtype, num_heads, num_kv_heads)) {
    // plain decode: only the own plan region is used
    return hip_status(fn, pkv_launch_plan(reinterpret_cast<int32_t*>(pb + l.plan), context_lens, num_seqs,
                                          max_blocks_per_seq, block_size, max_context_len,
                                          pkv_part_tokens(dtype, num_seqs, num_heads, num_kv_heads, block_size, max_context_len), stream));
  }
  const pkv_decode_args a = shared_args(l, nullptr, nullptr, nullptr, nullptr, block_tables, max_blocks_per_seq,
                                        context_lens, num_seqs, num_heads, num_kv_heads, 128, block_size, 1,
                                        max_context_len, 1.f, dtype, pb, nullptr);
  // (no groups: every sequence is decoded by its own units)
  return hip_status(fn, pkv_launch_shared_plans(a, num_groups > 0 ? group_start : nullptr, num_groups,
                                                reinterpret_cast<int32_t*>(pb + l.seq_start),
                                                reinterpret_cast<int32_t*>(pb + l.shared_plan),
                                                reinterpret_cast<int32_t*>(pb + l.plan), stream));
}

}  // extern "C"

// Shared-prefix decode from a plan buffer (built by pkv_decode_shared_plan, or
// just now into the workspace) and a partial buffer.  With num_groups == 0 or
// a shape the shared path does not cover the plan is a plain decode plan.
static pkv_status shared_decode(const char* fn, float* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_context_len, float scale, pkv_dtype dtype, const char* plan,
                                char* part, size_t part_bytes, bool plain, void* stream) {
  const SharedLayout l = shared_layout(num_seqs, num_heads, head_dim, max_context_len);
  if (plain)
    return pkv_decode_impl(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                           num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, dtype,
                           plan + l.plan, plan_bytes(num_seqs, max_context_len), part, part_bytes, false, stream);
  if (part_bytes < l.part_total)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                     part_bytes, l.part_total);
  pkv_decode_args a = shared_args(l, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                  num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                                  scale, dtype, plan, part);
  // split rows are merged inside the decode launch
  a.merge_tickets = reinterpret_cast<uint64_t*>(part + l.tickets);
  a.merge_epoch = next_merge_epoch();
  // the shared units, then every sequence's own units, on one epoch
  const int err = dtype == PKV_BF16 ? pkv_launch_shared_units(a, stream) : pkv_launch_shared_units_f32(a, stream);
  if (err) return hip_status(fn, err);
  return hip_status(fn, pkv_launch_decode(a, stream));
}

static pkv_status check_decode_pointers(const char* fn, float* out, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* block_tables,
                                        const int32_t* context_lens, float scale) {
  if (!std::isfinite(scale)) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: out, q and cache pointers must be 16-byte aligned", fn);
  return PKV_OK;
}

extern "C" {

pkv_status pkv_attention_decode_shared(float* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs, const int32_t* group_start,
                                       int32_t num_groups, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_context_len, float scale, pkv_dtype dtype, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_attention_decode_shared";
  if (num_groups < 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_groups < 0", fn);
  if (num_groups > 0 && num_seqs > 0 && !group_start) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: group_start is NULL", fn);
  // only the matrix-core kernels read a prefix for several sequences;
  // otherwise (or with no groups) this is plain decode
  if (!shared_applies(dtype, num_heads, num_kv_heads) || num_groups == 0 || num_seqs <= 0)
    return pkv_decode_impl(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                           num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, dtype,
                           nullptr, 0, workspace, workspace_bytes, true, stream);
  pkv_status st = check_shared(fn, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                               max_blocks_per_seq, max_context_len, dtype);
  if (st != PKV_OK) return st;
  if (num_groups > num_seqs) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: more groups than sequences", fn);
  st = check_decode_pointers(fn, out, q, k_cache, v_cache, block_tables, context_lens, scale);
  if (st != PKV_OK) return st;
  const SharedLayout l = shared_layout(num_seqs, num_heads, head_dim, max_context_len);
  if (workspace_bytes < l.total())
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                     workspace_bytes, l.total());
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace must be a 256-byte aligned device buffer", fn);
  char* ws = static_cast<char*>(workspace);
  const pkv_decode_args a = shared_args(l, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                        num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                        max_context_len, scale, dtype, ws, nullptr);
  const int err = pkv_launch_shared_plans(a, group_start, num_groups, reinterpret_cast<int32_t*>(ws + l.seq_start),
                                          reinterpret_cast<int32_t*>(ws + l.shared_plan),
                                          reinterpret_cast<int32_t*>(ws + l.plan), stream);
  if (err) return hip_status(fn, err);
  const size_t off = align256(l.plan_total);
  return shared_decode(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, dtype, ws,
                       ws + off, workspace_bytes - off, false, stream);
}

pkv_status pkv_attention_decode_shared_planned(float* out, const void* q, const void* k_cache, const void* v_cache,
                                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                               int32_t num_blocks, int32_t max_context_len, float scale,
                                               pkv_dtype dtype, const void* plan, size_t plan_bytes_given,
                                               void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_attention_decode_shared_planned";
  pkv_status st = check_shared(fn, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                               max_blocks_per_seq, max_context_len, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  st = check_decode_pointers(fn, out, q, k_cache, v_cache, block_tables, context_lens, scale);
  if (st != PKV_OK) return st;
  const SharedLayout l = shared_layout(num_seqs, num_heads, head_dim, max_context_len);
  if (!plan || (reinterpret_cast<uintptr_t>(plan) & 255u))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan must be a 256-byte aligned device buffer", fn);
  if (plan_bytes_given < l.plan_total)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: plan of %zu bytes is smaller than the %zu these sizes need", fn,
                     plan_bytes_given, l.plan_total);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace must be a 256-byte aligned device buffer", fn);
  return shared_decode(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, dtype,
                       static_cast<const char*>(plan), static_cast<char*>(workspace), workspace ? workspace_bytes : 0,
                       !shared_applies(dtype, num_heads, num_kv_heads), stream);
}

pkv_status pkv_attention_prefill_chunk(float* out, const void* q, const int32_t* query_start_loc,
                                       int32_t num_query_tokens, int32_t max_query_len, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                                       float scale, pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_attention_prefill_chunk";
  pkv_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || max_context_len < 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: negative size", fn);
  if (num_heads <= 0 || num_heads % num_kv_heads != 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                     fn, num_heads, num_kv_heads);
  if (num_blocks <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0", fn);
  if (max_blocks_per_seq <= 0) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: max_blocks_per_seq must be > 0", fn);
  if (!std::isfinite(scale)) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !query_start_loc || !k_cache || !v_cache || !block_tables || !context_lens)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: out, q and cache pointers must be 16-byte aligned", fn);
  const int64_t group = num_heads / num_kv_heads;
  const int64_t rows_per_wg = dtype == PKV_BF16 ? kPrefillRowsPerWg : kPrefillF32RowsPerWg;
  const int64_t tiles = (static_cast<int64_t>(max_query_len) * group + rows_per_wg - 1) / rows_per_wg;
  if (static_cast<int64_t>(num_seqs) * num_kv_heads * tiles > 0x7FFFFFFF)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: launch grid too large", fn);
  pkv_prefill_args a{};
  a.out = out;
  a.q = q;
  a.query_start_loc = query_start_loc;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_query_tokens = num_query_tokens;
  a.max_query_len = max_query_len;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_context_len = max_context_len;
  a.scale_log2 = scale != 0.f ? std::fabs(scale) * 1.4426950408889634f : 1.f;
  a.q_mode = scale > 0.f ? 0 : scale < 0.f ? 1 : 2;
  return hip_status(fn, dtype == PKV_BF16 ? pkv_launch_prefill(a, stream) : pkv_launch_prefill_f32(a, stream));
}

}  // extern "C"

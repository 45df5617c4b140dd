// C ABI entry points: argument validation, workspace layout and dispatch to the
// kernel launchers.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;
int32_t g_partition_tokens = 256;

constexpr int kBlock = 16;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

pkv_status check_common(const char* fn, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        pkv_dtype dtype) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (block_size != kBlock) return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: block_size must be 16 (got %d)", fn, block_size);
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

int32_t num_partitions(int32_t max_context_len) {
  const int32_t pt = g_partition_tokens;
  const int32_t np = (max_context_len + pt - 1) / pt;
  return np < 1 ? 1 : np;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

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
                                          num_blocks, num_kv_heads, row_bytes, stream));
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
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * kBlock * head_dim * elem_bytes(dtype);
  return hip_status(fn, pkv_launch_copy_blocks(k_cache, v_cache, src_dst, num_pairs, num_blocks,
                                               block_bytes, stream));
}

pkv_status pkv_set_decode_partition_tokens(int32_t tokens) {
  if (tokens < kBlock || tokens > 8192 || tokens % kBlock != 0)
    return pkv_failf(PKV_ERR_INVALID_ARG,
                     "pkv_set_decode_partition_tokens: %d is not a multiple of 16 in [16, 8192]", tokens);
  g_partition_tokens = tokens;
  return PKV_OK;
}

int32_t pkv_get_decode_partition_tokens(void) { return g_partition_tokens; }

size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                     int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int32_t np = num_partitions(max_context_len);
  if (np <= 1) return 0;
  const size_t units = static_cast<size_t>(num_seqs) * num_heads * np;
  return align256(units * 2 * sizeof(float)) + units * head_dim * sizeof(float);
}

pkv_status pkv_attention_decode(float* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_context_len, float scale, pkv_dtype dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_attention_decode";
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
  const size_t need = pkv_attention_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len);
  if (workspace_bytes < need)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                     workspace_bytes, need);
  if (need > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: workspace must be a 256-byte aligned device buffer", fn);
  const int32_t np = num_partitions(max_context_len);
  const int64_t grid = static_cast<int64_t>(num_seqs) * num_heads * np;
  if (grid > 0x7FFFFFFF) return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: launch grid too large", fn);

  pkv_decode_args a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t units = static_cast<size_t>(num_seqs) * num_heads * np;
  a.part_ml = need ? static_cast<float*>(workspace) : nullptr;
  a.part_acc = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(units * 2 * sizeof(float)))
                    : nullptr;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.partition_tokens = g_partition_tokens;
  a.num_partitions = np;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dtype = dtype;
  return hip_status(fn, pkv_launch_decode(a, stream));
}

}  // extern "C"

// HIP kernels for gfx950 (MI355X, CDNA4, wave64): cache write, block copy,
// the decode plan and paged decode attention with a context split (the
// partition merge runs inside the decode launch).
//
// Pages cited:
//   [CB]  "Batching Continuo y PagedAttention" (cruxr.ai)
//   [IPX] iplexlaw.co.kr commentary on the vLLM PagedAttention paper
//   [OS]  "PagedAttention: gestionar la KV cache como memoria de un sistema operativo"
//   [UL]  "Continuous Batching" (Ultralytics glossary)
//
// Pool layout: [num_blocks][num_kv_heads][block_size][head_dim], block_size 8,
// 16 or 32.  One (block, KV head) tile is block_size * head_dim contiguous
// elements (4 KiB for bf16, head_dim 128, 16-token blocks).
#include "pkv_decode_valu.h"
#include "pkv_plan.h"

namespace {

// ---------------------------------------------------------------------------
// Cache write ([OS] "Cómo funciona por dentro": a token's K/V go to the slot its
// table names).  One thread moves 16 bytes of one (token, KV head) row of K and
// the same 16 bytes of V; consecutive threads move consecutive bytes of a row,
// so reads of k/v are fully coalesced and each row lands as whole 16-byte
// stores in its (block, head) tile.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_kernel(char* __restrict__ k_cache,
                                                     char* __restrict__ v_cache,
                                                     const char* __restrict__ k,
                                                     const char* __restrict__ v,
                                                     const int64_t* __restrict__ slot_mapping,
                                                     int64_t total_units, int64_t num_slots,
                                                     int32_t num_kv_heads, int32_t row_bytes, int32_t bs_log2) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (u >= total_units) return;
  const int32_t chunks = row_bytes >> 4;                  // 16-byte units per row
  const int64_t per_token = static_cast<int64_t>(num_kv_heads) * chunks;
  const int64_t t = u / per_token;
  const int64_t rem = u - t * per_token;                  // h * chunks + c
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> bs_log2, off = slot & ((1 << bs_log2) - 1);
  const int32_t h = static_cast<int32_t>(rem / chunks);
  const int32_t c = static_cast<int32_t>(rem - static_cast<int64_t>(h) * chunks);
  const int64_t dst = (((blk * num_kv_heads + h) << bs_log2) + off) * row_bytes + (static_cast<int64_t>(c) << 4);
  const int64_t src = u << 4;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(k + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v + src);
  *reinterpret_cast<u32x4*>(k_cache + dst) = kv;
  *reinterpret_cast<u32x4*>(v_cache + dst) = vv;
}

// ---------------------------------------------------------------------------
// Copy-on-write block copy ([IPX] "Dos respuestas a una entrada").  A block is
// num_kv_heads * block_size * row_bytes contiguous bytes in each pool; workgroup
// (pair, chunk) streams 4 KiB chunks of it with 16-byte loads and stores.  The
// same kernel swaps blocks between pools ([CB] "Juntándolo todo: Arquitectura
// de vLLM": a preempted request's blocks go to CPU memory and come back):
// source and destination may be different pools, one of them pinned host
// memory mapped for the device.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_dst, char* __restrict__ v_dst,
                                                          const char* __restrict__ k_src,
                                                          const char* __restrict__ v_src,
                                                          const int32_t* __restrict__ src_dst,
                                                          int32_t src_blocks, int32_t dst_blocks,
                                                          int64_t block_bytes, int32_t chunks_per_block) {
  const int32_t pair = blockIdx.x / chunks_per_block;
  const int32_t chunk = blockIdx.x - pair * chunks_per_block;
  const int32_t src = src_dst[2 * pair], dst = src_dst[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const int64_t units = block_bytes >> 4;
  const int64_t u = static_cast<int64_t>(chunk) * 256 + threadIdx.x;
  if (u >= units) return;
  const int64_t so = static_cast<int64_t>(src) * block_bytes + (u << 4);
  const int64_t dof = static_cast<int64_t>(dst) * block_bytes + (u << 4);
  const u32x4 a = *reinterpret_cast<const u32x4*>(k_src + so);
  const u32x4 b = *reinterpret_cast<const u32x4*>(v_src + so);
  *reinterpret_cast<u32x4*>(k_dst + dof) = a;
  *reinterpret_cast<u32x4*>(v_dst + dof) = b;
}

// Plan: one workgroup turns the context lengths into the unit list (the body
// is plan_body, pkv_plan.h).
__global__ __launch_bounds__(1024) void plan_kernel(int32_t* __restrict__ plan,
                                                    const int32_t* __restrict__ context_lens,
                                                    int32_t num_seqs, int32_t max_blocks_per_seq,
                                                    int32_t block_size, int32_t max_context_len, int32_t part,
                                                    const int32_t* __restrict__ seq_start) {
  plan_body(plan, context_lens, num_seqs, max_blocks_per_seq, block_size, max_context_len, part, seq_start);
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void decode_valu_kernel(pkv_decode_args a) {
  decode_valu_body<T, D, BS>(a, blockIdx.x);
}

template <typename T, int D>
int launch_decode_valu(const pkv_decode_args& a, hipStream_t st) {
  const int64_t np = (a.max_context_len + a.part_tokens - 1) / a.part_tokens;
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.num_seqs) * (np < 1 ? 1 : np) * a.num_heads));
  if (a.block_size == 8) {
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 8>), grid, dim3(256), 0, st, a);
  } else if (a.block_size == 32) {
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 32>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 16>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

int pkv_launch_plan(int32_t* plan, const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                    int32_t block_size, int32_t max_context_len, int32_t part_tokens, void* stream,
                    const int32_t* seq_start) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), plan, context_lens,
                     num_seqs, max_blocks_per_seq, block_size, max_context_len, part_tokens, seq_start);
  return hipGetLastError();
}


int pkv_launch_append(void* k_cache, void* v_cache, const void* k, const void* v,
                      const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                      int32_t num_kv_heads, int32_t row_bytes, int32_t block_size, void* stream) {
  const int64_t units = static_cast<int64_t>(num_tokens) * num_kv_heads * (row_bytes >> 4);
  if (units == 0) return hipSuccess;
  const int64_t grid = (units + 255) / 256;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), static_cast<const char*>(k),
                     static_cast<const char*>(v), slot_mapping, units,
                     static_cast<int64_t>(num_blocks) * block_size, num_kv_heads, row_bytes,
                     block_size == 8 ? 3 : block_size == 16 ? 4 : 5);
  return hipGetLastError();
}

int pkv_launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst, int32_t num_pairs,
                           int32_t num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs == 0) return hipSuccess;
  const int32_t chunks = static_cast<int32_t>(((block_bytes >> 4) + 255) / 256);
  const int64_t grid = static_cast<int64_t>(num_pairs) * chunks;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), static_cast<const char*>(k_cache),
                     static_cast<const char*>(v_cache), src_dst, num_blocks, num_blocks, block_bytes, chunks);
  return hipGetLastError();
}

int pkv_launch_swap_blocks(void* k_dst, void* v_dst, int32_t dst_blocks, const void* k_src, const void* v_src,
                           int32_t src_blocks, const int32_t* src_dst, int32_t num_pairs, int64_t block_bytes,
                           void* stream) {
  if (num_pairs == 0) return hipSuccess;
  const int32_t chunks = static_cast<int32_t>(((block_bytes >> 4) + 255) / 256);
  const int64_t grid = static_cast<int64_t>(num_pairs) * chunks;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_dst), static_cast<char*>(v_dst),
                     static_cast<const char*>(k_src), static_cast<const char*>(v_src), src_dst, src_blocks,
                     dst_blocks, block_bytes, chunks);
  return hipGetLastError();
}

int pkv_launch_decode(const pkv_decode_args& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pkv_uses_mfma(a.dtype, a.num_heads, a.num_kv_heads, a.block_size))
    return a.dtype == PKV_BF16 ? pkv_launch_decode_group(a, stream) : pkv_launch_decode_group_f32(a, stream);
  if (a.dtype == PKV_BF16)
    return a.head_dim == 128 ? launch_decode_valu<uint16_t, 128>(a, st) : launch_decode_valu<uint16_t, 64>(a, st);
  return a.head_dim == 128 ? launch_decode_valu<float, 128>(a, st) : launch_decode_valu<float, 64>(a, st);
}

/*
 * pkv.h -- C ABI of libpkv.so: paged KV-cache decode attention for MI355X (gfx950).
 *
 * What the library computes is set by four web pages on continuous batching and
 * PagedAttention, cited below as
 *   [CB]  "Batching Continuo y PagedAttention" (cruxr.ai)
 *   [IPX] iplexlaw.co.kr commentary on the vLLM PagedAttention paper (arXiv v1)
 *   [OS]  "PagedAttention: gestionar la KV cache como memoria de un sistema operativo"
 *         (josueisai.com)
 *   [UL]  "Continuous Batching" (Ultralytics glossary)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pool layout ("paged KV cache"): k_cache and v_cache are each
 *        [num_blocks][num_kv_heads][block_size][head_dim]
 *    row-major, elements of `dtype`.  One block holds the keys (values) of
 *    block_size consecutive tokens of one sequence for every KV head
 *    ([CB] "PagedAttention: Memoria virtual para la KV cache": fixed-size blocks
 *    of P tokens, P = 16; [OS] "La idea prestada: paginación").
 *  - A slot is  block * block_size + offset;  slot -1 means "no token".
 *  - Block table: int32 [num_seqs][max_blocks_per_seq]; entry i of row s is the
 *    physical block that holds tokens 16i..16i+15 of sequence s
 *    ([CB] same section: the per-request page table; [IPX] "Separar orden lógico y
 *    ubicación física").  Entries past ceil(ctx/16) are never read.
 *  - Device calls take caller-owned device pointers (e.g. torch tensors) and a
 *    hipStream_t passed as void* (NULL = the null stream).  They only enqueue
 *    work: they return as soon as the kernels are launched, never synchronise
 *    and never allocate device memory.  Host-checkable arguments are validated
 *    before anything is launched; on error nothing is enqueued.
 *  - Data that lives on the device (slots, block ids, context lengths) is not
 *    visible to the host.  Kernels never touch memory outside the buffers
 *    described by the size arguments: out-of-range slots and block ids are
 *    skipped, and attention rows they affect are written as NaN (see each call).
 *  - Supported: block_size 8, 16 or 32 ([CB] "PagedAttention: Memoria virtual
 *    para la KV cache" names 16 as typical; the others exist to measure the
 *    trade-off it describes); head_dim 64 or 128; dtype PKV_F32 or PKV_BF16
 *    (the same dtype for q, K and V); num_heads a multiple of num_kv_heads.
 *    The matrix-core kernels -- grouped-query decode, shared-prefix decode,
 *    chunked prefill, each for bf16 and fp32 -- walk contexts in 16-key tiles and take every
 *    supported block size: a tile is two 8-token blocks, one 16-token block
 *    or half of a 32-token block.
 *  - Calls that enqueue work on one stream are ordered by that stream.  For one
 *    decode step the caller enqueues pkv_copy_blocks, then pkv_append, then the
 *    attention calls: copies must read shared blocks before this step writes.
 *  - Errors: every call returns a pkv_status; pkv_last_error() gives the text of
 *    the last failure on the calling thread.  No C++ exception crosses the ABI.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,    /* a host-checkable argument is wrong; nothing done     */
  PKV_ERR_OUT_OF_BLOCKS = 2,  /* the free pool is too small; allocator state unchanged */
  PKV_ERR_UNSUPPORTED = 3,    /* valid but not built (e.g. head_dim 96)                */
  PKV_ERR_HIP = 4,            /* a HIP runtime call failed (text in pkv_last_error)    */
  PKV_ERR_UNKNOWN_SEQ = 5     /* sequence id not live in this allocator                */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------------
 * Cache write.  [OS] "Cómo funciona por dentro": each new token's key and value
 * are written into the last block of its sequence's table; [CB] "PagedAttention:
 * Memoria virtual para la KV cache": blocks fill token by token.
 *
 *   for t in [0, num_tokens), h in [0, num_kv_heads):
 *     if 0 <= slot_mapping[t] < num_blocks*block_size:
 *       k_cache[slot/bs][h][slot%bs][:] = k[t][h][:]   (same for v)
 *
 * k, v: device [num_tokens][num_kv_heads][head_dim] in the pool dtype (a pure
 * byte copy: no conversion).  slot_mapping: device int64 [num_tokens].  Slots
 * outside the pool (including -1) are skipped.  Two tokens with the same slot in
 * one call race (the allocator never produces that).  num_tokens may be 0.
 * ------------------------------------------------------------------------ */
pkv_status pkv_append(void* k_cache, void* v_cache, const void* k, const void* v,
                      const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Copy-on-write block copy.  [IPX] "Dos respuestas a una entrada": a shared
 * block that still has room is copied before a writer changes it;
 * [CB] "PagedAttention: Memoria virtual para la KV cache": copy-on-write sharing
 * as in Unix fork().
 *
 *   for i in [0, num_pairs): k_cache[dst_i] = k_cache[src_i]; v_cache[dst_i] = v_cache[src_i]
 *
 * with (src_i, dst_i) = (src_dst[2i], src_dst[2i+1]), device int32, whole blocks
 * (all heads, all slots).  Destinations must be distinct and not among the
 * sources (the allocator guarantees it), so every copy reads the pre-call pool.
 * Pairs with an id outside [0, num_blocks) are skipped.  num_pairs may be 0.
 * ------------------------------------------------------------------------ */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst,
                           int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, pkv_dtype dtype,
                           void* stream);

/* ------------------------------------------------------------------------
 * Swap copies between pools.  [CB] "Juntándolo todo: Arquitectura de vLLM":
 * under memory pressure a request's KV blocks are copied to CPU memory and its
 * GPU blocks freed; when memory allows they are copied back and the request
 * resumes.
 *
 *   for i in [0, num_pairs): dst_k[dst_i] = src_k[src_i]; dst_v[dst_i] = src_v[src_i]
 *
 * with (src_i, dst_i) = (src_dst[2i], src_dst[2i+1]) (int32, device or pinned
 * host memory), whole blocks.  Each pool is [num_blocks][num_kv_heads][16]
 * [head_dim] in `dtype`, in device memory or in pinned host memory (e.g.
 * hipHostMalloc, torch pin_memory) that the device sees at the same address,
 * which the kernel reads or writes over the host link; pageable host memory
 * is rejected (PKV_ERR_INVALID_ARG, nothing launched).  The pools' 16-byte
 * alignment and the pair array's placement are checked the same way.  Pairs with an id outside their pool are skipped.
 * Destinations must be distinct and, when both pools are the same memory, not
 * among the sources.  Host-side data is read or written asynchronously: the
 * caller synchronises the stream before touching it.
 * ------------------------------------------------------------------------ */
pkv_status pkv_swap_blocks(void* dst_k_cache, void* dst_v_cache, int32_t dst_num_blocks, const void* src_k_cache,
                           const void* src_v_cache, int32_t src_num_blocks, const int32_t* src_dst,
                           int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention.  [OS] "Cómo funciona por dentro": the kernel follows the
 * block table to each block, scores the query against the block's keys and
 * forms one softmax-weighted sum of the values; [IPX] "Separar orden lógico y
 * ubicación física": attention follows the table in logical order; [UL] "Cómo
 * funciona la planificación a nivel de iteración": attention runs per sequence
 * because every sequence has its own context length.
 *
 *   for s, h:  g = h / (num_heads/num_kv_heads);  n = context_lens[s]
 *     K_j, V_j = key/value of token j < n of sequence s, KV head g, found at
 *                block_tables[s][j/block_size], offset j%block_size
 *     out[s][h][:] = sum_j softmax_j(scale * <q[s][h], K_j>) V_j      (0 if n == 0)
 *
 * q: device [num_seqs][num_heads][head_dim] in `dtype`; out: device float32
 * [num_seqs][num_heads][head_dim]; context_lens: device int32 [num_seqs].
 * Scores, softmax and accumulation are float32.  Query-head groups of two or
 * more heads per KV head run on the matrix cores: bf16 pools with the
 * probabilities carried as a bf16 pair (~16 significant bits), every K/V row
 * read once per group of up to 64 heads (once per 16 heads beyond); float32
 * pools with exact fp32 products, likewise.  One
 * query head per KV head runs on the vector ALUs, one head per workgroup.
 * max_context_len must be >= every context length (it sizes the context
 * split); a row whose length exceeds it or
 * max_blocks_per_seq*block_size, or whose table names a block outside
 * [0, num_blocks), is written as NaN.
 * workspace: device scratch of at least pkv_attention_workspace_bytes(...) bytes
 * for the decode plan, the partial results of split contexts (the context is
 * cut into partitions of 1024 tokens; 4096, 2048 or 1024 for the
 * matrix-core group kernels, shorter for batches of fewer (sequence, KV head)
 * pairs)
 * and one 8-byte merge ticket per (sequence, head): the last partition of a
 * row to finish merges the row's partials in the same launch.  No
 * initialisation is needed (a ticket counts only under the launch's own
 * 40-bit tag, its 24-bit count covers every partition a row can have, and the
 * merging unit sets it back to 0, so a launch captured in a HIP graph can be
 * replayed); the contents are meaningless between calls.
 * Calls that share one workspace must not overlap in time (e.g. run them on
 * one stream).  Calls with workspaces of their own may run at once, on
 * several streams or from several host threads: the library keeps no other
 * state between calls (the merge tag is drawn from an atomic counter).
 * ------------------------------------------------------------------------ */
size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                     int32_t max_context_len);

pkv_status pkv_attention_decode(float* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_context_len, float scale, pkv_dtype dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode plan.  Decode work is cut into units (sequence, context partition);
 * the plan lists them longest first for the decode kernel's dispatch order.
 * It depends only on the context lengths and sizes, so a caller may build it
 * once per step and reuse it for every layer (pkv_attention_decode_planned);
 * pkv_attention_decode builds it in its workspace on every call.
 *
 * plan: device buffer of at least pkv_decode_plan_bytes(num_seqs,
 * max_context_len) bytes, 16-byte aligned.  num_seqs, num_heads,
 * num_kv_heads, block_size, max_context_len and dtype choose the partition
 * size (1024 tokens for one query head per KV head; for groups 4096, 2048 or
 * 1024, the largest that still gives the GPU a full round of workgroups);
 * they must be those of the decode calls.  A sequence with a context length of 0 or an invalid one (see
 * pkv_attention_decode) gets a unit that writes its 0 or NaN rows.  A plan
 * records num_seqs, max_context_len, max_blocks_per_seq, block_size and the
 * partition size; a decode call with other values writes NaN rows instead of
 * using it.
 * ------------------------------------------------------------------------ */
size_t pkv_decode_plan_bytes(int32_t num_seqs, int32_t max_context_len);

pkv_status pkv_decode_plan(void* plan, size_t plan_bytes, const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t max_context_len, pkv_dtype dtype, void* stream);

/* pkv_attention_decode with a plan built by pkv_decode_plan from the same
 * context_lens, num_seqs, heads, dtype, max_blocks_per_seq, block_size and
 * max_context_len (and not changed since).  Same arguments and results otherwise; the
 * workspace of pkv_attention_workspace_bytes(...) is enough. */
pkv_status pkv_attention_decode_planned(float* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, int32_t max_context_len, float scale,
                                        pkv_dtype dtype, const void* plan, size_t plan_bytes,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode with the step's cache write.  [OS] "Cómo funciona por dentro": each
 * decode step writes the new token's key and value into the sequence's last
 * block, then attends over the whole context.  This call does both in the
 * decode launch: the result and the pools afterwards are those of
 *
 *   pkv_append(k_cache, v_cache, k, v, slot_mapping, num_seqs, ...);
 *   pkv_attention_decode(_planned)(out, q, k_cache, v_cache, ...);
 *
 * where k, v: device [num_seqs][num_kv_heads][head_dim] (pool dtype) hold each
 * sequence's new token and slot_mapping: device int64 [num_seqs] its slot,
 * which must be the slot of token context_lens[s]-1 (context_lens count the
 * new token).  The decode kernels store the row there and take that token from
 * k / v directly, saving the separate cache-write launch.  slot -1: the
 * sequence has no new token this step (nothing written; attention as usual);
 * any other slot than token context_lens[s]-1's: NaN rows, nothing written.
 * plan: from pkv_decode_plan, or NULL to build it in the workspace (then the
 * workspace must hold pkv_attention_workspace_bytes(...)).
 * ------------------------------------------------------------------------ */
pkv_status pkv_attention_decode_append(float* out, const void* q, const void* k, const void* v,
                                       const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_context_len, float scale, pkv_dtype dtype, const void* plan,
                                       size_t plan_bytes, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus the workspace), kernels, results and error rules as
 * pkv_attention_decode; the plan, split-context partials and merge tickets go
 * to a scratch array inside the library, PKV_NOALLOC_SCRATCH_BYTES on every
 * GPU the library runs on, held until the process ends (located once per
 * device, on that device's first call).  The call allocates nothing: sizes
 * whose pkv_attention_workspace_bytes(num_seqs, num_heads, head_dim,
 * max_context_len) exceeds PKV_NOALLOC_SCRATCH_BYTES give PKV_ERR_INVALID_ARG
 * with nothing enqueued (e.g. 256 sequences x 64 heads x 128 dims up to
 * 4096-token contexts fit, and 16 sequences x 32 heads at 32768 tokens).  The scratch needs no clearing between calls
 * (merge tickets count only under each launch's own tag and end at 0).  All
 * calls on one GPU share its array: calls that may overlap in time on one GPU
 * (other streams, other threads) race and give wrong results -- keep them on
 * one stream.  The scratch belongs to the device of `stream` (of the current
 * device for NULL).
 * ------------------------------------------------------------------------ */
#define PKV_NOALLOC_SCRATCH_BYTES (48u * 1024u * 1024u)

pkv_status pkv_attention_decode_noalloc(float* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, int32_t max_context_len, float scale,
                                        pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Decode with shared prefixes.  [OS] "El regalo extra: compartir memoria" and
 * [IPX] "Dos respuestas a una entrada": the parallel samples of one prompt
 * share the prompt's physical blocks.  The result is that of
 * pkv_attention_decode (same arguments, same definition, same error rules);
 * the groups only change how the blocks are read:
 *
 *   group_start: device int32 [num_groups + 1], non-decreasing from 0 to
 *   num_seqs; group g is sequences group_start[g] .. group_start[g+1]-1.
 *
 * For each group the library finds on the device the longest run of leading
 * block-table entries equal in every member and wholly below every member's
 * context (its tokens rounded down to a multiple of 16: with 8-token blocks
 * an odd last common block goes to the members' own parts), reads those K/V
 * tiles once for all members (Hq/Hkv <= 16: the members' query rows share
 * one matrix-core tile, up to 16 rows; bf16 pools on the bf16 matrix cores,
 * fp32 pools on the fp32 ones), decodes each member's remaining tokens on its
 * own, and merges the two parts by their softmax statistics.  A malformed
 * group_start, groups of one sequence, members with invalid contexts or
 * tables with no common first block simply give no shared part, so no hint
 * changes a result beyond rounding.  More than 16 query heads per KV head or
 * num_groups = 0 run plain decode.  The work is two launches on `stream`
 * (the shared parts, then the members' own parts).  workspace: at least
 * pkv_attention_decode_shared_workspace_bytes(...) bytes, 256-byte aligned,
 * caller-owned device memory.
 * ------------------------------------------------------------------------ */
size_t pkv_attention_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                                   int32_t max_context_len);
pkv_status pkv_attention_decode_shared(float* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs, const int32_t* group_start,
                                       int32_t num_groups, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_context_len, float scale, pkv_dtype dtype, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The shared-prefix plan once per step.  Like the decode plan, what
 * pkv_attention_decode_shared works out before reading K/V -- each group's
 * shared leading blocks, the shared units, every sequence's own units --
 * depends only on the tables, lengths and groups, not on the layer, so a
 * caller may build it once per step and use it for every layer's pools:
 *
 *   pkv_decode_shared_plan(plan, ...)                  once per step
 *   pkv_attention_decode_shared_planned(..., plan, ...) once per layer
 *
 * gives the same bits as pkv_attention_decode_shared on every layer.
 * plan: device buffer of at least pkv_decode_shared_plan_bytes(num_seqs,
 * max_context_len) bytes, 256-byte aligned; the other arguments as for
 * pkv_attention_decode_shared (num_heads, num_kv_heads, block_size and dtype
 * must be those of the decode calls; group_start may be NULL when num_groups
 * is 0).  Where the shared path does not apply (more than 16 query heads
 * per KV head) the plan is a plain decode plan and the planned call
 * runs plain decode.  A plan built for other sizes
 * or another head grouping makes the planned call write NaN rows.
 * The planned call's workspace: at least
 * pkv_attention_decode_shared_workspace_bytes(...) bytes (partials and merge
 * tickets; no initialisation needed), 256-byte aligned.
 * ------------------------------------------------------------------------ */
size_t pkv_decode_shared_plan_bytes(int32_t num_seqs, int32_t max_context_len);

pkv_status pkv_decode_shared_plan(void* plan, size_t plan_bytes, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                  const int32_t* group_start, int32_t num_groups, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t block_size, int32_t max_context_len, pkv_dtype dtype,
                                  void* stream);

pkv_status pkv_attention_decode_shared_planned(float* out, const void* q, const void* k_cache, const void* v_cache,
                                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                               int32_t num_blocks, int32_t max_context_len, float scale,
                                               pkv_dtype dtype, const void* plan, size_t plan_bytes,
                                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Causal chunked-prefill attention.  [UL] "Cómo funciona la planificación a
 * nivel de iteración" and "Límites y técnicas complementarias": a long prompt
 * is prefilled in chunks that run in the same step as other sequences' decode.
 * Sequence s owns query tokens query_start_loc[s] .. query_start_loc[s+1]-1;
 * with n_s of them they are the last n_s tokens of its context (their K/V
 * already written with pkv_append), so query i sits at position
 * p_i = context_lens[s] - n_s + i and attends keys 0..p_i:
 *
 *   for s, i < n_s, h:  g = h / (num_heads/num_kv_heads)
 *     out[qsl[s]+i][h][:] = sum_{j<=p_i} softmax_j(scale * <q[qsl[s]+i][h], K_j>) V_j
 *
 * q: device [num_query_tokens][num_heads][head_dim] in the pools' dtype; out:
 * device float32 of the same shape; query_start_loc: device int32
 * [num_seqs+1].  Both dtypes run on the matrix cores with float32 scores,
 * softmax and accumulation: bf16 pools on the bf16 MFMA (probabilities as a
 * bf16 pair, ~16 significant bits), float32 pools on the fp32 MFMA (exact
 * fp32 products).  max_query_len must be >= every n_s (it
 * sizes the grid).  A sequence whose query range is not inside
 * [0, num_query_tokens] or is longer than max_query_len is skipped (its rows
 * are not written); one whose context is shorter than n_s, longer than
 * max_context_len or max_blocks_per_seq*block_size, or whose table names a
 * block outside [0, num_blocks), gets NaN rows.  scale may be any finite
 * value (PKV_ERR_INVALID_ARG for NaN or infinity): the kernel takes row
 * maxima of scores scaled by |scale|, with the sign moved into the query
 * (a zero scale gives the plain mean of the visible V rows).  No workspace.
 * ------------------------------------------------------------------------ */
pkv_status pkv_attention_prefill_chunk(float* out, const void* q, const int32_t* query_start_loc,
                                       int32_t num_query_tokens, int32_t max_query_len, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                                       float scale, pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator.  [CB] "PagedAttention: Memoria virtual para la KV
 * cache" and "Juntándolo todo: Arquitectura de vLLM": a request gets a block when
 * first scheduled, a new block from the free pool when its last block is full,
 * and returns all blocks when it finishes; admission needs enough free blocks.
 * [OS] "Cómo funciona por dentro": the next free block, wherever it is.
 * [IPX] "Dos respuestas a una entrada": shared prompt blocks with refcounts,
 * copy-on-write of a shared block that still has room, full shared blocks stay
 * shared, unreferenced blocks are freed.
 *
 * Policy (fixed so that results are reproducible): the free list is FIFO --
 * blocks are taken from the front, freed blocks are appended at the back in
 * block-table order; the initial order is `initial_free_order` (a permutation of
 * [0, num_blocks)) or ascending ids.  Appending to a sequence whose last block is
 * partially filled and shared (refcount > 1) first moves it to a fresh block and
 * reports the (old, new) pair, which the caller copies with pkv_copy_blocks
 * before writing.  Sequence ids are 0, 1, 2, ... in creation order (create and
 * fork), never reused.  Calls are atomic: on any error the state is unchanged.
 * Not thread-safe: use one allocator from one thread.
 * ------------------------------------------------------------------------ */
typedef struct pkv_allocator pkv_allocator;

pkv_status pkv_allocator_create(int32_t num_blocks, int32_t block_size,
                                const int32_t* initial_free_order /* host, nullable */,
                                pkv_allocator** out);
void pkv_allocator_destroy(pkv_allocator* a);
int32_t pkv_allocator_num_free(const pkv_allocator* a);
int32_t pkv_allocator_num_blocks(const pkv_allocator* a);   /* pool size (-1 for NULL) */
int32_t pkv_allocator_block_size(const pkv_allocator* a);   /* tokens per block (0 for NULL) */

pkv_status pkv_seq_create(pkv_allocator* a, int64_t* seq_id);

/* Reserve slots for n_tokens new tokens of seq.  slots_out: host int64
 * [n_tokens].  cow_src_dst_out: host int32 [2]; *n_cow_out is 0 or 1. */
pkv_status pkv_seq_append_slots(pkv_allocator* a, int64_t seq, int32_t n_tokens,
                                int64_t* slots_out, int32_t* cow_src_dst_out,
                                int32_t* n_cow_out);

/* Batched form for one scheduler step: appends n_tokens[i] tokens to seqs[i]
 * for i in [0, count) (distinct sequences), writing all slots consecutively into
 * slots_out (host int64 [sum n_tokens]) and the copy pairs into cow_src_dst_out
 * (host int32 [count][2]; *n_cow_out pairs).  All-or-nothing. */
pkv_status pkv_seq_append_slots_batch(pkv_allocator* a, const int64_t* seqs,
                                      const int32_t* n_tokens, int32_t count,
                                      int64_t* slots_out, int32_t* cow_src_dst_out,
                                      int32_t* n_cow_out);

/* New sequence sharing every block of parent (refcounts + 1). */
pkv_status pkv_seq_fork(pkv_allocator* a, int64_t parent, int64_t* child);

/* Drop seq; blocks whose refcount reaches 0 return to the back of the free list. */
pkv_status pkv_seq_free(pkv_allocator* a, int64_t seq);

/* Copy seq's block table (up to cap entries) to out; *n_blocks = table length,
 * *n_tokens = context length.  Fails if cap < table length. */
pkv_status pkv_seq_block_table(const pkv_allocator* a, int64_t seq, int32_t* out, int32_t cap,
                               int32_t* n_blocks, int32_t* n_tokens);

/* Dense tables for a batch: tables_out host int32 [count][max_blocks] (unused
 * entries 0), context_lens_out host int32 [count]. */
pkv_status pkv_block_tables(const pkv_allocator* a, const int64_t* seqs, int32_t count,
                            int32_t max_blocks, int32_t* tables_out, int32_t* context_lens_out);

pkv_status pkv_block_refcount(const pkv_allocator* a, int32_t block, int32_t* rc);

/* Free blocks that appending n_tokens to seq would take (admission check). */
pkv_status pkv_seq_blocks_needed(const pkv_allocator* a, int64_t seq, int32_t n_tokens,
                                 int32_t* needed);

/* ------------------------------------------------------------------------
 * Continuous-batching scheduler (host).  [UL] "Cómo funciona la planificación a
 * nivel de iteración": after every step finished sequences leave and free
 * their memory and queued requests are admitted if they fit in the KV cache; a
 * new request is prefilled in the same step as the others decode.  "Límites y
 * técnicas complementarias": steps are capped in sequences (max_num_seqs) and
 * tokens (max_num_batched_tokens).  [CB] "Juntándolo todo: Arquitectura de
 * vLLM": admission needs enough free blocks; under memory pressure a request's
 * blocks are copied to CPU memory and freed, and copied back later.
 *
 * A request of output length L holds its sequence slot for L steps: the step
 * that admits it prefills its prompt (one token out), each of the next L-1
 * steps decodes one token; it leaves at the start of the following step.
 * Each pkv_scheduler_step, in order: (1) finished requests leave and their
 * blocks are freed; (2) running requests, in admission order, take one decode
 * slot each -- while the pool is short, the most recently admitted running
 * request is swapped out (its blocks, in table order, to host blocks taken
 * first in first out; if the host pool is full, that request and the later
 * ones wait this step); (3) if nothing was swapped out, swapped requests return
 * first in first out (a fresh table, then their decode slot); (4) queued
 * requests are admitted first in first out -- never ahead of a swapped one --
 * while a sequence slot, the token budget and free blocks for the whole prompt
 * allow (PKV_SCHED_STATIC: only when nothing is running or swapped), their
 * prompts taking slots.  The step's slot_mapping lists the prefill tokens
 * (admission order) then one decode token per decoding request.
 *
 * The caller runs, on one stream and in this order: the swap-out copies
 * (device block -> host block), the swap-in copies (host block -> device
 * block), pkv_append of the step's K/V at slot_mapping, then prefill and
 * decode attention.  The scheduler owns the allocator sequences it creates
 * (pkv_scheduler_request gives a request's sequence id for block tables); the
 * caller must not free or fork them.  Not thread-safe.
 * ------------------------------------------------------------------------ */
typedef struct pkv_scheduler pkv_scheduler;
typedef enum { PKV_SCHED_CONTINUOUS = 0, PKV_SCHED_STATIC = 1 } pkv_sched_policy;
typedef enum { PKV_REQ_WAITING = 0, PKV_REQ_RUNNING = 1, PKV_REQ_SWAPPED = 2, PKV_REQ_FINISHED = 3 } pkv_req_state;

typedef struct {
  int32_t num_finished;        /* requests that left at the start of this step   */
  int32_t num_swapped_out;     /* requests moved to host memory                  */
  int32_t num_swap_out_pairs;  /* (device block, host block) copies              */
  int32_t num_swapped_in;      /* requests back from host memory (they decode)   */
  int32_t num_swap_in_pairs;   /* (host block, device block) copies              */
  int32_t num_prefill;         /* requests admitted and prefilled                */
  int32_t num_prefill_tokens;  /* their prompt tokens                            */
  int32_t num_decode;          /* requests decoding one token                    */
} pkv_step_info;

/* alloc: the allocator whose blocks the scheduler manages (not owned).
 * num_host_blocks: host swap space in blocks (0 = no swapping). */
pkv_status pkv_scheduler_create(pkv_allocator* alloc, int32_t max_num_seqs, int32_t max_num_batched_tokens,
                                pkv_sched_policy policy, int32_t num_host_blocks, pkv_scheduler** out);
void pkv_scheduler_destroy(pkv_scheduler* s);

/* Queue a request; ids are 0, 1, 2, ... in call order.  Rejected (nothing
 * queued) if prompt_len is outside [1, max_num_batched_tokens], output_len < 1
 * (PKV_ERR_INVALID_ARG), or prompt+output tokens exceed the whole pool
 * (PKV_ERR_OUT_OF_BLOCKS). */
pkv_status pkv_scheduler_add_request(pkv_scheduler* s, int32_t prompt_len, int32_t output_len,
                                     int64_t* request_id);

/* One step (see above); *info gets the sizes of its output.  A step with no
 * request left to run schedules nothing (all counts but num_finished 0).
 * PKV_ERR_OUT_OF_BLOCKS: requests remain but none can run (host swap space
 * exhausted); finished requests have still left. */
pkv_status pkv_scheduler_step(pkv_scheduler* s, pkv_step_info* info);

/* Copy out the last step's lists (each pointer may be NULL to skip it), sized by
 * its pkv_step_info: finished[num_finished], swapped_out[num_swapped_out],
 * swap_out_pairs[num_swap_out_pairs][2], swapped_in[num_swapped_in],
 * swap_in_pairs[num_swap_in_pairs][2], prefill[num_prefill],
 * prefill_query_start_loc[num_prefill + 1], decode[num_decode],
 * slot_mapping[num_prefill_tokens + num_decode]. */
pkv_status pkv_scheduler_step_output(const pkv_scheduler* s, int64_t* finished, int64_t* swapped_out,
                                     int32_t* swap_out_pairs, int64_t* swapped_in, int32_t* swap_in_pairs,
                                     int64_t* prefill, int32_t* prefill_query_start_loc, int64_t* decode,
                                     int64_t* slot_mapping);

/* A request's state (pkv_req_state), allocator sequence id (-1 unless running),
 * tokens generated so far and cached context length.  Pointers may be NULL. */
pkv_status pkv_scheduler_request(const pkv_scheduler* s, int64_t request_id, int32_t* state, int64_t* seq_id,
                                 int32_t* generated, int32_t* context_len);

/* Steps that ran, request-steps (busy sequence slots summed over steps), and
 * the current queue sizes.  Pointers may be NULL. */
pkv_status pkv_scheduler_stats(const pkv_scheduler* s, int64_t* steps, int64_t* busy_slot_steps,
                               int32_t* num_waiting, int32_t* num_running, int32_t* num_swapped);

/* The scheduler's allocator and its limits (for callers that size buffers). */
pkv_allocator* pkv_scheduler_allocator(const pkv_scheduler* s);
int32_t pkv_scheduler_max_num_seqs(const pkv_scheduler* s);
int32_t pkv_scheduler_max_num_batched_tokens(const pkv_scheduler* s);

/* ------------------------------------------------------------------------
 * Step executor: the continuous-batching loop of [UL] "Cómo funciona la
 * planificación a nivel de iteración" run natively, one call per step and one
 * per layer, so that the host builds a step's indices once and the GPU does
 * everything else.
 *
 * pkv_batch_schedule runs pkv_scheduler_step, gathers the step's indices --
 * slot_mapping, the prefill query ranges, block tables and lengths, the decode
 * block tables and lengths, the swap-out and swap-in pairs -- into the
 * caller's pinned host staging buffer (two halves used in turn: a half is
 * rewritten only after the copy that read it two steps ago has finished, which
 * the call waits for on the host), copies them to the caller's device buffer
 * with one asynchronous copy on `stream`, and builds the decode plan there.
 * Then, for each layer, pkv_batch_layer enqueues on `stream`: the swap-out
 * copies (that layer's device pools -> its host pools), the swap-in copies,
 * pkv_append of the prompts' K/V rows, causal prefill of the admitted prompts
 * and decode of the running requests (pkv_attention_decode_append: the decode
 * tokens' K/V rows are written by the decode launch).  Per layer the caller passes
 *   q: [T][num_heads][head_dim], k and v: [T][num_kv_heads][head_dim] (pool
 *   dtype), out: float32 [T][num_heads][head_dim], with T =
 *   num_prefill_tokens + num_decode tokens in slot_mapping order (the prefill
 *   tokens of the admitted requests in admission order, then one decode token
 *   per decoding request); out gets prefill rows then decode rows.
 * k_host / v_host may be NULL when no swap copies are due.
 *
 * Limits: bf16 or float32 pools (PKV_ERR_INVALID_ARG for another dtype), the
 * allocator's block size 8, 16 or 32, head_dim 64 or 128, query heads a
 * multiple of KV heads; max_blocks_per_seq bounds every
 * request's table (PKV_ERR_INVALID_ARG from pkv_batch_schedule otherwise,
 * after the scheduler step).  Buffers: host_staging of
 * pkv_batch_host_bytes(...) bytes of pinned host memory and device_buffer of
 * pkv_batch_device_bytes(...) bytes, both caller-owned and kept until
 * pkv_batch_destroy; num_blocks is the device pool size (it bounds the swap
 * pairs of a step).  Not thread-safe; one stream per batch.
 * ------------------------------------------------------------------------ */
typedef struct pkv_batch pkv_batch;

size_t pkv_batch_host_bytes(int32_t max_num_seqs, int32_t max_num_batched_tokens, int32_t max_blocks_per_seq,
                            int32_t num_blocks);
size_t pkv_batch_device_bytes(int32_t max_num_seqs, int32_t max_num_batched_tokens, int32_t max_blocks_per_seq,
                              int32_t num_blocks, int32_t num_heads, int32_t head_dim);
pkv_status pkv_batch_create(pkv_scheduler* sched, int32_t max_blocks_per_seq, int32_t num_blocks,
                            int32_t num_host_blocks, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            pkv_dtype dtype, void* host_staging, size_t host_bytes, void* device_buffer,
                            size_t device_bytes, pkv_batch** out);
void pkv_batch_destroy(pkv_batch* b);
pkv_status pkv_batch_schedule(pkv_batch* b, void* stream, pkv_step_info* info);
pkv_status pkv_batch_layer(pkv_batch* b, void* k_cache, void* v_cache, void* k_host, void* v_host, const void* q,
                           const void* k, const void* v, float* out, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

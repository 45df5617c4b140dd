// The decode plan as a device function, included by the kernel sources: the
// plan kernel runs it alone, the shared-prefix plan kernel after computing the
// sequences' shared prefixes in the same workgroup.
#pragma once

#include "pkv_device.h"

namespace {

using pkvd::kPlanHdr;
using pkvd::len_ok;

// ---------------------------------------------------------------------------
// Plan: one workgroup turns the context lengths into the unit list.  Full
// partitions come first (sequence order), then remainders sorted by size,
// largest first (a counting sort over the part_tokens possible sizes; the
// order inside one size is whatever the LDS atomics give, which changes no
// result: every unit computes the same partial whenever it runs), then one
// (s, -1) unit per sequence with an empty or invalid context, whose rows the
// decode kernel writes as 0 or NaN.  With seq_start (shared-prefix decode) a
// sequence's units cover tokens seq_start[s] .. ctx - 1 only.
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 1024 threads of a workgroup (*total gets the
// sum): each wave scans with shuffles, then every thread adds the totals of
// the waves before it, read from LDS -- two barriers instead of one per step.
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* sm_waves, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sm_waves[wave] = v;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 1024 / 64; ++w) {
    const int32_t t = sm_waves[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// The plan of one 1024-thread workgroup (every thread calls it).
__device__ __forceinline__ void plan_body(int32_t* __restrict__ plan, const int32_t* __restrict__ context_lens,
                                          int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                                          int32_t max_context_len, int32_t part,
                                          const int32_t* __restrict__ seq_start) {
  __shared__ int32_t bucket[kMaxPartTokens];   // remainder size -> count, then -> next slot
  __shared__ int32_t sm_waves[1024 / 64];
  __shared__ int32_t sm_full, sm_special;
  const int tid = threadIdx.x;
  int32_t* units = plan + kPlanHdr;
  for (int i = tid; i < part; i += 1024) bucket[i] = 0;
  if (tid == 0) { sm_full = 0; sm_special = 0; }
  __syncthreads();
  int32_t full = 0;
  for (int32_t s = tid; s < num_seqs; s += 1024) {
    const int32_t ctx = context_lens[s];
    if (!len_ok(ctx, max_context_len, max_blocks_per_seq, block_size)) continue;
    const int32_t len = ctx - (seq_start ? seq_start[s] : 0);
    full += len / part;
    if (len % part) atomicAdd(&bucket[len % part], 1);
  }
  atomicAdd(&sm_full, full);
  __syncthreads();
  const int32_t n_full = sm_full;
  // bucket r's first slot = n_full + (remainders larger than r): a running sum
  // over r from large to small, one thread per bucket, in chunks of 1024.
  int32_t carry = n_full;
  for (int32_t base = part - 1; base >= 0; base -= 1024) {
    const int32_t r = base - tid;
    const int32_t c = r >= 1 ? bucket[r] : 0;
    int32_t chunk_total;
    const int32_t incl = block_inclusive_scan(c, sm_waves, &chunk_total);
    if (r >= 1) bucket[r] = carry + incl - c;
    carry += chunk_total;
  }
  const int32_t n_regular = carry;
  // full units at exclusive prefix positions, remainder units at their bucket
  // slot, rowless sequences after all of them
  int32_t run = 0;
  for (int32_t base = 0; base < num_seqs; base += 1024) {
    const int32_t s = base + tid;
    const int32_t ctx = s < num_seqs ? context_lens[s] : 0;
    const bool ok = s < num_seqs && len_ok(ctx, max_context_len, max_blocks_per_seq, block_size);
    const int32_t len = ok ? ctx - (seq_start ? seq_start[s] : 0) : 0;
    const int32_t nf = len / part;
    int32_t chunk_total;
    const int32_t first = run + block_inclusive_scan(nf, sm_waves, &chunk_total) - nf;
    for (int32_t q = 0; q < nf; ++q) {
      units[2 * (first + q)] = s;
      units[2 * (first + q) + 1] = q;
    }
    if (ok && len % part) {
      const int32_t slot = atomicAdd(&bucket[len % part], 1);
      units[2 * slot] = s;
      units[2 * slot + 1] = nf;
    }
    if (s < num_seqs && !ok) {
      const int32_t slot = n_regular + atomicAdd(&sm_special, 1);
      units[2 * slot] = s;
      units[2 * slot + 1] = -1;
    }
    run += chunk_total;
  }
  __syncthreads();
  if (tid == 0) {
    plan[0] = n_regular + sm_special;
    plan[1] = num_seqs;
    plan[2] = max_context_len;
    plan[3] = max_blocks_per_seq;
    plan[4] = part;
    plan[5] = block_size;
    plan[6] = 0;
    plan[7] = 0;
  }
}

}  // namespace

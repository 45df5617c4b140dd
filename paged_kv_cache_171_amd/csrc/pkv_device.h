// Device-side definitions shared by the HIP kernel sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pkv_internal.h"

namespace pkvd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;            // keys per tile of the MFMA kernels (one 16-token block, two 8-token blocks or half a 32-token one)
constexpr float kNegBig = -FLT_MAX;   // finite "minus infinity" for running maxima
// Plan layout (int32): a header of kPlanHdr words -- n_units, num_seqs,
// max_context_len, max_blocks_per_seq, part_tokens, block_size, 0, 0 -- then (s, p) per
// unit; p = -1 marks a sequence with no attention work (empty or invalid
// context).
constexpr int kPlanHdr = 8;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48 hold the
// same MFMA column): swap odd rows with even ones, then halves, taking the
// NaN-propagating maximum.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// A wave-uniform 32-bit load of a block id through the constant address
// space: the compiler issues it as a scalar load and tracks its wait itself.
// Scalar loads share their wait counter with LDS operations, not with the
// direct-to-LDS copies (counted with the vector loads), so waiting for one
// never drains the copies in flight.  j must be wave-uniform.
__device__ __forceinline__ int32_t load_block_id(const int32_t* table, int32_t j) {
  return ((const __attribute__((address_space(4))) int32_t*)table)[j];
}

// A context length that takes part in attention (others give a 0 row or a NaN row).
__device__ __forceinline__ bool len_ok(int32_t ctx, int32_t max_context_len, int32_t max_blocks_per_seq,
                                       int32_t block_size) {
  return ctx > 0 && ctx <= max_context_len && static_cast<int64_t>(ctx) <= static_cast<int64_t>(max_blocks_per_seq) * block_size;
}

// A shared-prefix plan (header: units, num_seqs, max_context_len,
// max_blocks_per_seq, prefix partition tokens, query heads per KV head) was
// built for these sizes.
__device__ __forceinline__ bool shared_plan_matches(const int32_t* sp, const pkv_decode_args& a) {
  return sp[1] == a.num_seqs && sp[2] == a.max_context_len && sp[3] == a.max_blocks_per_seq &&
         sp[4] == a.prefix_part_tokens && sp[5] == a.num_heads / a.num_kv_heads;
}

// The plan (and with shared-prefix decode the shared plan too) was built for
// these sizes.
__device__ __forceinline__ bool plan_matches(const int32_t* plan, const pkv_decode_args& a) {
  return plan[1] == a.num_seqs && plan[2] == a.max_context_len && plan[3] == a.max_blocks_per_seq &&
         plan[4] == a.part_tokens && plan[5] == a.block_size &&
         (a.shared_plan == nullptr || shared_plan_matches(a.shared_plan, a));
}

__device__ __forceinline__ const int32_t* plan_units(const int32_t* plan) { return plan + kPlanHdr; }

// First token of sequence s covered by its own plan units (0 unless a shared
// prefix covers the ones before it) and the partial slot its first unit writes.
__device__ __forceinline__ int32_t seq_start_of(const pkv_decode_args& a, int32_t s) {
  return a.seq_start ? a.seq_start[s] : 0;
}
__device__ __forceinline__ int32_t slot_base_of(const pkv_decode_args& a, int32_t start) {
  return start > 0 ? (start + a.prefix_part_tokens - 1) / a.prefix_part_tokens : 0;
}

// Log-sum-exp merge of the n partials (m in log2 units, l, acc) of one output
// element: sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M), M = max_p m_p.
// The partials are loaded 8 at a time (all loads of a chunk in flight
// together) and the chunks combined by the same rule; with n <= 8 this is the
// plain one-pass sum.  Load(p) reads one float.
// Slot `self` (if >= 0) is not read: its (m, l, acc) are sm, sl, so.
template <typename Load>
__device__ __forceinline__ float merge_partials_with(const float* ml, const float* acc, int32_t n, int32_t stride,
                                                     Load load, int32_t self = -1, float sm = 0.f, float sl = 0.f,
                                                     float so = 0.f) {
  constexpr int kChunk = 8;
  float M = -INFINITY, L = 0.f, o = 0.f;
  for (int32_t q0 = 0; q0 < n; q0 += kChunk) {
    float mv[kChunk], lv[kChunk], av[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const bool in = q0 + i < n && q0 + i != self;
      mv[i] = in ? load(ml + 2 * (q0 + i)) : q0 + i == self ? sm : -INFINITY;
      lv[i] = in ? load(ml + 2 * (q0 + i) + 1) : q0 + i == self ? sl : 0.f;
      av[i] = in ? load(acc + static_cast<int64_t>(q0 + i) * stride) : q0 + i == self ? so : 0.f;
    }
    float Mc = mv[0];
#pragma unroll
    for (int i = 1; i < kChunk; ++i) Mc = fmaxf(Mc, mv[i]);
    const float Mn = fmaxf(M, Mc);
    const float r = fast_exp2(M - Mn);     // 0 for the first chunk
    float Lc = 0.f, oc = 0.f;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (q0 + i < n) {
        const float f = fast_exp2(mv[i] - Mn);
        Lc += lv[i] * f;
        oc += av[i] * f;
      }
    }
    L = L * r + Lc;
    o = o * r + oc;
    M = Mn;
  }
  return o / L;
}

// The partition merge inside the decode launch.  The partials of a row whose
// merge happens in the launch are written and read with agent-scope atomic
// accesses, which go through to the level shared by all XCDs (each XCD's L2 is
// private), so no cache-wide write-back or invalidation is needed: ordering
// alone (every vector memory access of the thread complete) makes them
// visible.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): every vector memory access done
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Merge tickets.  A ticket is one 64-bit word per row: (epoch << 24) | units
// arrived.  The epoch (40 bits, nonzero) is new for every call, so a word
// left by another call counts as 0 arrivals and the buffer never needs
// clearing (a call of two launches counts the arrivals of both).  24 bits count every partition a row can have: a context of at
// most 2^31 - 1 tokens in 1024-token partitions is at most 2^21 of them, plus
// as many shared-prefix partitions.
constexpr int kTicketCountBits = 24;
constexpr uint64_t kTicketCountMask = (uint64_t{1} << kTicketCountBits) - 1;

// One arrival on a ticket (one thread): whether it was the last of `units`,
// in which case the ticket is set back to 0.  Each unit takes one ticket step,
// so the compare-and-swap loop ends after at most `units` rounds.
__device__ __forceinline__ bool ticket_arrive(uint64_t* ticket, uint64_t epoch, int32_t units) {
  const uint64_t tag = epoch << kTicketCountBits;
  uint64_t old = __hip_atomic_load(ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t arrived;
  for (;;) {
    arrived = ((old & ~kTicketCountMask) == tag ? (old & kTicketCountMask) : 0) + 1;
    if (__hip_atomic_compare_exchange_strong(ticket, &old, tag | arrived, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
  }
  const bool last = arrived == static_cast<uint64_t>(units);
  if (last) __hip_atomic_store(ticket, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// Every thread of a workgroup calls this after its store_coherent partial
// stores; the result (uniform) says whether the workgroup's unit is the last of
// the row's `units` units to arrive, in which case the other units' partials
// can be read with load_coherent and the ticket is already back at 0.
__device__ __forceinline__ bool arrive_last(uint64_t* ticket, uint64_t epoch, int32_t units, int* sm_flag) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) *sm_flag = ticket_arrive(ticket, epoch, units) ? 1 : 0;
  __syncthreads();
  return *sm_flag != 0;
}

// merge_partials over partials written with store_coherent.
__device__ __forceinline__ float merge_partials_coherent(const float* ml, const float* acc, int32_t n,
                                                         int32_t stride) {
  return merge_partials_with(ml, acc, n, stride, [](const float* p) { return load_coherent(p); });
}

// A look at a row's ticket before arriving: whether every other one of its
// `units` units has arrived already (their partials stored and complete, as
// they store before they arrive).  Arrivals only add to the count within a
// launch, so a unit that sees units - 1 is the last one, and no other unit
// waits for it: it need not store its own partial nor arrive; it merges the
// others' partials with its own (merge_partials_coherent_self) and sets the
// ticket back to 0 (reset_ticket).
__device__ __forceinline__ uint64_t peek_ticket(const uint64_t* ticket) {
  return __hip_atomic_load(const_cast<uint64_t*>(ticket), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ticket_all_others(uint64_t seen, uint64_t epoch, int32_t units) {
  const uint64_t tag = epoch << kTicketCountBits;
  const uint64_t arrived = (seen & ~kTicketCountMask) == tag ? (seen & kTicketCountMask) : 0;
  return arrived + 1 == static_cast<uint64_t>(units);
}
__device__ __forceinline__ void reset_ticket(uint64_t* ticket) {
  __hip_atomic_store(ticket, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float merge_partials_coherent_self(const float* ml, const float* acc, int32_t n,
                                                              int32_t stride, int32_t self, float sm, float sl,
                                                              float so) {
  return merge_partials_with(ml, acc, n, stride, [](const float* p) { return load_coherent(p); }, self, sm, sl, so);
}

}  // namespace pkvd

// Device-side definitions shared by the HIP kernel sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pkv_internal.h"

namespace pkvd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;            // tokens per block of the MFMA kernels (the pages' P = 16)
constexpr float kNegBig = -FLT_MAX;   // finite "minus infinity" for running maxima
// Plan layout (int32): a header of kPlanHdr words -- n_units, num_seqs,
// max_context_len, max_blocks_per_seq, part_tokens, block_size, 0, 0 -- then (s, p) per
// unit; p = -1 marks a sequence with no attention work (empty or invalid
// context).
constexpr int kPlanHdr = 8;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A context length that takes part in attention (others give a 0 row or a NaN row).
__device__ __forceinline__ bool len_ok(int32_t ctx, int32_t max_context_len, int32_t max_blocks_per_seq,
                                       int32_t block_size) {
  return ctx > 0 && ctx <= max_context_len && static_cast<int64_t>(ctx) <= static_cast<int64_t>(max_blocks_per_seq) * block_size;
}

// The plan was built for these sizes.
__device__ __forceinline__ bool plan_matches(const int32_t* plan, const pkv_decode_args& a) {
  return plan[1] == a.num_seqs && plan[2] == a.max_context_len && plan[3] == a.max_blocks_per_seq &&
         plan[4] == a.part_tokens && plan[5] == a.block_size;
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
__device__ __forceinline__ float merge_partials(const float* ml, const float* acc, int32_t n, int32_t stride) {
  float M = ml[0];
  for (int32_t q = 1; q < n; ++q) M = fmaxf(M, ml[2 * q]);
  float L = 0.f, o = 0.f;
  for (int32_t q = 0; q < n; ++q) {
    const float f = fast_exp2(ml[2 * q] - M);
    L += ml[2 * q + 1] * f;
    o += acc[static_cast<int64_t>(q) * stride] * f;
  }
  return o / L;
}

}  // namespace pkvd

// Device-side definitions shared by the HIP kernel sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pkv_internal.h"

namespace pkvd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;            // tokens per block (the pages' P = 16)
constexpr float kNegBig = -FLT_MAX;   // finite "minus infinity" for running maxima
constexpr int kPlanHdr = 4;           // plan header: n_units, num_seqs, max_context_len, max_blocks_per_seq

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A context length that takes part in attention (others give a 0 row or a NaN row).
__device__ __forceinline__ bool len_ok(int32_t ctx, int32_t max_context_len, int32_t max_blocks_per_seq) {
  return ctx > 0 && ctx <= max_context_len && ctx <= max_blocks_per_seq * kBlock;
}

// The plan was built for these sizes.
__device__ __forceinline__ bool plan_matches(const int32_t* plan, const pkv_decode_args& a) {
  return plan[1] == a.num_seqs && plan[2] == a.max_context_len && plan[3] == a.max_blocks_per_seq;
}

}  // namespace pkvd

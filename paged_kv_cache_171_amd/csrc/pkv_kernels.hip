// HIP kernels for gfx950 (MI355X, CDNA4, wave64): cache write, block copy,
// paged decode attention with a context split, and the partition merge.
//
// Pages cited:
//   [CB]  "Batching Continuo y PagedAttention" (cruxr.ai)
//   [IPX] iplexlaw.co.kr commentary on the vLLM PagedAttention paper
//   [OS]  "PagedAttention: gestionar la KV cache como memoria de un sistema operativo"
//   [UL]  "Continuous Batching" (Ultralytics glossary)
//
// Pool layout: [num_blocks][num_kv_heads][16][head_dim].  One (block, KV head)
// tile is 16 * head_dim contiguous elements (4 KiB for bf16, head_dim 128).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pkv_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;        // tokens per block ([CB]: P = 16)
constexpr int kWaves = 4;         // waves per decode workgroup
constexpr float kNegBig = -FLT_MAX;

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
                                                     int32_t num_kv_heads, int32_t row_bytes) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (u >= total_units) return;
  const int32_t chunks = row_bytes >> 4;                  // 16-byte units per row
  const int64_t per_token = static_cast<int64_t>(num_kv_heads) * chunks;
  const int64_t t = u / per_token;
  const int64_t rem = u - t * per_token;                  // h * chunks + c
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4, off = slot & 15;
  const int32_t h = static_cast<int32_t>(rem / chunks);
  const int32_t c = static_cast<int32_t>(rem - static_cast<int64_t>(h) * chunks);
  const int64_t dst = ((blk * num_kv_heads + h) * kBlock + off) * row_bytes + (static_cast<int64_t>(c) << 4);
  const int64_t src = u << 4;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(k + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v + src);
  *reinterpret_cast<u32x4*>(k_cache + dst) = kv;
  *reinterpret_cast<u32x4*>(v_cache + dst) = vv;
}

// ---------------------------------------------------------------------------
// Copy-on-write block copy ([IPX] "Dos respuestas a una entrada").  A block is
// num_kv_heads * 16 * row_bytes contiguous bytes in each pool; workgroup
// (pair, chunk) streams 4 KiB chunks of it with 16-byte loads and stores.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_cache,
                                                          char* __restrict__ v_cache,
                                                          const int32_t* __restrict__ src_dst,
                                                          int32_t num_blocks, int64_t block_bytes,
                                                          int32_t chunks_per_block) {
  const int32_t pair = blockIdx.x / chunks_per_block;
  const int32_t chunk = blockIdx.x - pair * chunks_per_block;
  const int32_t src = src_dst[2 * pair], dst = src_dst[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t units = block_bytes >> 4;
  const int64_t u = static_cast<int64_t>(chunk) * 256 + threadIdx.x;
  if (u >= units) return;
  const int64_t so = static_cast<int64_t>(src) * block_bytes + (u << 4);
  const int64_t dof = static_cast<int64_t>(dst) * block_bytes + (u << 4);
  const u32x4 a = *reinterpret_cast<const u32x4*>(k_cache + so);
  const u32x4 b = *reinterpret_cast<const u32x4*>(v_cache + so);
  *reinterpret_cast<u32x4*>(k_cache + dof) = a;
  *reinterpret_cast<u32x4*>(v_cache + dof) = b;
}

// ---------------------------------------------------------------------------
// Wave-level helpers.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LPR consecutive lanes (LPR in {8, 16, 32}); every lane of a
// group gets the group's sum.  Within a 16-lane DPP row: xor-1 and xor-2 quad
// permutes, then the half-row mirror (lane i <-> 7-i) and the row mirror
// (lane i <-> 15-i) each add the partner half.  32 needs one cross-row swap.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);                       // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                       // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Storage element traits: 16 bytes of storage -> EPL float32 values.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kEpl = 4;
  __device__ static __forceinline__ void unpack(const u32x4& w, float* f) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
};
template <> struct Elem<uint16_t> {  // bf16 bits
  static constexpr int kEpl = 8;
  __device__ static __forceinline__ void unpack(const u32x4& w, float* f) {
    // element 2k is the low half of dword k, element 2k+1 the high half
    f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xFFFF0000u);
    f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xFFFF0000u);
    f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xFFFF0000u);
    f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xFFFF0000u);
  }
};

// ---------------------------------------------------------------------------
// Paged decode attention, one query per (sequence, head) -- the VALU kernel.
//
// [OS] "Cómo funciona por dentro": follow the block table, score the query
// against each block's keys, then one softmax-weighted sum of the values.
// [OS] "Qué significa esto para lo que pagas": decode is memory-bound, so the
// kernel is built around streaming K/V tiles from HBM once, at full width.
//
// Workgroup = (sequence s, query head h, context partition p) with 4 waves;
// partition p holds blocks [p*BPP, (p+1)*BPP) of the sequence, and wave w takes
// every 4th of them.  A wave reads a (block, head) tile with NLD 1 KiB loads:
// lane l reads 16 bytes at l*16 of each KiB, i.e. token i*TPL + l/LPR of the
// tile, dims (l%LPR)*EPL ... +EPL -- the same dims of q that the lane holds.
// The dot product is a group_sum over the LPR lanes of a token row (DPP, no
// LDS), so the score of a token lands in every lane of its row, which is
// exactly the set of lanes that holds that token's V row for the P*V step.
// Each row keeps its own running max / sum / accumulator (online softmax in
// base 2, q pre-scaled by scale*log2 e); rows, then waves (through LDS), are
// merged with the log-sum-exp rule at the end.  K/V tiles go straight to
// registers: every element is used once by one lane, so staging through LDS
// would only add traffic.  Masked tokens (past the context) are removed by
// select, never by multiplying with 0, so NaN in unused slots cannot leak.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DecodeShape {
  static constexpr int kEpl = Elem<T>::kEpl;            // elements per lane per load
  static constexpr int kLpr = D / kEpl;                 // lanes per token row
  static constexpr int kTpl = 64 / kLpr;                // tokens per load
  static constexpr int kNld = kBlock / kTpl;            // loads per tile
  static constexpr int kBpi = kNld <= 4 ? 2 : 1;        // tiles in flight per wave
  static_assert(kLpr == 8 || kLpr == 16 || kLpr == 32, "unsupported shape");
};

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_valu_kernel(pkv_decode_args a) {
  using S = DecodeShape<T, D>;
  constexpr int EPL = S::kEpl, LPR = S::kLpr, TPL = S::kTpl, NLD = S::kNld, BPI = S::kBpi;

  __shared__ float sm_acc[kWaves][D];
  __shared__ float sm_ml[kWaves][2];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane / LPR;
  const int col = lane % LPR;

  // blockIdx -> (p, s, h): partitions from the last to the first so that the
  // workgroups dispatched last are the short remainders.
  const int32_t Hq = a.num_heads;
  int64_t bid = blockIdx.x;
  const int32_t h = static_cast<int32_t>(bid % Hq); bid /= Hq;
  const int32_t s = static_cast<int32_t>(bid % a.num_seqs); bid /= a.num_seqs;
  const int32_t p = a.num_partitions - 1 - static_cast<int32_t>(bid);

  const int32_t ctx = a.context_lens[s];
  const int32_t cap = a.max_blocks_per_seq * kBlock;
  const bool bad_len = ctx < 0 || ctx > a.max_context_len || ctx > cap;
  const int64_t orow = (static_cast<int64_t>(s) * Hq + h) * D;
  if (bad_len || ctx == 0) {
    // Only partition 0 owns the output row; it writes NaN (bad length) or 0.
    if (p == 0 && threadIdx.x < D) a.out[orow + threadIdx.x] = bad_len ? __builtin_nanf("") : 0.0f;
    return;
  }
  const int32_t pt = a.partition_tokens;
  const int32_t tok0 = p * pt;
  if (tok0 >= ctx) return;                                  // empty partition
  const int32_t np_s = (ctx + pt - 1) / pt;
  const int32_t nblk = (ctx + kBlock - 1) / kBlock;
  const int32_t blk_begin = tok0 / kBlock;
  const int32_t blk_end = min(nblk, (tok0 + pt) / kBlock);

  const int32_t g = h / (Hq / a.num_kv_heads);
  const int64_t tile_elems = static_cast<int64_t>(kBlock) * D;
  const int64_t head_off = static_cast<int64_t>(g) * tile_elems;
  const int64_t block_stride = static_cast<int64_t>(a.num_kv_heads) * tile_elems;
  const T* __restrict__ kc = reinterpret_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = reinterpret_cast<const T*>(a.v_cache);
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;

  // q slice of this lane, pre-scaled into base-2 units
  float qv[EPL];
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.q) + orow + col * EPL);
    Elem<T>::unpack(w, qv);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] *= a.scale_log2;
  }

  float m = kNegBig, l = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  bool bad = false;

  for (int32_t j0 = blk_begin + wave; j0 < blk_end; j0 += kWaves * BPI) {
    u32x4 kt[BPI][NLD], vt[BPI][NLD];
    int32_t tb[BPI];
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
      const int32_t j = j0 + bi * kWaves;
      int32_t b = 0;
      tb[bi] = -1;
      if (j < blk_end) {
        b = table[j];
        if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; b = 0; }
        tb[bi] = j * kBlock;
      }
      const u32x4* kp = reinterpret_cast<const u32x4*>(kc + b * block_stride + head_off);
      const u32x4* vp = reinterpret_cast<const u32x4*>(vc + b * block_stride + head_off);
      if (j < blk_end) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) kt[bi][i] = __builtin_nontemporal_load(kp + i * 64 + lane);
#pragma unroll
        for (int i = 0; i < NLD; ++i) vt[bi][i] = __builtin_nontemporal_load(vp + i * 64 + lane);
      }
    }
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
      if (tb[bi] < 0) break;
      const bool full = tb[bi] + kBlock <= ctx;
      float sc[NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        float kf[EPL];
        Elem<T>::unpack(kt[bi][i], kf);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part = fmaf(qv[e], kf[e], part);
        sc[i] = group_sum<LPR>(part);
      }
      float mt = m;
      if (full) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) mt = fmaxf(mt, sc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const bool valid = tb[bi] + i * TPL + row < ctx;
          sc[i] = valid ? sc[i] : -INFINITY;
          mt = fmaxf(mt, sc[i]);
        }
      }
      const float alpha = fast_exp2(m - mt);
      m = mt;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const float pr = fast_exp2(sc[i] - m);
        l += pr;
        float vf[EPL];
        Elem<T>::unpack(vt[bi][i], vf);
        if (!full) {
          const bool valid = tb[bi] + i * TPL + row < ctx;
#pragma unroll
          for (int e = 0; e < EPL; ++e) vf[e] = valid ? vf[e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pr, vf[e], acc[e]);
      }
    }
  }

  // merge the TPL rows of the wave (lanes that hold the same dims)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    const float mo = __shfl_xor(m, off);
    const float lo = __shfl_xor(l, off);
    const float mx = fmaxf(m, mo);
    const float fa = fast_exp2(m - mx), fb = fast_exp2(mo - mx);
    l = l * fa + lo * fb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float ao = __shfl_xor(acc[e], off);
      acc[e] = acc[e] * fa + ao * fb;
    }
    m = mx;
  }
  if (lane == 0) sm_bad[wave] = bad ? 1 : 0;
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_acc[wave][col * EPL + e] = acc[e];
  }
  if (lane == 0) { sm_ml[wave][0] = m; sm_ml[wave][1] = l; }
  __syncthreads();

  if (threadIdx.x < D) {
    const int t = threadIdx.x;
    float M = sm_ml[0][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_ml[w][0]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm_ml[w][0] - M);
      L += sm_ml[w][1] * f;
      o += sm_acc[w][t] * f;
    }
    if (sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3]) { o = __builtin_nanf(""); L = __builtin_nanf(""); }
    if (np_s == 1) {
      a.out[orow + t] = o / L;
    } else {
      const int64_t pidx = (static_cast<int64_t>(s) * Hq + h) * a.num_partitions + p;
      a.part_acc[pidx * D + t] = o;
      if (t == 0) { a.part_ml[2 * pidx] = M; a.part_ml[2 * pidx + 1] = L; }
    }
  }
}

// ---------------------------------------------------------------------------
// Partition merge: for every (s, h) whose context spans more than one
// partition, M = max_p m_p, L = sum_p l_p 2^(m_p - M), out = sum_p acc_p 2^(m_p - M) / L.
// This is the log-sum-exp identity that makes the split softmax equal the
// unsplit one.  One thread per output element.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void merge_partitions_kernel(pkv_decode_args a) {
  const int64_t sh = blockIdx.x;                       // s * Hq + h
  const int32_t s = static_cast<int32_t>(sh / a.num_heads);
  const int32_t ctx = a.context_lens[s];
  const int32_t cap = a.max_blocks_per_seq * kBlock;
  if (ctx <= 0 || ctx > a.max_context_len || ctx > cap) return;   // written by the decode kernel
  const int32_t np_s = (ctx + a.partition_tokens - 1) / a.partition_tokens;
  if (np_s <= 1) return;
  const float* ml = a.part_ml + sh * a.num_partitions * 2;
  const float* acc = a.part_acc + sh * a.num_partitions * D;
  float M = ml[0];
  for (int32_t p = 1; p < np_s; ++p) M = fmaxf(M, ml[2 * p]);
  float L = 0.f, o = 0.f;
  const int t = threadIdx.x;
  for (int32_t p = 0; p < np_s; ++p) {
    const float f = fast_exp2(ml[2 * p] - M);
    L += ml[2 * p + 1] * f;
    o += acc[static_cast<int64_t>(p) * D + t] * f;
  }
  a.out[sh * D + t] = o / L;
}

template <typename T, int D>
int launch_decode_typed(const pkv_decode_args& a, hipStream_t st) {
  const int64_t grid = static_cast<int64_t>(a.num_seqs) * a.num_heads * a.num_partitions;
  hipLaunchKernelGGL((decode_valu_kernel<T, D>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.num_partitions > 1) {
    hipLaunchKernelGGL((merge_partitions_kernel<D>), dim3(static_cast<uint32_t>(a.num_seqs) * a.num_heads),
                       dim3(D), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

int pkv_launch_append(void* k_cache, void* v_cache, const void* k, const void* v,
                      const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                      int32_t num_kv_heads, int32_t row_bytes, void* stream) {
  const int64_t units = static_cast<int64_t>(num_tokens) * num_kv_heads * (row_bytes >> 4);
  if (units == 0) return hipSuccess;
  const int64_t grid = (units + 255) / 256;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), static_cast<const char*>(k),
                     static_cast<const char*>(v), slot_mapping, units,
                     static_cast<int64_t>(num_blocks) * kBlock, num_kv_heads, row_bytes);
  return hipGetLastError();
}

int pkv_launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst, int32_t num_pairs,
                           int32_t num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs == 0) return hipSuccess;
  const int32_t chunks = static_cast<int32_t>(((block_bytes >> 4) + 255) / 256);
  const int64_t grid = static_cast<int64_t>(num_pairs) * chunks;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), src_dst, num_blocks, block_bytes, chunks);
  return hipGetLastError();
}

int pkv_launch_decode(const pkv_decode_args& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.dtype == PKV_BF16) {
    if (a.head_dim == 128) return launch_decode_typed<uint16_t, 128>(a, st);
    return launch_decode_typed<uint16_t, 64>(a, st);
  }
  if (a.head_dim == 128) return launch_decode_typed<float, 128>(a, st);
  return launch_decode_typed<float, 64>(a, st);
}

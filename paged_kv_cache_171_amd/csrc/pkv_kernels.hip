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
#include "pkv_device.h"

namespace {

using pkvd::u32x4;
using pkvd::kNegBig;
using pkvd::kPlanHdr;
using pkvd::fast_exp2;
using pkvd::len_ok;
using pkvd::plan_matches;

constexpr int kWaves = 4;         // waves per decode workgroup

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
// num_kv_heads * 16 * row_bytes contiguous bytes in each pool; workgroup
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

// Global-memory (address space 1) pointers.  uniform_gptr moves a pointer that
// every lane agrees on into scalar registers, so loads use the scalar-base +
// 32-bit lane-offset form of global_load.
typedef const __attribute__((address_space(1))) char* gptr_t;
typedef const __attribute__((address_space(1))) u32x4* gptr4_t;
typedef const __attribute__((address_space(1))) int32_t* gptri_t;

__device__ __forceinline__ gptr_t uniform_gptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ u32x4 load16_nt(gptr_t base, uint32_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<gptr4_t>(base + off));
}

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
// kernel is built around streaming every K/V tile from HBM exactly once.
//
// Work units.  A sequence's context is cut into partitions of part_tokens
// tokens (1024 here); a unit is (sequence s, partition p) and one workgroup
// handles one unit for one query head.  The plan (plan_kernel) lists the units longest first --
// every full partition, then the remainders by decreasing size -- so that the
// workgroups dispatched last are the short ones and the ragged batches of
// continuous batching ([UL] "Cómo funciona la planificación a nivel de
// iteración") do not leave a long unit running alone at the end.  The grid is
// units x heads with the head fastest, so the workgroups that run together
// read the tiles of all heads of the same blocks.
//
// Inside a workgroup.  The unit's blocks are dealt to the 4 waves in turn.  A
// (block, head) tile is 16 * D contiguous elements read with NLD 1 KiB loads:
// lane l reads 16 bytes at l*16 of each KiB, i.e. token i*TPL + l/LPR of the
// tile, dims (l%LPR)*EPL ... +EPL -- the dims of q the lane holds.  The dot
// product is a group_sum over the LPR lanes of a token row (DPP, no LDS), so a
// token's score lands in every lane of its row -- the lanes that hold that
// token's V row for the P*V step.  Each row keeps its own online-softmax state
// (base 2, q pre-scaled by scale*log2 e); rows, then waves (through LDS), are
// merged with the log-sum-exp rule.  K/V go straight to registers: every
// element is used once by one lane, so staging through LDS would only add
// traffic.  Masked tokens (past the context) are removed by select, never by
// multiplying with 0, so NaN in unused slots cannot leak.  A unit of a
// sequence with one partition writes the output row; otherwise it writes a
// partial (max, sum, unnormalised accumulator) for merge_partitions_kernel.
// ---------------------------------------------------------------------------
template <typename T, int D, int BS>
struct DecodeShape {
  static constexpr int kEpl = Elem<T>::kEpl;            // elements per lane per load
  static constexpr int kLpr = D / kEpl;                 // lanes per token row
  static constexpr int kTpl = 64 / kLpr;                // tokens per 1 KiB load
  static constexpr int kNld = BS / kTpl;                // KiB per tile
  static constexpr int kBpi = kNld <= 4 ? 2 : 1;        // tiles in flight per wave
  static_assert(kLpr == 8 || kLpr == 16 || kLpr == 32, "unsupported shape");
  static_assert(kNld >= 1, "a tile must fill at least one 1 KiB load");
};

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
__global__ __launch_bounds__(1024) void plan_kernel(int32_t* __restrict__ plan,
                                                    const int32_t* __restrict__ context_lens,
                                                    int32_t num_seqs, int32_t max_blocks_per_seq,
                                                    int32_t block_size, int32_t max_context_len, int32_t part,
                                                    const int32_t* __restrict__ seq_start) {
  __shared__ int32_t bucket[kMaxPartTokens];   // remainder size -> count, then -> next slot
  __shared__ int32_t scan[1024];
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
    scan[tid] = c;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t y = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += y;
      __syncthreads();
    }
    if (r >= 1) bucket[r] = carry + scan[tid] - c;
    const int32_t chunk_total = scan[1023];
    __syncthreads();
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
    scan[tid] = nf;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t y = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += y;
      __syncthreads();
    }
    const int32_t first = run + scan[tid] - nf;
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
    const int32_t chunk_total = scan[1023];
    __syncthreads();
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

template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void decode_valu_kernel(pkv_decode_args a) {
  using S = DecodeShape<T, D, BS>;
  constexpr int kBlock = BS;          // tokens per block of this instance
  constexpr int EPL = S::kEpl, LPR = S::kLpr, TPL = S::kTpl, NLD = S::kNld, BPI = S::kBpi;

  __shared__ float sm_acc[kWaves][D];
  __shared__ float sm_ml[kWaves][2];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int row = lane / LPR;
  const int col = lane % LPR;

  const int32_t Hq = a.num_heads;
  const int32_t u = static_cast<int32_t>(blockIdx.x / Hq);
  const int32_t h = static_cast<int32_t>(blockIdx.x - static_cast<uint32_t>(u) * Hq);
  const int32_t* plan = a.plan;
  if (!plan_matches(plan, a)) {
    // a plan built for other sizes: every row is NaN
    if (u < a.num_seqs && threadIdx.x < D)
      a.out[(static_cast<int64_t>(u) * Hq + h) * D + threadIdx.x] = __builtin_nanf("");
    return;
  }
  if (u >= plan[0]) return;
  const int32_t* units = pkvd::plan_units(plan);
  const int32_t s = units[2 * u];
  const int32_t p = units[2 * u + 1];
  const int32_t ctx = a.context_lens[s];
  const int64_t orow = (static_cast<int64_t>(s) * Hq + h) * D;
  if (p < 0) {
    // no attention work: an empty context gives 0, an invalid one NaN
    if (threadIdx.x < D) a.out[orow + threadIdx.x] = ctx == 0 ? 0.f : __builtin_nanf("");
    return;
  }
  const int32_t part = a.part_tokens;
  const int32_t start = pkvd::seq_start_of(a, s);
  const int32_t base = pkvd::slot_base_of(a, start);
  const int32_t np_s = (ctx - start + part - 1) / part;
  const int32_t nblk = (ctx + kBlock - 1) / kBlock;
  const int32_t blk_begin = start / kBlock + p * (part / kBlock);
  const int32_t blk_end = min(nblk, blk_begin + part / kBlock);

  constexpr int64_t kTileBytes = static_cast<int64_t>(kBlock) * D * sizeof(T);
  const int64_t block_bytes = static_cast<int64_t>(a.num_kv_heads) * kTileBytes;
  const int64_t head_off = static_cast<int64_t>(h / (Hq / a.num_kv_heads)) * kTileBytes;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache);
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

  // The block ids of the next iteration are fetched (scalar loads) while the
  // current iteration's tiles are in flight.
  int32_t nxt[BPI];
#pragma unroll
  for (int bi = 0; bi < BPI; ++bi) {
    const int32_t j = blk_begin + wave + bi * kWaves;
    nxt[bi] = j < blk_end ? table[j] : 0;
  }
  for (int32_t j0 = blk_begin + wave; j0 < blk_end; j0 += kWaves * BPI) {
    u32x4 kt[BPI][NLD], vt[BPI][NLD];
    int32_t tb[BPI];
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
      const int32_t j = j0 + bi * kWaves;
      int32_t b = nxt[bi];
      tb[bi] = -1;
      if (j < blk_end) {
        if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; b = 0; }
        tb[bi] = j * kBlock;
        const u32x4* kp = reinterpret_cast<const u32x4*>(kc + b * block_bytes + head_off);
        const u32x4* vp = reinterpret_cast<const u32x4*>(vc + b * block_bytes + head_off);
        // rows past the context (the tail of a sequence's last block) are not
        // loaded: those lanes read nothing and hold 0
        const int32_t valid = ctx - j * kBlock;
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          kt[bi][i] = i * TPL + row < valid ? __builtin_nontemporal_load(kp + i * 64 + lane) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          vt[bi][i] = i * TPL + row < valid ? __builtin_nontemporal_load(vp + i * 64 + lane) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
      const int32_t j = j0 + kWaves * BPI + bi * kWaves;
      nxt[bi] = j < blk_end ? table[j] : 0;
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

  // merge the rows of the wave (lanes that hold the same dims) ...
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
  // ... then the four waves, through LDS
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_acc[wave][col * EPL + e] = acc[e];
  }
  if (lane == 0) { sm_ml[wave][0] = m; sm_ml[wave][1] = l; sm_bad[wave] = bad ? 1 : 0; }
  __syncthreads();
  float M = 0.f, L = 0.f, o = 0.f;
  const int t = threadIdx.x;
  if (t < D) {
    M = sm_ml[0][0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) M = fmaxf(M, sm_ml[v][0]);
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float f = fast_exp2(sm_ml[v][0] - M);
      L += sm_ml[v][1] * f;
      o += sm_acc[v][t] * f;
    }
    if (sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3]) { o = __builtin_nanf(""); L = __builtin_nanf(""); }
  }
  if (np_s == 1 && base == 0) {
    if (t < D) a.out[orow + t] = o / L;
    return;
  }
  // a split context: this partition's (max, sum, accumulator) for the merge kernel
  const int64_t pidx = (static_cast<int64_t>(s) * Hq + h) * a.num_partitions + base + p;
  if (t < D) {
    a.part_acc[pidx * D + t] = o;
    if (t == 0) { a.part_ml[2 * pidx] = M; a.part_ml[2 * pidx + 1] = L; }
  }
}

// ---------------------------------------------------------------------------
// Partition merge, one workgroup per (s, h), for contexts cut into more than
// one partition:  M = max_p m_p,  out = sum_p acc_p 2^(m_p - M) / sum_p l_p
// 2^(m_p - M) -- the log-sum-exp identity that makes the split softmax equal
// the unsplit one.  A separate launch keeps the decode kernel free of
// cross-workgroup synchronisation: a device-scope release/acquire per split
// unit writes back and invalidates an XCD L2 and costs far more (measured 2x on
// the 13B-shaped batch) than this launch, whose kernel boundary publishes all
// partials at once.  It is launched only when some context can be split.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void merge_partitions_kernel(pkv_decode_args a) {
  const int64_t sh = blockIdx.x;                       // s * Hq + h
  const int32_t s = static_cast<int32_t>(sh / a.num_heads);
  if (!plan_matches(a.plan, a)) return;                // the decode kernel wrote NaN rows
  const int32_t ctx = a.context_lens[s];
  if (!len_ok(ctx, a.max_context_len, a.max_blocks_per_seq, a.block_size)) return;
  // slots 0 .. base-1 hold the shared-prefix partials (if any), then the
  // sequence's own partitions
  const int32_t start = pkvd::seq_start_of(a, s);
  const int32_t base = pkvd::slot_base_of(a, start);
  const int32_t np_s = (ctx - start + a.part_tokens - 1) / a.part_tokens;
  if (base == 0 && np_s <= 1) return;
  const int64_t prow = sh * a.num_partitions;
  a.out[sh * D + threadIdx.x] =
      pkvd::merge_partials(a.part_ml + 2 * prow, a.part_acc + prow * D + threadIdx.x, base + np_s, D);
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
  int err;
  if (pkv_uses_mfma(a.dtype, a.num_heads, a.num_kv_heads, a.block_size)) {
    err = pkv_launch_decode_group(a, stream);
  } else if (a.dtype == PKV_BF16) {
    err = a.head_dim == 128 ? launch_decode_valu<uint16_t, 128>(a, st) : launch_decode_valu<uint16_t, 64>(a, st);
  } else {
    err = a.head_dim == 128 ? launch_decode_valu<float, 128>(a, st) : launch_decode_valu<float, 64>(a, st);
  }
  // no context can be split (and no shared prefix adds partials): no merge
  if (err != hipSuccess || (a.seq_start == nullptr && a.max_context_len <= a.part_tokens)) return err;
  const uint32_t rows = static_cast<uint32_t>(a.num_seqs) * a.num_heads;
  if (a.head_dim == 128) {
    hipLaunchKernelGGL((merge_partitions_kernel<128>), dim3(rows), dim3(128), 0, st, a);
  } else {
    hipLaunchKernelGGL((merge_partitions_kernel<64>), dim3(rows), dim3(64), 0, st, a);
  }
  return hipGetLastError();
}

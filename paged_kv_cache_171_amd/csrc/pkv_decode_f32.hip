// Paged decode attention for float32 pools with grouped-query heads (2 or more
// query heads per KV head) on the gfx950 fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: exact fp32 products, fp32 accumulation).
//
// Pages cited:
//   [OS]  "PagedAttention: gestionar la KV cache como memoria de un sistema
//         operativo", "Cómo funciona por dentro": attention follows the block
//         table, scores each block, then one softmax-weighted sum;
//         "Qué significa esto para lo que pagas": decode is memory-bound.
//   [CB]  "Batching Continuo y PagedAttention", "PagedAttention: Memoria
//         virtual para la KV cache": the query heads that share a KV head
//         read the same blocks.
//
// The G query heads of a KV group are the rows of one 16-row MFMA tile, so
// every K/V row is read once for all of them (the vector-ALU kernel reads it
// once per query head); a group of more than 64 heads is cut into slices of
// 16 rows, one workgroup each (17..64 heads: the wide kernel below, one
// workgroup for all slices).  Work units are the plan's (sequence, partition)
// pairs (4096, 2048 or 1024 tokens by batch), one workgroup per (unit, KV
// head, slice); its four waves take the
// unit's 16-key tiles in turn (a tile: two 8-token blocks, one 16-token block
// or half a 32-token block) and keep an online softmax per row; the waves are
// merged through LDS, and the unit writes the output rows or the partials
// that the row's last unit to finish merges (the layout of the vector-ALU
// kernel's partials).
//
// Shared-prefix decode ([OS] "El regalo extra: compartir memoria"): the same
// body takes a fork group's shared leading blocks once for all its members,
// whose (member, query head) pairs become the tile's rows (16 / G members per
// unit); each member's own tokens are then decoded by the plain kernels in a
// second launch, and a row's last unit to finish merges it.
//
// Matrix-core layout of v_mfma_f32_16x16x4_f32: lane l, n = l % 16,
// g = l / 16, supplies A[n][g] and B[g][n] and receives D[4g + j][n] in
// register j.  The group kernel loads its operands from memory as:
//     S^T = K Q^T   k = 4m + t  <->  dim 16m + 4g + t  (lane (n, g) loads
//                   K[key n] and q[row n] at dims 16m + 4g .. +3)
//     O^T += V^T P^T  k = kk  <->  key 4g + kk, output row i of tile dt
//                   <->  dim DT i + dt (lane n loads dims DT n .. DT n + DT-1
//                   of the four V rows 4g .. 4g+3)
// so the S^T result is the P^T operand and every per-row quantity lives in
// the lanes whose n is the row.  The wide kernel reads V from LDS as each
// lane's own 16-byte slots instead (output row i of tile dt <-> dim
// 4i + 64(dt/4) + dt%4), like the float32 prefill kernel.
#include "pkv_device.h"

namespace {

using pkvd::fast_exp2;
using pkvd::kNegBig;
using pkvd::kPlanHdr;
using pkvd::load_block_id;
using pkvd::max_over_rows;
using pkvd::plan_matches;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroupWaves = 4;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max4(f32x4 v) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0], v[1]),
                                       __builtin_elementwise_maximum(v[2], v[3]));
}

// Two waves per SIMD: each wave holds the K and V rows of two tiles (the next
// one loads while this one is on the matrix cores).
template <int D, int BS>
__device__ __forceinline__ void decode_group_f32_body(const pkv_decode_args& a, uint32_t bid, bool shared_unit) {
  constexpr int KQ = D / 16;   // 16-byte pieces of a K or q row per lane
  constexpr int DT = D / 16;   // 16-dim output tiles; a lane holds DT dims of each of its V rows
  constexpr int DV = DT / 4;   // 16-byte pieces of those
  constexpr int kT = 16;       // keys per tile
  constexpr int OROW = D + 4;  // padded LDS row (floats) of the wave merge
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int64_t kHeadTile = static_cast<int64_t>(BS) * D;   // floats of one (block, head) tile
  __shared__ float sm_o[kGroupWaves][16][OROW];
  __shared__ float sm_ml[kGroupWaves][16][2];
  __shared__ int sm_bad[kGroupWaves];
  __shared__ int sm_last;
  __shared__ int sm_member_last[16], sm_member_slots[16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;

  const int32_t Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  // 16-row slices of the group (shared-prefix units have G <= 16: one slice)
  const int32_t nsl = shared_unit ? 1 : (G + 15) / 16;
  // the slices of one (unit, KV head) get workgroup ids 8 apart, i.e. one XCD
  // (workgroups go to the 8 XCDs in turn), so they read its K/V through one L2
  const uint32_t x = nsl == 1 ? bid : (bid / (8u * nsl)) * 8u + bid % 8u;
  const int32_t slice = nsl == 1 ? 0 : static_cast<int32_t>((bid / 8u) % static_cast<uint32_t>(nsl));
  const int32_t u = static_cast<int32_t>(x / static_cast<uint32_t>(Hkv));
  const int32_t kvh = static_cast<int32_t>(x - static_cast<uint32_t>(u) * Hkv);
  const int32_t R = min(16, G - 16 * slice);          // rows of this slice
  const int32_t hb = kvh * G + 16 * slice;            // query head of row 0
  // The unit: rows r < nrows are (sequence s0 + r / GR, query head hb + r % GR);
  // it walks the 16-key tiles t_begin .. t_end-1 of s0's context, keys below
  // ctx valid, and writes the output rows (direct) or partial slot `slot` of
  // each row.
  int32_t s0, nrows, GR, ctx, t_begin, t_end, slot, nslots = 0;
  bool direct;
  if (shared_unit) {
    // a group's shared leading blocks: the rows are the group's sequences (a
    // plan built for other sizes runs no shared unit; the sequences' own units
    // then write NaN rows)
    const int32_t* sp = a.shared_plan;
    if (!pkvd::shared_plan_matches(sp, a) || u >= sp[0]) return;
    const int32_t* su = sp + kPlanHdr + 4 * u;
    s0 = su[0];
    nrows = min(su[1], 16 / G) * G;
    GR = G;
    ctx = su[3];
    t_begin = su[2] * (a.prefix_part_tokens / kT);
    t_end = min(ctx / kT, t_begin + a.prefix_part_tokens / kT);
    slot = su[2];
    direct = false;
  } else {
    const int32_t* plan = a.plan;
    if (!plan_matches(plan, a)) {
      // a plan built for other sizes: every row is NaN
      if (u < a.num_seqs)
        for (int idx = threadIdx.x; idx < R * D; idx += 64 * kGroupWaves)
          a.out[(static_cast<int64_t>(u) * Hq + hb) * D + idx] = __builtin_nanf("");
      return;
    }
    if (u >= plan[0]) return;
    const int32_t* units = pkvd::plan_units(plan);
    const int32_t s = units[2 * u];
    const int32_t p = units[2 * u + 1];
    ctx = a.context_lens[s];
    if (p < 0) {
      // no attention work: an empty context gives 0, an invalid one NaN
      for (int idx = threadIdx.x; idx < R * D; idx += 64 * kGroupWaves)
        a.out[(static_cast<int64_t>(s) * Hq + hb) * D + idx] = ctx == 0 ? 0.f : __builtin_nanf("");
      return;
    }
    const int32_t part = a.part_tokens;
    const int32_t start = pkvd::seq_start_of(a, s);
    const int32_t base = pkvd::slot_base_of(a, start);
    const int32_t np_s = (ctx - start + part - 1) / part;
    s0 = s;
    nrows = R;
    GR = R;
    t_begin = start / kT + p * (part / kT);
    t_end = min((ctx + kT - 1) / kT, t_begin + part / kT);
    slot = base + p;
    nslots = base + np_s;
    direct = np_s == 1 && base == 0;
  }
  const int32_t ntiles = (ctx + kT - 1) / kT;

  const int64_t block_stride = static_cast<int64_t>(Hkv) * kHeadTile;
  float* const kc = const_cast<float*>(static_cast<const float*>(a.k_cache)) + kvh * kHeadTile;
  float* const vc = const_cast<float*>(static_cast<const float*>(a.v_cache)) + kvh * kHeadTile;
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s0) * a.max_blocks_per_seq;
  const int32_t nblk = (ctx + BS - 1) / BS;

  // q of the unit's rows as the B operand (rows >= nrows: q = 0, never written)
  f32x4 qv[KQ];
  {
    const int32_t hr = n < nrows ? n : 0;
    const float* qrow = static_cast<const float*>(a.q) + ((static_cast<int64_t>(s0) + hr / GR) * Hq + hb + hr % GR) * D;
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(qrow + 16 * m + 4 * g);
      qv[m] = n < nrows ? w : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // The step's new token (decode with the cache write): in the tile of token
  // ctx-1 its K and V rows come from the step's rows when the new slot is
  // token ctx-1's, and the lanes holding them store them into the pool; a
  // slot elsewhere gives NaN rows and stores nothing.
  const int64_t new_slot = (a.new_slots && !shared_unit) ? a.new_slots[s0] : -1;
  const int32_t last_tile = ntiles - 1;
  const int32_t last_row = (ctx - 1) % kT;
  const float* nk = a.new_k ? static_cast<const float*>(a.new_k) + (static_cast<int64_t>(s0) * Hkv + kvh) * D : nullptr;
  const float* nv = a.new_v ? static_cast<const float*>(a.new_v) + (static_cast<int64_t>(s0) * Hkv + kvh) * D : nullptr;

  const float c2 = a.scale_log2;               // scale * log2(e), any sign
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, lsum = 0.f;
  bool bad = false;

  // The tile's block ids (wave-uniform): its block, or with 8-token blocks its
  // two (the second clamped to the context's last block: keys past the context
  // are never read from it); a key past the context reads the tile's first key
  // instead (a cached token: finite data, masked to probability 0).
  auto load_tile = [&](int32_t it, f32x4 (&kv)[KQ], f32x4 (&vv)[4][DV]) {
    const int32_t t = t_begin + wave + kGroupWaves * it;
    const int32_t key0 = kT * t;
    const int32_t j0 = key0 / BS;
    const int32_t raw_a = load_block_id(table, __builtin_amdgcn_readfirstlane(j0));
    int32_t raw_b = raw_a;
    if constexpr (BS == 8) raw_b = load_block_id(table, __builtin_amdgcn_readfirstlane(min(j0 + 1, nblk - 1)));
    int32_t id_a = raw_a, id_b = raw_b;
    if (static_cast<uint32_t>(id_a) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; id_a = 0; }
    if (static_cast<uint32_t>(id_b) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; id_b = 0; }
    bool from_new = false;
    int32_t id_last = 0;
    if (t == last_tile && new_slot >= 0) {
      const int32_t raw_last = (BS == 8 && last_row >= 8) ? raw_b : raw_a;
      from_new = static_cast<uint32_t>(raw_last) < static_cast<uint32_t>(a.num_blocks) &&
                 new_slot == static_cast<int64_t>(raw_last) * BS + (ctx - 1) % BS;
      if (!from_new) bad = true;
      id_last = raw_last;
    }
    auto row_ptr = [&](const float* pool, const float* fresh, int32_t off) {
      if (from_new && key0 + off == ctx - 1) return fresh;
      const int32_t o2 = key0 + off < ctx ? off : 0;
      const int32_t id = (BS == 8 && o2 >= 8) ? id_b : id_a;
      return pool + id * block_stride + ((key0 + o2) % BS) * D;
    };
    {
      const float* krow = row_ptr(kc, nk, n);
#pragma unroll
      for (int m = 0; m < KQ; ++m) kv[m] = *reinterpret_cast<const f32x4*>(krow + 16 * m + 4 * g);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float* vrow = row_ptr(vc, nv, 4 * g + kk) + DT * n;
#pragma unroll
      for (int c = 0; c < DV; ++c) vv[kk][c] = *reinterpret_cast<const f32x4*>(vrow + 4 * c);
    }
    if (from_new && slice == 0) {
      // the new token's rows into the pool (by the first slice's workgroup):
      // K from the lanes of key row last_row, V from the lanes of group
      // last_row / 4
      const int64_t dst = id_last * block_stride + static_cast<int64_t>((ctx - 1) % BS) * D;
      if (n == last_row) {
#pragma unroll
        for (int m = 0; m < KQ; ++m) *reinterpret_cast<f32x4*>(kc + dst + 16 * m + 4 * g) = kv[m];
      }
      if (g == last_row / 4) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          if (kk == last_row % 4) {
#pragma unroll
            for (int c = 0; c < DV; ++c) *reinterpret_cast<f32x4*>(vc + dst + DT * n + 4 * c) = vv[kk][c];
          }
      }
    }
  };
  // S^T = K Q^T (two accumulator chains), the online softmax over the tile's
  // 16 keys (base 2, maximum taken every tile), then O^T += V^T P^T
  auto compute_tile = [&](int32_t it, const f32x4 (&kv)[KQ], const f32x4 (&vv)[4][DV]) {
    const int32_t key0 = kT * (t_begin + wave + kGroupWaves * it);
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
    for (int m = 0; m < KQ; ++m)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (m & 1) acc1 = mfma4(kv[m][tt], qv[m][tt], acc1);
        else acc0 = mfma4(kv[m][tt], qv[m][tt], acc0);
      }
    f32x4 sc = (acc0 + acc1) * c2;               // S[row n][key key0 + 4g + j], base 2
    if (key0 + kT > ctx) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (key0 + 4 * g + j >= ctx) sc[j] = -INFINITY;
    }
    const float mx = max_over_rows(max4(sc));
    const float mnew = __builtin_elementwise_maximum(m_run, mx);
    const float alpha = fast_exp2(m_run - mnew);
    m_run = mnew;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(sc[j] - m_run);
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) o[dt] = mfma4(vv[kk][dt / 4][dt % 4], pr[kk], o[dt]);
  };
  // this wave's tiles t_begin + wave, + 4, ...; two register sets, the loop
  // unrolled by two so that each stays in place
  const int32_t nit = (t_end - t_begin - wave + kGroupWaves - 1) / kGroupWaves;
  f32x4 kA[KQ], vA[4][DV], kB[KQ], vB[4][DV];
  if (nit > 0) load_tile(0, kA, vA);
  for (int32_t it = 0; it < nit; it += 2) {
    if (it + 1 < nit) load_tile(it + 1, kB, vB);
    compute_tile(it, kA, vA);
    if (it + 1 >= nit) break;
    if (it + 2 < nit) load_tile(it + 2, kA, vA);
    compute_tile(it + 1, kB, vB);
  }

  // merge the four waves through LDS: lane (n, g) holds dims DT (4g + j) + dt
  // of row n in o[dt][j]; its row's sum is spread over the four lane groups
  float L = lsum;
  L += __shfl_xor(L, 16);
  L += __shfl_xor(L, 32);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) sm_o[wave][n][DT * (4 * g + j) + dt] = o[dt][j];
  if (g == 0) { sm_ml[wave][n][0] = m_run; sm_ml[wave][n][1] = L; }
  if (lane == 0) sm_bad[wave] = bad ? 1 : 0;
  __syncthreads();
  const bool any_bad = (sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3]) != 0;
  for (int idx = threadIdx.x; idx < nrows * D; idx += 64 * kGroupWaves) {
    const int r = idx / D, d = idx - (idx / D) * D;
    float M = sm_ml[0][r][0];
#pragma unroll
    for (int w = 1; w < kGroupWaves; ++w) M = fmaxf(M, sm_ml[w][r][0]);
    float Ls = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
      const float f = fast_exp2(sm_ml[w][r][0] - M);
      Ls += sm_ml[w][r][1] * f;
      acc += sm_o[w][r][d] * f;
    }
    if (any_bad) { acc = __builtin_nanf(""); Ls = __builtin_nanf(""); }
    const int64_t row = (static_cast<int64_t>(s0) + r / GR) * Hq + hb + r % GR;
    if (direct) {
      a.out[row * D + d] = acc / Ls;
    } else {
      const int64_t pidx = row * a.num_partitions + slot;
      pkvd::store_coherent(a.part_acc + pidx * D + d, acc);
      if (d == 0) { pkvd::store_coherent(a.part_ml + 2 * pidx, M); pkvd::store_coherent(a.part_ml + 2 * pidx + 1, Ls); }
    }
  }
  if (direct) return;
  if (!shared_unit) {
    // a split context: the last of the sequence's units (for this KV head and
    // slice) to finish merges its rows
    const int64_t row0 = static_cast<int64_t>(s0) * Hq + hb;
    if (!pkvd::arrive_last(a.merge_tickets + row0, a.merge_epoch, nslots, &sm_last)) return;
    for (int idx = threadIdx.x; idx < R * D; idx += 64 * kGroupWaves) {
      const int64_t prow = (row0 + idx / D) * a.num_partitions;
      const int d = idx - (idx / D) * D;
      a.out[(row0 + idx / D) * D + d] = pkvd::merge_partials_coherent(a.part_ml + 2 * prow,
                                                                      a.part_acc + prow * D + d, nslots, D);
    }
    return;
  }
  // a shared-prefix unit arrives once for each member sequence (on the ticket
  // of its G rows, counting its prefix and its own partitions) and merges the
  // members it was the last unit of
  const int32_t members = nrows / G;
  pkvd::wait_vmem();
  __syncthreads();
  if (threadIdx.x < members) {
    const int32_t s = s0 + threadIdx.x;
    const int32_t start = pkvd::seq_start_of(a, s);
    const int32_t slots = pkvd::slot_base_of(a, start) + (a.context_lens[s] - start + a.part_tokens - 1) / a.part_tokens;
    sm_member_slots[threadIdx.x] = slots;
    sm_member_last[threadIdx.x] =
        pkvd::ticket_arrive(a.merge_tickets + static_cast<int64_t>(s) * Hq + kvh * G, a.merge_epoch, slots) ? 1 : 0;
  }
  __syncthreads();
  for (int32_t mi = 0; mi < members; ++mi) {
    if (!sm_member_last[mi]) continue;
    const int32_t slots = sm_member_slots[mi];
    const int64_t row0 = static_cast<int64_t>(s0 + mi) * Hq + kvh * G;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * kGroupWaves) {
      const int64_t prow = (row0 + idx / D) * a.num_partitions;
      const int d = idx - (idx / D) * D;
      a.out[(row0 + idx / D) * D + d] = pkvd::merge_partials_coherent(a.part_ml + 2 * prow,
                                                                      a.part_acc + prow * D + d, slots, D);
    }
  }
}

template <int D, int BS>
__global__ __launch_bounds__(64 * kGroupWaves, 2) void decode_group_f32_kernel(pkv_decode_args a) {
  decode_group_f32_body<D, BS>(a, blockIdx.x, false);
}

// The shared-prefix units of a shared-prefix decode (one workgroup per
// possible unit and KV head; those past the shared plan's count exit).
template <int D, int BS>
__global__ __launch_bounds__(64 * kGroupWaves, 2) void decode_shared_f32_kernel(pkv_decode_args a) {
  decode_group_f32_body<D, BS>(a, blockIdx.x, true);
}

// ---------------------------------------------------------------------------
// Decode for wide query-head groups over float32 pools: 17..64 query heads per
// KV head.  One workgroup per (unit, KV head) for all the group's 16-row
// slices: each 16-key tile's K and V rows are copied once into LDS (a ring of
// three stages, direct global->LDS copies two tiles ahead, one barrier per
// tile; K rows' 16-byte slots XOR-swizzled by row) and wave w computes slice
// w from there, so each K/V byte crosses from L2 into the CU once instead of
// once per slice workgroup.  Scores and the merge are those of the group
// kernel above; a row's running maximum moves only once a score passes it by
// 2^8 (so most tiles skip the rescale of O), and V is read as each lane's own
// 16-byte slots (lane n: dims 4n.. and 64 + 4n..), which keeps the 16 lanes
// of a read in distinct banks.  The cache write copies token
// ctx-1's rows into the stage from the step's rows and the workgroup stores
// them into the pool.  Partitions start at multiples of 1024 tokens (wide
// groups take no shared prefix).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_addr_f32(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}
__device__ __forceinline__ void copy16_to_lds_f32(const void* p, const void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(p), "{m0}"(lds_addr_f32(lds)) : "memory");
}
__device__ __forceinline__ f32x4 lds_read16_f32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ void copy16_to_lds_at_f32(const char* base, uint32_t voff, const void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_addr_f32(lds)) : "memory");
}
template <int N> __device__ __forceinline__ void wait_vm_f32() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

template <int D, int BS>
__global__ __launch_bounds__(64 * kGroupWaves, 3) void decode_wide_group_f32_kernel(pkv_decode_args a) {
  constexpr int KQ = D / 16;   // 16-byte pieces of a K or q row per lane
  constexpr int DT = D / 16;   // 16-dim output tiles; a lane holds DT dims of each of its V rows
  constexpr int DV = DT / 4;   // 16-byte pieces of those
  constexpr int RB = D * 4;    // bytes per K or V row
  constexpr int kSlots = RB / 16;
  constexpr int kTileBytes = 16 * RB;
  constexpr int kTileKiB = kTileBytes / 1024;
  constexpr int kStageBytes = 2 * kTileBytes;          // K then V
  constexpr int kThreads = 64 * kGroupWaves;
  constexpr int kCopies = kStageBytes / (16 * kThreads);
  constexpr int kStages = 3;
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(kStageBytes % (16 * kThreads) == 0 && (kCopies == 2 || kCopies == 4), "stage shape");
  constexpr int64_t kHeadTile = static_cast<int64_t>(BS) * D;   // floats of one (block, head) tile
  __shared__ __align__(16) char ring[kStages][kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;

  const int32_t Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  const int32_t nsl = (G + 15) / 16;               // 2..4 slices
  const bool active = wave < nsl;
  const int32_t R = active ? min(16, G - 16 * wave) : 0;
  const uint32_t bid = blockIdx.x;
  const int32_t* plan = a.plan;
  if (!plan_matches(plan, a)) {
    // a plan built for other sizes: every row is NaN
    const int32_t u0 = static_cast<int32_t>(bid / static_cast<uint32_t>(Hkv));
    const int32_t kvh0 = static_cast<int32_t>(bid - static_cast<uint32_t>(u0) * Hkv);
    if (u0 < a.num_seqs)
      for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
        a.out[(static_cast<int64_t>(u0) * Hq + kvh0 * G) * D + idx] = __builtin_nanf("");
    return;
  }
  // rounds of 256 workgroups (one per CU) in alternating order, so that the
  // longest units (listed first) share a CU with the shortest of the next round
  const uint32_t live = static_cast<uint32_t>(plan[0]) * static_cast<uint32_t>(Hkv);
  if (bid >= live) return;
  const uint32_t rnd = bid / 256u, rk = bid % 256u;
  const uint32_t nr = min(256u, live - rnd * 256u);
  const uint32_t b2 = (rnd & 1u) ? rnd * 256u + (nr - 1u - rk) : bid;
  const int32_t u = static_cast<int32_t>(b2 / static_cast<uint32_t>(Hkv));
  const int32_t kvh = static_cast<int32_t>(b2 - static_cast<uint32_t>(u) * Hkv);
  const int32_t* units = pkvd::plan_units(plan);
  const int32_t s = units[2 * u];
  const int32_t p = units[2 * u + 1];
  const int32_t ctx = a.context_lens[s];
  const int64_t grow0 = static_cast<int64_t>(s) * Hq + kvh * G;   // the group's first output row
  if (p < 0) {
    // no attention work: an empty context gives 0, an invalid one NaN
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
      a.out[grow0 * D + idx] = ctx == 0 ? 0.f : __builtin_nanf("");
    return;
  }
  const int32_t part = a.part_tokens;
  const int32_t np_s = (ctx + part - 1) / part;
  const int32_t k_begin = p * part;
  const int32_t k_end = min(ctx, k_begin + part);
  const int32_t ntiles = (k_end - k_begin + 15) / 16;
  const bool direct = np_s == 1;
  const int32_t nblk = (ctx + BS - 1) / BS;
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const int64_t block_bytes = static_cast<int64_t>(Hkv) * kHeadTile * 4;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache) + kvh * kHeadTile * 4;
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache) + kvh * kHeadTile * 4;
  bool bad = false;

  // The step's new token: the unit that holds token ctx-1 checks its slot.
  const int64_t new_slot = (a.new_slots && k_end == ctx) ? a.new_slots[s] : -1;
  int32_t new_blk = 0;
  bool use_new = false;
  if (new_slot >= 0) {
    new_blk = load_block_id(table, __builtin_amdgcn_readfirstlane((ctx - 1) / BS));
    use_new = static_cast<uint32_t>(new_blk) < static_cast<uint32_t>(a.num_blocks) &&
              new_slot == static_cast<int64_t>(new_blk) * BS + (ctx - 1) % BS;
    if (!use_new) bad = true;      // not token ctx-1's slot: NaN rows, nothing stored
  }
  const char* nk = use_new ? reinterpret_cast<const char*>(a.new_k) + (static_cast<int64_t>(s) * Hkv + kvh) * RB
                           : nullptr;
  const char* nv = use_new ? reinterpret_cast<const char*>(a.new_v) + (static_cast<int64_t>(s) * Hkv + kvh) * RB
                           : nullptr;

  // Copy c of wave w fills KiB kGroupWaves*c + w of a stage: tile half t (0: K,
  // 1: V), rows in lane order; K's LDS slot k holds the row's slot k ^ (row
  // mod slots).  A 1 KiB copy reads rows of one pool block.
  uint32_t cp_off[kCopies], cp_slot[kCopies];
  int32_t cp_key[kCopies];
#pragma unroll
  for (int c = 0; c < kCopies; ++c) {
    const int kib = kGroupWaves * c + wave;
    const int t = kib / kTileKiB;
    const int off = (kib % kTileKiB) * 1024 + 16 * lane;
    const int row = off / RB, k = (off % RB) / 16;
    const int slot = t == 0 ? (k ^ (row % kSlots)) : k;
    cp_key[c] = row;
    cp_off[c] = static_cast<uint32_t>((row % BS) * RB + 16 * slot);
    cp_slot[c] = static_cast<uint32_t>(16 * slot);
  }
  // the tile's block ids: the block of its rows 0-7 and of rows 8-15 (the
  // same unless blocks hold 8 tokens; the second clamped to the last block)
  auto tile_ids = [&](int32_t tt, int32_t& ida, int32_t& idb) {
    const int32_t j0 = (k_begin + 16 * tt) / BS;
    ida = load_block_id(table, __builtin_amdgcn_readfirstlane(j0));
    idb = ida;
    if constexpr (BS == 8) idb = load_block_id(table, __builtin_amdgcn_readfirstlane(min(j0 + 1, nblk - 1)));
  };
  auto issue = [&](int32_t tt, int32_t ida, int32_t idb, char* stage) {
    if (static_cast<uint32_t>(ida) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; ida = 0; }
    if (static_cast<uint32_t>(idb) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; idb = 0; }
    const int32_t key0 = k_begin + 16 * tt;
    if (key0 + 16 < ctx) {
      // a tile wholly before token ctx-1: each copy reads rows of one block
      // (with 8-token blocks: both rows in one half of the tile)
#pragma unroll
      for (int c = 0; c < kCopies; ++c) {
        const int kib = kGroupWaves * c + wave;
        const int t = kib / kTileKiB;
        const bool hi = BS == 8 && (kib % kTileKiB) * 1024 / RB >= 8;
        const char* base = (t == 0 ? kc : vc) + static_cast<int64_t>(hi ? idb : ida) * block_bytes + (key0 % BS) * RB;
        copy16_to_lds_at_f32(base, cp_off[c], stage + kib * 1024);
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < kCopies; ++c) {
      const int kib = kGroupWaves * c + wave;
      const int t = kib / kTileKiB;
      const int32_t key = key0 + cp_key[c];
      const int32_t id = (BS == 8 && cp_key[c] >= 8) ? idb : ida;
      // (a 32-token block holds two tiles: the tile's rows start at key0 mod BS);
      // keys past the context read row 0 of the tile (finite data, masked)
      const char* src = key < ctx ? (t == 0 ? kc : vc) + id * block_bytes + (key0 % BS) * RB + cp_off[c]
                                  : (t == 0 ? kc : vc) + ida * block_bytes + (key0 % BS) * RB + cp_slot[c];
      if (use_new && key == ctx - 1) src = (t == 0 ? nk : nv) + cp_slot[c];
      copy16_to_lds_f32(src, stage + kib * 1024);
    }
  };

#pragma unroll
  for (int tt = 0; tt < kStages - 1; ++tt)
    if (tt < ntiles) {
      int32_t ida, idb;
      tile_ids(tt, ida, idb);
      issue(tt, ida, idb, ring[tt]);
    }
  int32_t nida = 0, nidb = 0;
  if (kStages - 1 < ntiles) tile_ids(kStages - 1, nida, nidb);

  // the wave's query rows as the B operand (rows >= R: q = 0, never written;
  // a wave without a slice reads the group's first row and zeroes it)
  f32x4 qv[KQ];
  {
    const float* qrow = static_cast<const float*>(a.q) + (grow0 + (n < R ? 16 * wave + n : 0)) * D;
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(qrow + 16 * m + 4 * g);
      qv[m] = n < R ? w : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const float c2 = a.scale_log2;               // scale * log2(e), any sign
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, thr = kNegBig, lsum = 0.f;

  const uint32_t ring0 = lds_addr_f32(ring[0]);
  uint32_t k_addr[KQ];
#pragma unroll
  for (int m = 0; m < KQ; ++m) {
    k_addr[m] = ring0 + n * RB + 16 * ((4 * m + g) ^ (n % kSlots));
    asm volatile("" : "+v"(k_addr[m]));
  }
  uint32_t v_addr = ring0 + kTileBytes + 4 * g * RB + 16 * n;
  asm volatile("" : "+v"(v_addr));

  auto compute_tile = [&](int32_t tt, uint32_t stage_off) {
    const int32_t key0 = k_begin + 16 * tt;
    f32x4 kv[KQ];
#pragma unroll
    for (int m = 0; m < KQ; ++m) kv[m] = lds_read16_f32(k_addr[m] + stage_off);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    f32x4 acc[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) acc[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KQ; ++m)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) acc[t4] = mfma4(kv[m][t4], qv[m][t4], acc[t4]);
    __builtin_amdgcn_s_setprio(0);
    const f32x4 acc0 = acc[0] + acc[2], acc1 = acc[1] + acc[3];
    f32x4 vv[4][DV];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int c = 0; c < DV; ++c) vv[kk][c] = lds_read16_f32(v_addr + stage_off + kk * RB + 256 * c);
    f32x4 sc = (acc0 + acc1) * c2;               // S[row n][key key0 + 4g + j], base 2
    if (key0 + 16 > ctx) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (key0 + 4 * g + j >= ctx) sc[j] = -INFINITY;
    }
    const float lane_mx = max4(sc);
    if (__builtin_amdgcn_ballot_w64(lane_mx > thr)) {
      // a row's running maximum moves only once a score passes it by 2^8
      const float mx = max_over_rows(lane_mx);
      const bool up = mx > thr;
      const float mnew = up ? mx : m_run;
      const float alpha = fast_exp2(m_run - mnew);
      m_run = mnew;
      thr = up ? mx + 8.f : thr;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(sc[j] - m_run);
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) o[dt] = mfma4(vv[kk][dt / 4][dt % 4], pr[kk], o[dt]);
    __builtin_amdgcn_s_setprio(0);
  };

  for (int32_t t0 = 0; t0 < ntiles; t0 += kStages) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int32_t tt = t0 + st;
      if (tt >= ntiles) break;
      // this tile's copies have landed once at most the next tile's copies are
      // outstanding (copies complete in issue order)
      if (tt + 1 < ntiles) wait_vm_f32<kCopies>();
      else wait_vm_f32<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int32_t tn = tt + kStages - 1;
      const int32_t ida = nida, idb = nidb;
      if (tn + 1 < ntiles) tile_ids(tn + 1, nida, nidb);
      __builtin_amdgcn_s_barrier();
      if (active) compute_tile(tt, static_cast<uint32_t>(st * kStageBytes));
      if (tn < ntiles) issue(tn, ida, idb, ring[(st + kStages - 1) % kStages]);
    }
  }

  // a bad block id anywhere in the unit's range, or a wrong new slot, poisons
  // its rows (every wave checks the same ids and slot: the flag is the same on
  // every thread, so no vote through LDS)
  const bool any_bad = bad;
  if (use_new && threadIdx.x < 2 * RB / 16) {
    // the new token's K and V rows into the pool (16 bytes per thread)
    const int half = threadIdx.x / (RB / 16), piece = threadIdx.x % (RB / 16);
    const char* src = (half == 0 ? nk : nv) + 16 * piece;
    char* dst = const_cast<char*>(half == 0 ? kc : vc) + new_blk * block_bytes + ((ctx - 1) % BS) * RB + 16 * piece;
    *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
  }
  if (!active) return;
  float L = lsum;
  L += __shfl_xor(L, 16);
  L += __shfl_xor(L, 32);
  const int64_t row0 = grow0 + 16 * wave;          // the wave's first row
  // lane (n, g) holds dims 16g + 4j + 64(dt/4) + dt%4 of row n in o[dt][j]
  if (direct) {
    if (n < R) {
      const float inv = any_bad ? __builtin_nanf("") : 1.f / L;
      float* orow = a.out + (row0 + n) * D;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < DV; ++c) {
          const f32x4 v = f32x4{o[4 * c][j], o[4 * c + 1][j], o[4 * c + 2][j], o[4 * c + 3][j]} * inv;
          *reinterpret_cast<f32x4*>(orow + 16 * g + 4 * j + 64 * c) = v;
        }
    }
    return;
  }
  // a split context: the wave's partial, then one step on its slice's ticket
  if (n < R) {
    const int64_t pidx = (row0 + n) * a.num_partitions + p;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        pkvd::store_coherent(a.part_acc + pidx * D + 16 * g + 4 * j + 64 * (dt / 4) + dt % 4,
                             any_bad ? __builtin_nanf("") : o[dt][j]);
    if (g == 0) {
      pkvd::store_coherent(a.part_ml + 2 * pidx, m_run);
      pkvd::store_coherent(a.part_ml + 2 * pidx + 1, any_bad ? __builtin_nanf("") : L);
    }
  }
  pkvd::wait_vmem();
  int last = 0;
  if (lane == 0) last = pkvd::ticket_arrive(a.merge_tickets + row0, a.merge_epoch, np_s) ? 1 : 0;
  last = __shfl(last, 0);
  if (!last) return;
  for (int idx = lane; idx < R * D; idx += 64) {
    const int64_t prow = (row0 + idx / D) * a.num_partitions;
    const int d = idx - (idx / D) * D;
    a.out[(row0 + idx / D) * D + d] =
        pkvd::merge_partials_coherent(a.part_ml + 2 * prow, a.part_acc + prow * D + d, np_s, D);
  }
}

template <int D>
void launch_bs(int block_size, dim3 grid, hipStream_t st, const pkv_decode_args& a, bool shared) {
  if (shared) {
    if (block_size == 8)
      hipLaunchKernelGGL((decode_shared_f32_kernel<D, 8>), grid, dim3(64 * kGroupWaves), 0, st, a);
    else if (block_size == 32)
      hipLaunchKernelGGL((decode_shared_f32_kernel<D, 32>), grid, dim3(64 * kGroupWaves), 0, st, a);
    else
      hipLaunchKernelGGL((decode_shared_f32_kernel<D, 16>), grid, dim3(64 * kGroupWaves), 0, st, a);
    return;
  }
  if (block_size == 8)
    hipLaunchKernelGGL((decode_group_f32_kernel<D, 8>), grid, dim3(64 * kGroupWaves), 0, st, a);
  else if (block_size == 32)
    hipLaunchKernelGGL((decode_group_f32_kernel<D, 32>), grid, dim3(64 * kGroupWaves), 0, st, a);
  else
    hipLaunchKernelGGL((decode_group_f32_kernel<D, 16>), grid, dim3(64 * kGroupWaves), 0, st, a);
}

}  // namespace

int pkv_launch_decode_group_f32(const pkv_decode_args& a, void* stream) {
  const int64_t np = (a.max_context_len + a.part_tokens - 1) / a.part_tokens;
  if (pkv_wide_group(a.dtype, a.num_heads, a.num_kv_heads)) {
    // one workgroup per (unit, KV head) for all the group's slices
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.num_seqs) * (np < 1 ? 1 : np) * a.num_kv_heads));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 block(64 * kGroupWaves);
    if (a.head_dim == 128) {
      if (a.block_size == 8) hipLaunchKernelGGL((decode_wide_group_f32_kernel<128, 8>), grid, block, 0, st, a);
      else if (a.block_size == 32) hipLaunchKernelGGL((decode_wide_group_f32_kernel<128, 32>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((decode_wide_group_f32_kernel<128, 16>), grid, block, 0, st, a);
    } else {
      if (a.block_size == 8) hipLaunchKernelGGL((decode_wide_group_f32_kernel<64, 8>), grid, block, 0, st, a);
      else if (a.block_size == 32) hipLaunchKernelGGL((decode_wide_group_f32_kernel<64, 32>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((decode_wide_group_f32_kernel<64, 16>), grid, block, 0, st, a);
    }
    return hipGetLastError();
  }
  const int32_t slices = (a.num_heads / a.num_kv_heads + 15) / 16;
  const int64_t units = static_cast<int64_t>(a.num_seqs) * (np < 1 ? 1 : np) * a.num_kv_heads;
  const int64_t grid = slices == 1 ? units : (units + 7) / 8 * 8 * slices;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.head_dim == 128) launch_bs<128>(a.block_size, dim3(static_cast<uint32_t>(grid)), st, a, false);
  else launch_bs<64>(a.block_size, dim3(static_cast<uint32_t>(grid)), st, a, false);
  return hipGetLastError();
}

// The shared-prefix units over float32 pools (the sequences' own units follow
// in a launch of the plain decode kernels).
int pkv_launch_shared_units_f32(const pkv_decode_args& a, void* stream) {
  const int64_t npp = (a.max_context_len + a.prefix_part_tokens - 1) / a.prefix_part_tokens;
  const int64_t shared = static_cast<int64_t>(a.num_seqs) * (npp < 1 ? 1 : npp) * a.num_kv_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.head_dim == 128) launch_bs<128>(a.block_size, dim3(static_cast<uint32_t>(shared)), st, a, true);
  else launch_bs<64>(a.block_size, dim3(static_cast<uint32_t>(shared)), st, a, true);
  return hipGetLastError();
}

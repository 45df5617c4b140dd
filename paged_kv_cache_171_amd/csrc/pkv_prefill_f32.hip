// Causal chunked-prefill attention for float32 pools on the gfx950 fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: exact fp32 products, fp32 accumulation).
//
// Pages cited:
//   [UL]  "Continuous Batching" (Ultralytics glossary), "Cómo funciona la
//         planificación a nivel de iteración" and "Límites y técnicas
//         complementarias": long prompts are prefilled in chunks that share a
//         step with other sequences' decode.
//   [OS]  "PagedAttention: gestionar la KV cache como memoria de un sistema
//         operativo", "Cómo funciona por dentro": attention follows the block
//         table, scores each block, then one softmax-weighted sum.
//
// Sequence s owns query tokens q0..q1-1 (n = q1 - q0, the last n tokens of its
// context of ctx tokens); query i sits at position ctx - n + i and attends keys
// 0..ctx-n+i.  The rows of KV head kvh are (query i, head kvh*G + r), r < G,
// numbered token-major; each wave takes one 16-row tile and walks its keys 16
// at a time (a 16-key tile: two 8-token blocks, one 16-token block or half a
// 32-token block); a workgroup's four waves take neighbouring row tiles of one
// (sequence, KV head) and share each key tile: its K and V rows are copied
// once into LDS (a ring of three stages, direct global->LDS copies two tiles
// ahead, one barrier per tile) and every wave reads its operands from there.
//
// Matrix-core layout of v_mfma_f32_16x16x4_f32: lane l, n = l % 16,
// g = l / 16, supplies A[n][g] and B[g][n] and receives D[4g + j][n] in
// register j.  The k index of a product can be any bijection shared by A and
// B; this kernel picks them so that every lane loads whole 16-byte pieces:
//     S^T = K Q^T   k = 4m + t  <->  dim 16m + 4g + t  (lane (n, g) loads
//                   K[key n] and Q[row n] at dims 16m + 4g .. +3)
//     O^T += V^T P^T  k = kk  <->  key 4g + kk, and output row i of tile dt
//                   <->  dim 4i + 64(dt/4) + dt%4 (lane n loads its 16-byte
//                   slots n and 16 + n of the four V rows 4g .. 4g+3, so the
//                   16 lanes of a read fall in distinct banks)
// so the S^T result, lane (n, g) holding S[row n][key 4g + j], is already the
// P^T operand, and every per-row quantity lives in the lanes whose n is the
// row.  The softmax is the online one in base 2; a row's running maximum
// moves only once a score passes it by 2^8 (P stays below 256 and exact
// fp32), so most tiles skip the rescale of O.
#include "pkv_device.h"

namespace {

using pkvd::fast_exp2;
using pkvd::kNegBig;
using pkvd::len_ok;
using pkvd::load_block_id;
using pkvd::max_over_rows;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kF32Waves = kPrefillF32RowsPerWg / 16;   // one 16-row tile per wave

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max4(f32x4 v) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0], v[1]),
                                       __builtin_elementwise_maximum(v[2], v[3]));
}

// LDS copy helpers (direct global->LDS, 16 bytes per lane at lds + 16 lane).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}
__device__ __forceinline__ void copy16_to_lds_va(const void* p, const void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(p), "{m0}"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ f32x4 lds_read16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ void copy16_to_lds_at(const char* base, uint32_t voff, const void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_addr(lds)) : "memory");
}
template <int N> __device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// The workgroup's four waves (64 rows) share each 16-key tile: its K and V
// rows are copied once into a ring of kStages LDS stages, kStages-1 tiles
// ahead of the tile being computed, and every wave reads its operands from
// there.  K rows keep their 16-byte slots XOR-swizzled by row (slot ^ row), so
// that the sixteen rows a K read touches fall in different banks.  Three
// stages of 16 KiB (head_dim 128) leave room for three workgroups per CU.
template <int D, int BS>
__global__ __launch_bounds__(64 * kF32Waves, 3) void prefill_chunk_f32_kernel(pkv_prefill_args a) {
  constexpr int KQ = D / 16;   // 16-byte pieces of a K or q row per lane
  constexpr int DT = D / 16;   // 16-dim output tiles; a lane holds DT dims of each of its V rows
  constexpr int DV = DT / 4;   // 16-byte pieces of those
  constexpr int RB = D * 4;    // bytes per K or V row
  constexpr int kSlots = RB / 16;
  constexpr int kTileBytes = 16 * RB;
  constexpr int kTileKiB = kTileBytes / 1024;
  constexpr int kStageBytes = 2 * kTileBytes;          // K then V
  constexpr int kThreads = 64 * kF32Waves;
  constexpr int kCopies = kStageBytes / (16 * kThreads);
  constexpr int kStages = 3;
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(kStageBytes % (16 * kThreads) == 0 && (kCopies == 2 || kCopies == 4), "stage shape");
  static_assert(RB * 8 >= 1024, "a 1 KiB copy covers rows of one 8-token block");
  constexpr int64_t kHeadTile = static_cast<int64_t>(BS) * D;   // floats of one (block, head) tile
  __shared__ __align__(16) char ring[kStages][kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;

  const int32_t Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  const int32_t SG = a.num_seqs * Hkv;
  const int32_t sg = static_cast<int32_t>(blockIdx.x % static_cast<uint32_t>(SG));
  const int32_t rt = static_cast<int32_t>(blockIdx.x / static_cast<uint32_t>(SG));
  const int32_t s = sg / Hkv, kvh = sg - (sg / Hkv) * Hkv;
  const int32_t q0 = a.query_start_loc[s], q1 = a.query_start_loc[s + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.num_query_tokens || q1 - q0 > a.max_query_len) return;   // nowhere safe to write
  const int32_t nq = q1 - q0;
  const int32_t rows = nq * G;
  const int32_t r0 = rt * kPrefillF32RowsPerWg;
  if (r0 >= rows) return;
  const int32_t r_end_wg = min(rows, r0 + kPrefillF32RowsPerWg);
  const int32_t rbase = r0 + wave * 16;
  const int32_t r_end = min(r_end_wg, rbase + 16);       // <= rbase: a wave without rows
  const int32_t ctx = a.context_lens[s];
  if (ctx < nq || !len_ok(ctx, a.max_context_len, a.max_blocks_per_seq, BS)) {
    for (int idx = threadIdx.x; idx < (r_end_wg - r0) * D; idx += kThreads) {
      const int32_t r = r0 + idx / D, d = idx % D;
      a.out[((static_cast<int64_t>(q0) + r / G) * Hq + kvh * G + r % G) * D + d] = __builtin_nanf("");
    }
    return;
  }
  const int32_t first_pos = ctx - nq;          // position of query 0
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const int64_t block_bytes = static_cast<int64_t>(Hkv) * kHeadTile * 4;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache) + kvh * kHeadTile * 4;
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache) + kvh * kHeadTile * 4;
  const int32_t nblk = (ctx + BS - 1) / BS;
  const int32_t wg_lim = first_pos + (r_end_wg - 1) / G + 1;    // keys the workgroup needs
  const int32_t ntiles = (wg_lim + 15) / 16;
  bool bad = false;

  // this lane's row; rows past the tile's end get key limit 0 and q = 0 (their
  // results are never written)
  const int32_t r = rbase + n;
  const bool valid = r < r_end;
  const int32_t i = valid ? r / G : 0;
  const int32_t lim = valid ? first_pos + i + 1 : 0;
  const int32_t tile_lim = r_end > rbase ? first_pos + (r_end - 1) / G + 1 : 0;   // keys any row of the wave needs
  const int32_t nomask_lim = first_pos + rbase / G + 1;                            // keys every row of the wave sees

  // Copy i of wave w fills KiB kF32Waves*i + w of a stage: tile half t (0: K,
  // 1: V), rows in lane order; K's LDS slot k holds the row's slot k ^ (row
  // mod slots).  A 1 KiB copy reads rows of one pool block.
  uint32_t cp_off[kCopies], cp_off0[kCopies];
  int32_t cp_key[kCopies];
#pragma unroll
  for (int c = 0; c < kCopies; ++c) {
    const int kib = kF32Waves * c + wave;
    const int t = kib / kTileKiB;
    const int off = (kib % kTileKiB) * 1024 + 16 * lane;
    const int row = off / RB, k = (off % RB) / 16;
    const int slot = t == 0 ? (k ^ (row % kSlots)) : k;
    cp_key[c] = row;
    cp_off[c] = static_cast<uint32_t>((row % BS) * RB + 16 * slot);
    cp_off0[c] = static_cast<uint32_t>(16 * slot);
  }
  // the tile's block ids: the block of its rows 0-7 and of rows 8-15 (the
  // same unless blocks hold 8 tokens; the second clamped to the last block)
  auto tile_ids = [&](int32_t tt, int32_t& ida, int32_t& idb) {
    const int32_t j0 = (16 * tt) / BS;
    ida = load_block_id(table, __builtin_amdgcn_readfirstlane(j0));
    idb = ida;
    if constexpr (BS == 8) idb = load_block_id(table, __builtin_amdgcn_readfirstlane(min(j0 + 1, nblk - 1)));
  };
  auto issue = [&](int32_t tt, int32_t ida, int32_t idb, char* stage) {
    if (static_cast<uint32_t>(ida) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; ida = 0; }
    if (static_cast<uint32_t>(idb) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; idb = 0; }
    const int32_t key0 = 16 * tt;
    if (key0 + 16 <= ctx) {
      // a whole tile: each copy reads rows of one block (with 8-token blocks,
      // both rows in one half of the tile) at a per-lane offset
#pragma unroll
      for (int c = 0; c < kCopies; ++c) {
        const int kib = kF32Waves * c + wave;
        const int t = kib / kTileKiB;
        const bool hi = BS == 8 && (kib % kTileKiB) * 1024 / RB >= 8;
        const char* base = (t == 0 ? kc : vc) + static_cast<int64_t>(hi ? idb : ida) * block_bytes + (key0 % BS) * RB;
        copy16_to_lds_at(base, cp_off[c], stage + kib * 1024);
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < kCopies; ++c) {
      const int kib = kF32Waves * c + wave;
      const int t = kib / kTileKiB;
      const int32_t id = (BS == 8 && cp_key[c] >= 8) ? idb : ida;
      const char* base = (t == 0 ? kc : vc) + id * block_bytes;
      // keys past the context read row 0 of the tile (a cached token: finite
      // data, masked to probability 0)
      // (a 32-token block holds two tiles: the tile's rows start at key0 mod BS)
      const char* src = key0 + cp_key[c] < ctx ? base + (key0 % BS) * RB + cp_off[c]
                                               : (t == 0 ? kc : vc) + ida * block_bytes + (key0 % BS) * RB + cp_off0[c];
      copy16_to_lds_va(src, stage + kib * 1024);
    }
  };

  f32x4 qv[KQ];
  {
    const float* qrow = static_cast<const float*>(a.q) +
                        ((static_cast<int64_t>(q0) + i) * Hq + kvh * G + (valid ? r % G : 0)) * D;
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      f32x4 w = *reinterpret_cast<const f32x4*>(qrow + 16 * m + 4 * g);
      if (!valid || a.q_mode == 2) w = f32x4{0.f, 0.f, 0.f, 0.f};
      if (a.q_mode == 1) w = -w;                 // the scale's sign, exactly
      qv[m] = w;
    }
  }

  const float c2 = a.scale_log2;               // > 0 (the scale's sign is in q)
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, thr = kNegBig, lsum = 0.f;
  const float rescale_raw = 8.f / c2;          // 2^8 of growth, in raw score units

  // LDS read addresses of stage 0 (the other stages at fixed offsets): K row n,
  // logical slot 4m + g at its swizzled place; V rows 4g + kk, slot n ..
  const uint32_t ring0 = lds_addr(ring[0]);
  uint32_t k_addr[KQ];
#pragma unroll
  for (int m = 0; m < KQ; ++m) {
    k_addr[m] = ring0 + n * RB + 16 * ((4 * m + g) ^ (n % kSlots));
    asm volatile("" : "+v"(k_addr[m]));
  }
  uint32_t v_addr = ring0 + kTileBytes + 4 * g * RB + 16 * n;
  asm volatile("" : "+v"(v_addr));

  auto compute_tile = [&](int32_t tt, uint32_t stage_off) {
    const int32_t key0 = 16 * tt;
    f32x4 kv[KQ];
#pragma unroll
    for (int m = 0; m < KQ; ++m) kv[m] = lds_read16(k_addr[m] + stage_off);
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
      for (int c = 0; c < DV; ++c) vv[kk][c] = lds_read16(v_addr + stage_off + kk * RB + 256 * c);
    f32x4 sc = acc0 + acc1;
    if (key0 + 16 > nomask_lim) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (key0 + 4 * g + j >= lim) sc[j] = -INFINITY;
    }
    const float lane_mx = max4(sc);
    if (__builtin_amdgcn_ballot_w64(lane_mx > thr)) {
      // a row's running maximum moves only once a score passes it by 2^8
      const float mx = max_over_rows(lane_mx);
      const bool up = mx > thr;
      const float mnew = up ? mx * c2 : m_run;
      const float alpha = fast_exp2(m_run - mnew);
      m_run = mnew;
      thr = up ? mx + rescale_raw : thr;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(fmaf(sc[j], c2, -m_run));
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) o[dt] = mfma4(vv[kk][dt / 4][dt % 4], p[kk], o[dt]);
    __builtin_amdgcn_s_setprio(0);
  };

  // prologue: the first kStages-1 tiles' copies; the ids of the next one
#pragma unroll
  for (int tt = 0; tt < kStages - 1; ++tt)
    if (tt < ntiles) {
      int32_t ida, idb;
      tile_ids(tt, ida, idb);
      issue(tt, ida, idb, ring[tt]);
    }
  int32_t nida = 0, nidb = 0;
  if (kStages - 1 < ntiles) tile_ids(kStages - 1, nida, nidb);

  for (int32_t t0 = 0; t0 < ntiles; t0 += kStages) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int32_t tt = t0 + st;
      if (tt >= ntiles) break;
      // this tile's copies have landed once at most the later issued tiles'
      // copies are outstanding (copies complete in issue order)
      const int32_t ahead = min(kStages - 2, ntiles - 1 - tt);
      if (ahead >= 2) wait_vm<2 * kCopies>();
      else if (ahead == 1) wait_vm<kCopies>();
      else wait_vm<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int32_t tn = tt + kStages - 1;
      const int32_t ida = nida, idb = nidb;
      if (tn + 1 < ntiles) tile_ids(tn + 1, nida, nidb);
      __builtin_amdgcn_s_barrier();
      if (16 * tt < tile_lim) compute_tile(tt, static_cast<uint32_t>(st * kStageBytes));
      // every wave passed the barrier after it finished the tile before this
      // one, so that tile's stage takes tile tt + kStages - 1
      if (tn < ntiles) issue(tn, ida, idb, ring[(st + kStages - 1) % kStages]);
    }
  }

  float L = lsum;
  L += __shfl_xor(L, 16);
  L += __shfl_xor(L, 32);
  // a bad block id in the workgroup's range poisons its rows
  const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
  if (!valid) return;
  const float inv = any_bad ? __builtin_nanf("") : 1.f / L;
  float* orow = a.out + ((static_cast<int64_t>(q0) + i) * Hq + kvh * G + r % G) * D;
  // lane (n, g) holds dims 16g + 4j + 64(dt/4) + dt%4 of row n in o[dt][j]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < DV; ++c) {
      const f32x4 v = f32x4{o[4 * c][j], o[4 * c + 1][j], o[4 * c + 2][j], o[4 * c + 3][j]} * inv;
      *reinterpret_cast<f32x4*>(orow + 16 * g + 4 * j + 64 * c) = v;
    }
}

template <int D>
void launch_bs(int block_size, dim3 grid, hipStream_t st, const pkv_prefill_args& a) {
  if (block_size == 8)
    hipLaunchKernelGGL((prefill_chunk_f32_kernel<D, 8>), grid, dim3(64 * kF32Waves), 0, st, a);
  else if (block_size == 32)
    hipLaunchKernelGGL((prefill_chunk_f32_kernel<D, 32>), grid, dim3(64 * kF32Waves), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_chunk_f32_kernel<D, 16>), grid, dim3(64 * kF32Waves), 0, st, a);
}

}  // namespace

int pkv_launch_prefill_f32(const pkv_prefill_args& a, void* stream) {
  const int32_t group = a.num_heads / a.num_kv_heads;
  const int64_t tiles =
      (static_cast<int64_t>(a.max_query_len) * group + kPrefillF32RowsPerWg - 1) / kPrefillF32RowsPerWg;
  const int64_t grid = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * tiles;
  if (grid == 0) return hipSuccess;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.head_dim == 128) launch_bs<128>(a.block_size, dim3(static_cast<uint32_t>(grid)), st, a);
  else launch_bs<64>(a.block_size, dim3(static_cast<uint32_t>(grid)), st, a);
  return hipGetLastError();
}

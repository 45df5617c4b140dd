// MFMA kernels for gfx950 (CDNA4, wave64): attention of query-head groups that
// share one KV head, where the work is a real dense contraction.
//
//   decode_group_mfma_kernel   -- decode with grouped-query heads (G = Hq/Hkv
//                                 query heads read the same K/V tiles; groups
//                                 past 64 heads in 16-row slice workgroups)
//   decode_wide_group_kernel   -- the same for 17..64 heads per KV head: one
//                                 workgroup for all slices, K/V staged in LDS
//   decode_shared_mfma_kernel  -- a fork group's shared prefix blocks read once
//                                 for all its members (the members are rows)
//   prefill_chunk_mfma_kernel  -- causal attention of a prefill chunk: every
//                                 (query token, head) row of a KV group against
//                                 its sequence's paged context
//
// Pages cited:
//   [OS]  "PagedAttention: gestionar la KV cache como memoria de un sistema
//         operativo" (josueisai.com), "Cómo funciona por dentro": attention follows
//         the block table, scores each block, then one softmax-weighted sum.
//   [UL]  "Continuous Batching" (Ultralytics glossary), "Cómo funciona la
//         planificación a nivel de iteración" and "Límites y técnicas
//         complementarias": long prompts are prefilled in chunks that share a
//         step with other sequences' decode.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16, checked on the device): lane l
// with n = l % 16 and g = l / 16 supplies row n of A and column n of B, each as
// 8 bf16 of the k-slots of group g, and receives D[4g + j][n], j = 0..3.
//
// Both kernels compute the transposed products
//     S^T = K Q^T        (A = 16 keys of a block x 32 dims, B = Q^T)
//     O^T += V^T P^T     (A = V^T: 16 dims x 32 keys, B = P^T)
// so that every per-row quantity (running max, sum, the row's output) lives in
// the lanes whose n is that row, and the P^T operand is exactly the S^T result
// of two blocks: lane (n, g) holds keys 4g..4g+3 of each block for row n.
// V is stored token-major in the pool, so V^T is formed with the gfx950
// transposed LDS read ds_read_tr16_b64: within each 16-lane group, lane i gets
// element i % 4 of the 4-element segments addressed by lanes 4j + i/4
// (j = 0..3).  Lane s of group g therefore points at V[key 4g + s/4][dims
// 16c + 4(s%4) ..], and receives V[key 4g + j][dim 16c + s] for j = 0..3.
//
// P is split into a bf16 high part and a bf16 remainder, two MFMAs each, so
// that the probabilities keep ~16 significant bits: a plain bf16 P would put an
// error of up to 2^-9 |v_j - v_k| on a row whose weight sits on two keys j, k.  Masked keys are removed by select
// (score -inf, V row 0), never by multiplying, so NaN in unused slots cannot
// reach the output.
#include "pkv_device.h"
#include "pkv_plan.h"

namespace {

using pkvd::u32x4;
using pkvd::kBlock;
using pkvd::kNegBig;
using pkvd::kPlanHdr;
using pkvd::fast_exp2;
using pkvd::len_ok;
using pkvd::plan_matches;
using pkvd::max_over_rows;
using pkvd::load_block_id;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;                      // waves of a group-decode workgroup
constexpr int kGroupThreads = 64 * kWaves;

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ u32x4 load16_nt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Transposed read of one 4-key x 16-dim piece of V from LDS (see the header).
__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// The same reads from a 32-bit LDS byte address, and a 16-byte LDS read.
__device__ __forceinline__ s16x4 lds_read_tr_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(static_cast<uintptr_t>(addr)));
}
__device__ __forceinline__ u32x4 lds_read16_at(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(static_cast<uintptr_t>(addr));
}
// The LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

__device__ __forceinline__ bf16x8 join(const s16x4& lo, const s16x4& hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Decode for a query-head group.  One workgroup per (unit, KV head, slice),
// where a unit is a (sequence, 4096-token partition) of the plan (longest
// first).  The G query heads of the group are the 16 MFMA rows (rows >= G hold
// q = 0 and are never written); a group of more than 16 heads is cut into
// slices of 16, one workgroup each, which read the same K/V (mostly from L2).  The unit's blocks are dealt to the 4 waves in turn; per
// block a wave
//   - loads the K tile straight into the A-operand layout (lane (n, g) reads
//     16 B of key n at dims 32c + 8g) and forms S^T = K Q^T (D/32 MFMAs),
//   - moves the V tile into its own 16-row LDS tile by direct global->LDS
//     loads (no registers), with the 16-byte slots of row r XOR-swizzled by
//     2*(r / (256/row bytes) mod (slots/2)) so that the transposed reads hit
//     every bank pair at most twice; rows of keys past the context are filled
//     from key 0 of the block (finite data) and get probability 0,
//   - forms V^T with one transposed read per 16 dims and accumulates
//     O^T += V^T P^T with 16x16x16 MFMAs (P^T is exactly the S^T of the block).
// Each wave keeps an online softmax per row; the waves are merged through LDS
// with the log-sum-exp rule, and the unit writes the output rows (one-partition
// sequences) or (max, sum, accumulator) partials -- the same partial format as
// the VALU decode kernel -- which the row's last unit to finish merges.
// ---------------------------------------------------------------------------
typedef short s16x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const s16x4v& a, const s16x4v& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 16-byte slot k of V row r lives at slot k ^ vswz(r) of the LDS tile.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  constexpr int kSlots = D * 2 / 16;            // 16-byte slots per row
  constexpr int kRowsPerLine = 256 / (D * 2);   // rows per 256-byte bank line
  return 2 * ((r / kRowsPerLine) % (kSlots / 2));
}

template <int D, int BS>
__device__ __forceinline__ void decode_group_mfma_body(const pkv_decode_args& a, uint32_t bid, bool shared_unit) {
  constexpr int KC = D / 32;            // 32-dim chunks of q.k
  constexpr int DC = D / 16;            // 16-dim chunks of the output
  constexpr int RB = D * 2;             // bytes per key row
  constexpr int kT = 16;                // keys per MFMA tile (the unit of the walk)
  constexpr int NLD = kT * RB / 1024;   // 1 KiB direct-to-LDS loads per V tile
  constexpr int OROW = D + 4;           // padded LDS row (floats) of the wave merge
  constexpr int kVBytes = kWaves * 2 * kT * RB;     // two V tiles per wave
  constexpr int kOBytes = kWaves * 16 * OROW * 4;
  constexpr int kSmem = kVBytes > kOBytes ? kVBytes : kOBytes;
  constexpr int64_t kHeadTile = static_cast<int64_t>(BS) * RB;   // one (block, head) tile of the pool
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(RB * 8 % 1024 == 0 || RB * 4 % 1024 == 0, "a 1 KiB load covers rows of one 8-row half");
  __shared__ __align__(16) char smem[kSmem];
  __shared__ float sm_ml[kWaves][16][2];
  __shared__ int sm_bad[kWaves];
  __shared__ int sm_last;
  __shared__ int sm_member_last[kMaxMfmaGroup], sm_member_slots[kMaxMfmaGroup];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;

  const int32_t Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  // A plan unit's group of more than 16 query heads is cut into slices of 16
  // rows, one workgroup each (shared-prefix units have G <= 16: one slice).
  const int32_t nsl = shared_unit ? 1 : (G + kMaxMfmaGroup - 1) / kMaxMfmaGroup;
  // the slices of one (unit, KV head) get workgroup ids 8 apart, i.e. one XCD
  // (workgroups go to the 8 XCDs in turn), so they read its K/V through one L2
  // (the grid is padded to whole groups of 8; padding units exit at the plan)
  const uint32_t x = nsl == 1 ? bid : (bid / (8u * nsl)) * 8u + bid % 8u;
  const int32_t slice = nsl == 1 ? 0 : static_cast<int32_t>((bid / 8u) % static_cast<uint32_t>(nsl));
  const int32_t u = static_cast<int32_t>(x / static_cast<uint32_t>(Hkv));
  const int32_t kvh = static_cast<int32_t>(x - static_cast<uint32_t>(u) * Hkv);
  const int32_t slice_rows = min(kMaxMfmaGroup, G - kMaxMfmaGroup * slice);
  // The unit: rows r < nrows are (sequence s0 + r / GR, query head hb + r % GR);
  // it walks the 16-key tiles t_begin .. t_end-1 of s0's context (tile t is
  // tokens 16t .. 16t+15, whatever blocks hold them), keys below ctx valid,
  // and writes the output rows (direct) or partial slot `slot` of each row.
  int32_t s0, nrows, ctx, t_begin, t_end, slot;
  int32_t GR = G;                                        // rows per sequence
  const int32_t hb = kvh * G + kMaxMfmaGroup * slice;    // query head of row 0
  int32_t nslots = 0;     // partial slots of each row (merged in this launch)
  bool direct;
  if (shared_unit) {
    // a group's shared leading blocks: the rows are the group's sequences (a
    // plan built for other sizes runs no shared unit; the sequences' own units
    // then write NaN rows)
    const int32_t* sp = a.shared_plan;
    if (!pkvd::shared_plan_matches(sp, a) || u >= sp[0]) return;
    const int32_t* su = sp + kPlanHdr + 4 * u;
    s0 = su[0];
    nrows = min(su[1], kMaxMfmaGroup / G) * G;
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
        for (int idx = threadIdx.x; idx < slice_rows * D; idx += kGroupThreads)
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
      for (int idx = threadIdx.x; idx < slice_rows * D; idx += kGroupThreads)
        a.out[(static_cast<int64_t>(s) * Hq + hb) * D + idx] = ctx == 0 ? 0.f : __builtin_nanf("");
      return;
    }
    const int32_t part = a.part_tokens;
    const int32_t start = pkvd::seq_start_of(a, s);     // a multiple of 16
    const int32_t base = pkvd::slot_base_of(a, start);
    const int32_t np_s = (ctx - start + part - 1) / part;
    const int32_t ntiles = (ctx + kT - 1) / kT;
    s0 = s;
    nrows = slice_rows;
    GR = slice_rows;
    t_begin = start / kT + p * (part / kT);
    t_end = min(ntiles, t_begin + part / kT);
    slot = base + p;
    nslots = base + np_s;
    direct = np_s == 1 && base == 0;
  }

  const int64_t block_bytes = static_cast<int64_t>(Hkv) * kHeadTile;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache) + kvh * kHeadTile;
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache) + kvh * kHeadTile;
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s0) * a.max_blocks_per_seq;
  const int32_t nblk = (ctx + BS - 1) / BS;

  char* vs = smem + wave * (2 * kT * RB);      // this wave's two V tiles

  // Q^T as the B operand: lane (n, g) holds dims 32c + 8g .. +8 of row n.
  bf16x8 qb[KC];
  {
    const int hr = n < nrows ? n : 0;
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((static_cast<int64_t>(s0 + hr / GR) * Hq + hb + hr % GR) * D) * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 64 * c + 16 * g);
      if (n >= nrows) w = u32x4{0, 0, 0, 0};
      qb[c] = as_bf16x8(w);
    }
  }

  // per-lane pieces of the V tile traffic: for each 1 KiB copy, the tile row
  // r this lane reads times RB plus the byte offset within the row (swizzled
  // slot), and the transposed-read address (key row 4g + n/4, dims 4(n%4) of
  // each 16-dim chunk)
  int dma_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int r = (1024 * i + 16 * lane) / RB, k = ((1024 * i + 16 * lane) % RB) / 16;
    dma_off[i] = r * RB + 16 * (k ^ vswz<D>(r));
  }
  const int tr_row = 4 * g + (n >> 2);
  const int tr_sw = vswz<D>(tr_row);
  const int tr_k0 = (n & 3) >> 1;       // slot of dims 4(n%4) within a 32-byte chunk pair

  f32x4 o[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegBig, lsum = 0.f;
  bool bad = false;

  // The step's new token (decode with the cache write).  Only the wave that
  // loads the tile of token ctx-1 uses it: there it checks that the new slot
  // is token ctx-1's, takes that row (and the unused rows after it) from the
  // new K/V and stores the row into the pool.  The slot is loaded here and
  // waited for only there.
  const int64_t new_slot = (a.new_slots && !shared_unit) ? a.new_slots[s0] : -1;
  const int32_t last_tile = (ctx + kT - 1) / kT - 1;
  const int32_t last_row = (ctx - 1) % kT;                   // row of token ctx-1 in its tile
  const int64_t new_src = (static_cast<int64_t>(s0) * Hkv + kvh) * RB;

  // The wave's tiles' block ids (at most kMaxPartTokens/16/4 = 64 tiles), one
  // tile per lane, fetched once before the loop: the block of rows 0-7 (lo)
  // and of rows 8-15 (hi) of the tile -- the same block unless blocks hold 8
  // tokens; a block past the context is never read (its rows get row 0's).
  const int32_t nit = (t_end - t_begin - wave + kWaves - 1) / kWaves;
  int32_t ids_lo = 0, ids_hi = 0;
  if (lane < nit) {
    const int32_t t = t_begin + wave + kWaves * lane;
    ids_lo = table[(kT * t) / BS];
    if constexpr (BS == 8) ids_hi = kT * t + 8 < ctx ? table[(kT * t + 8) / BS] : ids_lo;
  }
  // Byte offset of row r of tile t in its block's (block, head) tile: the
  // tile's offset in the block (0 unless a block holds two tiles) plus the
  // row's (within its 8-token block, when blocks hold 8 tokens).
  auto tile_off = [&](int32_t t) -> int64_t { return BS == 32 ? static_cast<int64_t>(t & 1) * kT * RB : 0; };
  auto row_in = [&](int r) -> int { return BS == 8 ? (r & 7) * RB : r * RB; };

  // Loads of the wave's tile `it`: K into registers, V into an LDS tile.  V
  // rows of keys past the context are copied from row 0 of the tile instead
  // (finite data; their probabilities are 0), so the copies need no branches.
  auto issue = [&](int32_t it, u32x4 (&kt)[KC], char* tile) {
    const int32_t t = t_begin + wave + kWaves * it;
    if constexpr (BS != 8) {
      // one block holds the whole tile (a tile is a block, or half of one)
      const int32_t raw_id = __builtin_amdgcn_readlane(ids_lo, it);
      int32_t id = raw_id;
      if (static_cast<uint32_t>(id) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; id = 0; }
      const char* kp = kc + id * block_bytes + tile_off(t);
      const char* vp = vc + id * block_bytes + tile_off(t);
      const int32_t valid_rows = min(kT, ctx - t * kT);
      int mode = 0;       // 0: all rows from the pool; 1: the new token's block; 2: a wrong slot
      if (t == last_tile && new_slot >= 0)
        mode = (static_cast<uint32_t>(raw_id) < static_cast<uint32_t>(a.num_blocks) &&
                new_slot == static_cast<int64_t>(raw_id) * BS + (ctx - 1) % BS) ? 1 : 2;
      if (mode != 1) {
        if (mode == 2) bad = true;    // not token ctx-1's slot: NaN rows, nothing stored
#pragma unroll
        for (int c = 0; c < KC; ++c)
          kt[c] = n < valid_rows ? load16_nt(kp + n * RB + 64 * c + 16 * g) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int src = (1024 * i + 16 * lane) / RB < valid_rows ? dma_off[i] : dma_off[i] % RB;
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vp + src),
                                           (__attribute__((address_space(3))) void*)(tile + 1024 * i), 16, 0, 0);
        }
      } else {
        const char* nk = reinterpret_cast<const char*>(a.new_k) + new_src;
        const char* nv = reinterpret_cast<const char*>(a.new_v) + new_src;
#pragma unroll
        for (int c = 0; c < KC; ++c)
          kt[c] = n < last_row ? load16_nt(kp + n * RB + 64 * c + 16 * g)
                  : n == last_row ? *reinterpret_cast<const u32x4*>(nk + 64 * c + 16 * g) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const char* src = (1024 * i + 16 * lane) / RB < last_row ? vp + dma_off[i] : nv + dma_off[i] % RB;
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                           (__attribute__((address_space(3))) void*)(tile + 1024 * i), 16, 0, 0);
        }
        if (n == last_row && slice == 0) {   // the first slice stores the row
#pragma unroll
          for (int c = 0; c < KC; ++c) {
            *reinterpret_cast<u32x4*>(const_cast<char*>(kp) + last_row * RB + 64 * c + 16 * g) = kt[c];
            *reinterpret_cast<u32x4*>(const_cast<char*>(vp) + last_row * RB + 64 * c + 16 * g) =
                *reinterpret_cast<const u32x4*>(nv + 64 * c + 16 * g);
          }
        }
      }
      return;
    }
    const int32_t raw_lo = __builtin_amdgcn_readlane(ids_lo, it);
    const int32_t raw_hi = BS == 8 ? __builtin_amdgcn_readlane(ids_hi, it) : raw_lo;
    int32_t id_lo = raw_lo, id_hi = raw_hi;
    if (static_cast<uint32_t>(id_lo) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; id_lo = 0; }
    if (BS == 8) {
      if (static_cast<uint32_t>(id_hi) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; id_hi = 0; }
    } else {
      id_hi = id_lo;
    }
    const int64_t toff = tile_off(t);
    const char* kbase = kc + toff;
    const char* vbase = vc + toff;
    // block of tile row r (the same for every row unless blocks hold 8 tokens)
    auto blk = [&](int r) -> int64_t { return static_cast<int64_t>(BS == 8 && r >= 8 ? id_hi : id_lo) * block_bytes; };
    const int32_t valid_rows = min(kT, ctx - t * kT);
    int mode = 0;       // 0: all rows from the pool; 1: the new token's tile; 2: a wrong slot
    if (t == last_tile && new_slot >= 0) {
      const int32_t raw_last = BS == 8 && last_row >= 8 ? raw_hi : raw_lo;
      mode = (static_cast<uint32_t>(raw_last) < static_cast<uint32_t>(a.num_blocks) &&
              new_slot == static_cast<int64_t>(raw_last) * BS + (ctx - 1) % BS) ? 1 : 2;
    }
    if (mode != 1) {
      if (mode == 2) bad = true;    // not token ctx-1's slot: NaN rows, nothing stored
      // keys past the context are not loaded (their scores are masked)
      const char* kp = kbase + blk(n) + n * RB - (BS == 8 && n >= 8 ? 8 * RB : 0);
#pragma unroll
      for (int c = 0; c < KC; ++c) kt[c] = n < valid_rows ? load16_nt(kp + 64 * c + 16 * g) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const char* src;
        if constexpr (BS == 8) {
          const int row = dma_off[i] / RB, col = dma_off[i] % RB;
          const int r = row < valid_rows ? row : 0;
          src = vbase + blk(r) + row_in(r) + col;
        } else {
          // one block holds the whole tile: the rows at their offsets, row 0's past the context
          src = vbase + blk(0) + ((1024 * i + 16 * lane) / RB < valid_rows ? dma_off[i] : dma_off[i] % RB);
        }
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (__attribute__((address_space(3))) void*)(tile + 1024 * i), 16, 0, 0);
      }
    } else {
      // the tile of the new token: its row, and the unused rows after it,
      // come from the new K/V (finite data; the unused rows are masked); the
      // lanes of the new row store it into the pool
      const char* nk = reinterpret_cast<const char*>(a.new_k) + new_src;
      const char* nv = reinterpret_cast<const char*>(a.new_v) + new_src;
      const char* kp = kbase + blk(n) + row_in(n);
#pragma unroll
      for (int c = 0; c < KC; ++c)
        kt[c] = n < last_row ? load16_nt(kp + 64 * c + 16 * g)
                : n == last_row ? *reinterpret_cast<const u32x4*>(nk + 64 * c + 16 * g) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = dma_off[i] / RB, col = dma_off[i] % RB;
        const char* src = row < last_row ? vbase + blk(row) + row_in(row) + col : nv + col;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (__attribute__((address_space(3))) void*)(tile + 1024 * i), 16, 0, 0);
      }
      if (n == last_row && slice == 0) {   // the first slice stores the row
        char* vp = const_cast<char*>(vbase) + blk(n) + row_in(n);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          *reinterpret_cast<u32x4*>(const_cast<char*>(kp) + 64 * c + 16 * g) = kt[c];
          *reinterpret_cast<u32x4*>(vp + 64 * c + 16 * g) = *reinterpret_cast<const u32x4*>(nv + 64 * c + 16 * g);
        }
      }
    }
  };
  // Online-softmax update of tile `it` from its K registers and V tile.
  auto compute = [&](int32_t it, const u32x4 (&kt)[KC], const char* tile) {
    const int32_t t = t_begin + wave + kWaves * it;
    const int32_t valid_rows = min(kT, ctx - t * kT);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) acc = mfma(as_bf16x8(kt[c]), qb[c], acc);
    float sc[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sc[jj] = 4 * g + jj < valid_rows ? acc[jj] * a.scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    s16x4v ph, pl;
    float ps = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float pr = fast_exp2(sc[jj] - mnew);
      ps += pr;
      const __bf16 hi = static_cast<__bf16>(pr);
      const __bf16 lo = static_cast<__bf16>(pr - static_cast<float>(hi));
      ph[jj] = __builtin_bit_cast(short, hi);
      pl[jj] = __builtin_bit_cast(short, lo);
    }
    lsum = lsum * alpha + ps;
    const char* trb = tile + tr_row * RB + 8 * (n & 1);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const s16x4 vt = lds_read_tr(trb + 16 * ((2 * c + tr_k0) ^ tr_sw));
      f32x4 tacc = o[c] * alpha;
      tacc = mfma16(vt, ph, tacc);
      o[c] = mfma16(vt, pl, tacc);
    }
  };
  (void)nblk;
  // Two tiles per step: both tiles' K and V loads are issued, then both are
  // computed, so a wave keeps 2 x (K + V) tiles in flight.
  u32x4 ktA[KC], ktB[KC];
  char* tileA = vs;
  char* tileB = vs + kT * RB;
  for (int32_t it = 0; it < nit; it += 2) {
    issue(it, ktA, tileA);
    if (it + 1 < nit) issue(it + 1, ktB, tileB);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    compute(it, ktA, tileA);
    if (it + 1 < nit) compute(it + 1, ktB, tileB);
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // merge the four waves through LDS (the V tiles are reused)
  __syncthreads();
  float* so = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int c = 0; c < DC; ++c)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) so[(wave * 16 + n) * OROW + 16 * c + 4 * g + jj] = o[c][jj];
  if (g == 0) { sm_ml[wave][n][0] = m; sm_ml[wave][n][1] = lsum; }
  if (lane == 0) sm_bad[wave] = bad ? 1 : 0;
  __syncthreads();
  int bad_any = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) bad_any |= sm_bad[w];
  const bool any_bad = bad_any != 0;
  for (int idx = threadIdx.x; idx < nrows * D; idx += kGroupThreads) {
    const int r = idx / D, d = idx - (idx / D) * D;
    float M = sm_ml[0][r][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_ml[w][r][0]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm_ml[w][r][0] - M);
      L += sm_ml[w][r][1] * f;
      acc += so[(w * 16 + r) * OROW + d] * f;
    }
    if (any_bad) { acc = __builtin_nanf(""); L = __builtin_nanf(""); }
    const int64_t row = static_cast<int64_t>(s0 + r / GR) * Hq + hb + r % GR;
    if (direct) {
      a.out[row * D + d] = acc / L;
    } else {
      const int64_t pidx = row * a.num_partitions + slot;
      pkvd::store_coherent(a.part_acc + pidx * D + d, acc);
      if (d == 0) { pkvd::store_coherent(a.part_ml + 2 * pidx, M); pkvd::store_coherent(a.part_ml + 2 * pidx + 1, L); }
    }
  }
  // a split context: the last of the sequence's units (for this KV head and
  // slice) to finish merges its rows
  if (direct) return;
  if (!shared_unit) {
    const int64_t row0 = static_cast<int64_t>(s0) * Hq + hb;
    if (!pkvd::arrive_last(a.merge_tickets + row0, a.merge_epoch, nslots, &sm_last)) return;
    for (int idx = threadIdx.x; idx < nrows * D; idx += kGroupThreads) {
      const int64_t prow = (row0 + idx / D) * a.num_partitions;
      const int d = idx - (idx / D) * D;
      a.out[(row0 + idx / D) * D + d] =
          pkvd::merge_partials_coherent(a.part_ml + 2 * prow, a.part_acc + prow * D + d, nslots, D);
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
    for (int idx = threadIdx.x; idx < G * D; idx += kGroupThreads) {
      const int64_t prow = (row0 + idx / D) * a.num_partitions;
      const int d = idx - (idx / D) * D;
      a.out[(row0 + idx / D) * D + d] =
          pkvd::merge_partials_coherent(a.part_ml + 2 * prow, a.part_acc + prow * D + d, slots, D);
    }
  }
}

// 8-token blocks take two block ids per tile: three workgroups per CU, so the
// body keeps its registers
template <int D, int BS>
__global__ __launch_bounds__(kGroupThreads, BS == 8 ? 3 : 4) void decode_group_mfma_kernel(pkv_decode_args a) {
  decode_group_mfma_body<D, BS>(a, blockIdx.x, false);
}

// The shared-prefix units of a shared-prefix decode (one workgroup per
// possible unit and KV head; those past the shared plan's count exit).  The
// sequences' own units follow in a launch of the plain decode kernels.
template <int D, int BS>
__global__ __launch_bounds__(kGroupThreads, BS == 8 ? 3 : 4) void decode_shared_mfma_kernel(pkv_decode_args a) {
  decode_group_mfma_body<D, BS>(a, blockIdx.x, true);
}

// ---------------------------------------------------------------------------
// Shared-prefix plan.  [OS] "El regalo extra: compartir memoria" and [IPX] "Dos
// respuestas a una entrada": the parallel samples of one prompt hold the same
// physical blocks for that prompt, so one read of each shared K/V tile can
// serve every sample -- the samples become the rows of the MFMA tile, as the
// query heads of a group do in grouped-query decode.
//
// Sequences group_start[g] .. group_start[g+1]-1 form group g (the caller's
// hint).  One wave per group finds its shared prefix: the longest run of
// leading table entries that are equal in every member and lie wholly below
// every member's context.  Every member's seq_start becomes that many tokens;
// the group is cut into sub-groups of at most 16 / G sequences (16 MFMA rows),
// and each sub-group gets one unit per prefix partition.  A malformed
// group_start (not 0 .. num_seqs, decreasing), a group of one, a member with an
// invalid context or no common first block give no prefix: such sequences are
// decoded whole by their own units, so the hint can never change a result.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t wave_min(int32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ void shared_plan_body(const pkv_decode_args& a, const int32_t* __restrict__ group_start,
                                                 int32_t num_groups, int32_t* __restrict__ seq_start,
                                                 int32_t* __restrict__ shared_plan) {
  __shared__ int32_t sm_units, sm_bad;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t S = a.num_seqs, MB = a.max_blocks_per_seq, BSZ = a.block_size;
  if (tid == 0) { sm_units = 0; sm_bad = 0; }
  __syncthreads();
  if (num_groups <= 0 && tid == 0) sm_bad = 1;      // no groups: no shared prefix
  for (int32_t i = tid; num_groups > 0 && i <= num_groups; i += 1024) {
    const int32_t v = group_start[i];
    bool ok = v >= 0 && v <= S;
    if (i == 0) ok = ok && v == 0;
    if (i == num_groups) ok = ok && v == S;
    else ok = ok && v <= group_start[i + 1];
    if (!ok) atomicOr(&sm_bad, 1);
  }
  __syncthreads();
  if (sm_bad) {
    for (int32_t s = tid; s < S; s += 1024) seq_start[s] = 0;
  } else {
    const int32_t per_sub = kMaxMfmaGroup / (a.num_heads / a.num_kv_heads);
    for (int32_t grp = wave; grp < num_groups; grp += 1024 / 64) {
      const int32_t b = group_start[grp], e = group_start[grp + 1];
      const int32_t n = e - b;
      // whole blocks below every member's context (-1: an invalid context)
      int32_t lim = 0x7FFFFFFF;
      for (int32_t m = b + lane; m < e; m += 64) {
        const int32_t ctx = a.context_lens[m];
        lim = min(lim, len_ok(ctx, a.max_context_len, MB, BSZ) ? ctx / BSZ : -1);
      }
      lim = wave_min(lim);
      int32_t cp = 0;
      if (n >= 2 && lim > 0) {
        const int32_t* t0 = a.block_tables + static_cast<int64_t>(b) * MB;
        cp = lim;
        for (int32_t j0 = 0; j0 < lim; j0 += 64) {
          const int32_t j = j0 + lane;
          bool eq = true;
          if (j < lim) {
            // the members' entries are loaded eight at a time, all before any
            // is compared, so the loads overlap instead of waiting on each other
            // (past the last member the last one is read again)
            const int32_t ref = t0[j];
            const int32_t* col = a.block_tables + j;
            for (int32_t m0 = b + 1; m0 < e; m0 += 8) {
              int32_t x[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) x[i] = col[static_cast<int64_t>(min(m0 + i, e - 1)) * MB];
#pragma unroll
              for (int i = 0; i < 8; ++i) eq = eq & (x[i] == ref);
            }
          }
          const uint64_t differ = __ballot(!eq);
          if (differ) {
            cp = j0 + __ffsll(static_cast<unsigned long long>(differ)) - 1;
            break;
          }
        }
      }
      // the prefix is walked in 16-key tiles: with 8-token blocks an odd last
      // common block is left to the members' own units
      const int32_t pref = (cp * BSZ) & ~15;
      for (int32_t m = b + lane; m < e; m += 64) seq_start[m] = pref;
      if (pref > 0) {
        const int32_t nsub = (n + per_sub - 1) / per_sub;
        const int32_t npp = (pref + a.prefix_part_tokens - 1) / a.prefix_part_tokens;
        int32_t first = 0;
        if (lane == 0) first = atomicAdd(&sm_units, nsub * npp);
        first = __shfl(first, 0);
        for (int32_t k = lane; k < nsub * npp; k += 64) {
          const int32_t sub = k / npp, pp = k - sub * npp;
          int32_t* unit = shared_plan + kPlanHdr + 4 * (first + k);
          unit[0] = b + sub * per_sub;
          unit[1] = min(per_sub, n - sub * per_sub);
          unit[2] = pp;
          unit[3] = pref;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    shared_plan[0] = sm_units;
    shared_plan[1] = S;
    shared_plan[2] = a.max_context_len;
    shared_plan[3] = MB;
    shared_plan[4] = a.prefix_part_tokens;
    shared_plan[5] = a.num_heads / a.num_kv_heads;     // query heads per KV head (rows per member)
    shared_plan[6] = 0;
    shared_plan[7] = 0;
  }
}

// Both plans of a shared-prefix launch in one workgroup: the groups' shared
// prefixes (seq_start, the shared plan), then the plan of every sequence's own
// tokens from those starts (the barrier makes the starts visible to every
// thread of the workgroup).
__global__ __launch_bounds__(1024) void shared_plans_kernel(pkv_decode_args a, const int32_t* __restrict__ group_start,
                                                            int32_t num_groups, int32_t* __restrict__ seq_start,
                                                            int32_t* __restrict__ shared_plan, int32_t* __restrict__ plan) {
  shared_plan_body(a, group_start, num_groups, seq_start, shared_plan);
  __syncthreads();
  plan_body(plan, a.context_lens, a.num_seqs, a.max_blocks_per_seq, a.block_size, a.max_context_len, a.part_tokens,
            seq_start);
}

// ---------------------------------------------------------------------------
// Causal chunked prefill.  Sequence s owns query tokens q0..q1-1 (n = q1 - q0
// of them, the last n tokens of its context of ctx tokens, already written to
// the cache); query i sits at position ctx - n + i and attends keys 0..ctx-n+i.
// The rows of KV head kvh are (query i, head kvh*G + r) for r < G, numbered
// token-major so that a 16-row MFMA tile spans few positions; a workgroup takes
// 128 consecutive rows (8 waves x one 16-row tile), so every K/V element it
// stages is used by 128 rows.
//
// Keys are walked two blocks (32 keys) at a time through a ring of kStages
// LDS stages.  A stage holds the pair's K and V tiles; the 512 threads fill it
// with direct global->LDS copies (16 bytes per lane, no registers), kStages-1
// pairs ahead of the pair being computed, so the copies of later pairs are in
// flight while this one is on the matrix cores.  One barrier per pair: after
// it, the stage of the pair computed last is free and is refilled.  K rows keep
// their 16-byte slots XOR-swizzled by row (slot ^ r mod slots), V rows by
// vswz, so that the A-operand reads of K and the transposed reads of V spread
// over the LDS banks.  Keys past the context are copied from key 0 of the pair
// (finite data) and masked to probability 0; pairs past a tile's last causal
// position are skipped for that tile.
//
// Workgroup b takes group (s, kvh) = b % (S*Hkv) and row tile b / (S*Hkv), so
// when S*Hkv is a multiple of 8 the tiles of one group share an XCD (dispatch
// is round-robin over the 8 XCDs) and read the same K/V from that XCD's L2.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int kswz(int r) { return r % (D * 2 / 16); }

constexpr int kPrefillWaves = 8;                     // waves per prefill workgroup
constexpr int kPrefillThreads = 64 * kPrefillWaves;

// Direct global->LDS copy of 16 bytes per lane from a wave-uniform base plus a
// per-lane 32-bit offset (the scalar-base form of the instruction); lane l's
// bytes land at LDS address lds + 16 l.  Issued as assembly so that the
// compiler, which cannot tell LDS stages apart, does not drain every
// outstanding copy before each LDS read; the caller waits on vmcnt itself
// (copies complete in issue order) and issues no compiler-visible vector load
// between a copy and its wait.  The LDS destination goes in m0, which the
// compiler loads for the statement (a register operand, so it knows m0 is
// taken).
__device__ __forceinline__ void copy16_to_lds_at(const char* base, uint32_t voff, const void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_addr(lds)) : "memory");
}

// A row's running maximum is raised only when a score exceeds it by more than
// this (log2 units): until then probabilities stay below 2^8, exact enough in
// fp32 and in the bf16 pair, and the accumulator rescale is skipped.
constexpr float kRescaleLog2 = 8.f;

template <int D, int BS>
__global__ __launch_bounds__(kPrefillThreads, 4) void prefill_chunk_mfma_kernel(pkv_prefill_args a) {
  constexpr int KC = D / 32;
  constexpr int DC = D / 16;
  constexpr int RB = D * 2;
  constexpr int kTiles = kPrefillRowsPerWg / 16 / kPrefillWaves;   // 16-row tiles per wave
  constexpr int kStages = 4;                       // LDS ring depth (pairs)
  constexpr int kTileBytes = kBlock * RB;          // 16 keys' K (or V) rows of one head: an LDS tile
  constexpr int kTileKiB = kTileBytes / 1024;
  constexpr int kStageBytes = 4 * kTileBytes;      // K0 K1 V0 V1
  constexpr int kCopies = kStageBytes / (16 * kPrefillThreads);   // 16-byte copies per thread per stage
  static_assert(kStageBytes % (16 * kPrefillThreads) == 0 && kTiles >= 1, "prefill shape");
  constexpr int64_t kHeadTile = static_cast<int64_t>(BS) * RB;   // one (block, head) tile of the pool
  constexpr int kBPP = 2 * kBlock / BS;            // blocks per 32-key pair
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(RB * 8 >= 1024, "a 1 KiB copy covers rows of one 8-token block");
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
  const int32_t r0 = rt * kPrefillRowsPerWg;
  if (r0 >= rows) return;
  const int32_t r_end = min(rows, r0 + kPrefillRowsPerWg);
  const int32_t ctx = a.context_lens[s];
  if (ctx < nq || !len_ok(ctx, a.max_context_len, a.max_blocks_per_seq, BS)) {
    for (int idx = threadIdx.x; idx < (r_end - r0) * D; idx += kPrefillThreads) {
      const int32_t r = r0 + idx / D, d = idx % D;
      a.out[((static_cast<int64_t>(q0) + r / G) * Hq + kvh * G + r % G) * D + d] = __builtin_nanf("");
    }
    return;
  }
  const int32_t first_pos = ctx - nq;            // position of query 0
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const int64_t block_bytes = static_cast<int64_t>(Hkv) * kHeadTile;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache) + kvh * kHeadTile;
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache) + kvh * kHeadTile;

  const int32_t wg_lim = first_pos + (r_end - 1) / G + 1;      // keys the workgroup needs
  const int32_t npairs = (wg_lim + 2 * kBlock - 1) / (2 * kBlock);
  const int32_t nblk = (ctx + BS - 1) / BS;
  bool bad = false;

  // Copy i of wave w fills KiB kPrefillWaves*i + w of a stage: tile t = that KiB
  // / (tile KiB) (0: K0, 1: K1, 2: V0, 3: V1), rows of the tile in lane order;
  // LDS row r holds slot k of the tile row at the swizzled source slot.  The
  // copy reads rows of one pool block (block cp_blk[i] of the pair: a 1 KiB
  // copy never spans two blocks); the per-lane source offsets within it are
  // fixed: the row's, and the block's row 0 for keys past the context (finite
  // data that gets probability 0).
  uint32_t cp_off[kCopies], cp_off0[kCopies];
  int32_t cp_key[kCopies], cp_blk[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int kib = kPrefillWaves * i + wave;
    const int t = kib / kTileKiB;
    const int off = (kib % kTileKiB) * 1024 + 16 * lane;
    const int r = off / RB, k = (off % RB) / 16;
    const int slot = t < 2 ? (k ^ kswz<D>(r)) : (k ^ vswz<D>(r));
    const int key = kBlock * (t & 1) + r;                 // key of the row within the pair
    cp_key[i] = key;
    cp_blk[i] = ((kib % kTileKiB) * 1024 / RB + kBlock * (t & 1)) / BS;   // the copy's first row's block
    cp_off[i] = static_cast<uint32_t>((key % BS) * RB + 16 * slot);
    cp_off0[i] = static_cast<uint32_t>(16 * slot);
  }
  // the pair's block ids: ids[q] holds keys 32 pp + BS q ..; past the last
  // block a copy takes the pair's first block (all its rows past the context)
  auto issue = [&](int32_t pp, int32_t (&ids)[kBPP], char* stage) {
#pragma unroll
    for (int q = 0; q < kBPP; ++q)
      if (static_cast<uint32_t>(ids[q]) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; ids[q] = 0; }
    const bool tail = (pp + 1) * 2 * kBlock > ctx;     // some keys of the pair lie past the context
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int kib = kPrefillWaves * i + wave;
      const int t = kib / kTileKiB;
      const int32_t j = kBPP * pp + cp_blk[i];
      const int32_t id = j < nblk ? ids[cp_blk[i]] : ids[0];
      const char* base = (t < 2 ? kc : vc) + id * block_bytes;
      uint32_t voff = cp_off[i];
      if (tail && pp * 2 * kBlock + cp_key[i] >= ctx) voff = cp_off0[i];
      copy16_to_lds_at(base, voff, stage + kib * 1024);
    }
  };
  // the block ids of pair pp (entries past the context's last block are not
  // read: the last one is read again instead)
  auto pair_ids = [&](int32_t pp, int32_t (&ids)[kBPP]) {
#pragma unroll
    for (int q = 0; q < kBPP; ++q) ids[q] = load_block_id(table, __builtin_amdgcn_readfirstlane(min(kBPP * pp + q, nblk - 1)));
  };
#pragma unroll
  for (int pp = 0; pp < kStages - 1; ++pp)
    if (pp < npairs) {
      int32_t ids[kBPP];
      pair_ids(pp, ids);
      issue(pp, ids, ring[pp]);
    }
  // the ids of the next pair to issue, loaded a pair ahead of its copies
  int32_t nids[kBPP];
#pragma unroll
  for (int q = 0; q < kBPP; ++q) nids[q] = 0;
  if (kStages - 1 < npairs) pair_ids(kStages - 1, nids);

  // this lane's rows (one per tile) and their key limits; invalid rows: limit 0,
  // q = 0 (their results are never written).  Keys below nomask_lim are visible
  // to every valid row of the tile.
  bf16x8 qb[kTiles][KC];
  int32_t lim[kTiles];
  int32_t tile_lim[kTiles];      // keys any row of the tile needs (uniform)
  int32_t nomask_lim[kTiles];
  int32_t wave_lim = 0;
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    const int32_t rbase = r0 + (wave * kTiles + tt) * 16;
    const int32_t r = rbase + n;
    const bool valid = r < r_end;
    const int32_t i = valid ? r / G : 0;
    lim[tt] = valid ? first_pos + i + 1 : 0;
    const int32_t rlast = min(r_end, rbase + 16) - 1;
    tile_lim[tt] = rlast >= rbase ? first_pos + rlast / G + 1 : 0;
    nomask_lim[tt] = first_pos + rbase / G + 1;
    wave_lim = max(wave_lim, tile_lim[tt]);
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((static_cast<int64_t>(q0) + i) * Hq + kvh * G + (valid ? r % G : 0)) * D * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 64 * c + 16 * g);
      if (!valid || a.q_mode == 2) w = u32x4{0, 0, 0, 0};
      if (a.q_mode == 1) w ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};   // -q, exactly
      qb[tt][c] = as_bf16x8(w);
    }
  }

  const float c2 = a.scale_log2;                 // > 0 (the scale's sign is in q)
  const float rescale_raw = kRescaleLog2 / c2;   // kRescaleLog2 in raw score units

  // m: the row's running maximum in log2 units (scores times c2); thr: the raw
  // score above which it is raised (the maximum it was last set from, plus
  // rescale_raw)
  f32x4 o[kTiles][DC];
  float m[kTiles], thr[kTiles], lsum[kTiles];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    m[tt] = kNegBig;
    thr[tt] = kNegBig;
    lsum[tt] = 0.f;
#pragma unroll
    for (int c = 0; c < DC; ++c) o[tt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // per-lane LDS offsets within a stage: K A-operand rows (key n of each block,
  // slot 4c + g) and the V transposed-read rows (key 4g + n/4); the V addresses
  // are those of stage 0, the other stages sit at fixed offsets from them
  const int k_row = n * RB;
  const int k_sw = kswz<D>(n);
  const int tr_row = 4 * g + (n >> 2);
  const int tr_sw = vswz<D>(tr_row);
  const int tr_k0 = (n & 3) >> 1;
  // (held opaque, so that each stays one register and a stage's reads take
  // the stage offset as an immediate instead of re-adding its parts per pair)
  const uint32_t ring0 = lds_addr(ring[0]);
  uint32_t k_addr[KC], tr_addr[DC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    k_addr[c] = ring0 + k_row + 16 * ((4 * c + g) ^ k_sw);
    asm volatile("" : "+v"(k_addr[c]));
  }
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    tr_addr[c] = ring0 + 2 * kTileBytes + tr_row * RB + 8 * (n & 1) + 16 * ((2 * c + tr_k0) ^ tr_sw);
    asm volatile("" : "+v"(tr_addr[c]));
  }

  // One pair of blocks (32 keys) from its stage.
  auto pair = [&](int32_t pp, const char* stage) {
    const int32_t key0 = pp * 2 * kBlock;
    if (key0 >= wave_lim) return;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      if (key0 >= tile_lim[tt]) continue;
      // S^T = K Q^T for the two blocks, K straight from LDS in the A layout
      const uint32_t stage_off = static_cast<uint32_t>(stage - ring[0]);
      // the matrix-core phases (K Q^T here, P V below) run at a raised issue
      // priority, so that a SIMD whose other waves are in their softmax keeps
      // its matrix core fed and their vector instructions fill the gaps
      __builtin_amdgcn_s_setprio(1);
      f32x4 acc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        bf16x8 ka[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) ka[c] = as_bf16x8(lds_read16_at(k_addr[c] + stage_off + b * kTileBytes));
        acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) acc[b] = mfma(ka[c], qb[tt][c], acc[b]);
      }
      float sc[8];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sc[4 * b + jj] = acc[b][jj];
      if (key0 + 2 * kBlock > nomask_lim[tt]) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (key0 + b * kBlock + 4 * g + jj >= lim[tt]) sc[4 * b + jj] = -INFINITY;
      }
      __builtin_amdgcn_s_setprio(0);
      // the lane's maximum (NaN-propagating three-input instructions, no
      // operand quieting) against the row's threshold: only when some score
      // passes it are the row maxima formed and the row maximum raised (with
      // the rescale); the branch is uniform over the wave
      const float lane_mx = __builtin_elementwise_maximum(
          __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[0], sc[1]),
                                        __builtin_elementwise_maximum(sc[2], sc[3])),
          __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[4], sc[5]),
                                        __builtin_elementwise_maximum(sc[6], sc[7])));
      if (__builtin_amdgcn_ballot_w64(lane_mx > thr[tt])) {
        const float mx = max_over_rows(lane_mx);
        const bool up = mx > thr[tt];            // the same in the four lanes of a row
        const float mnew = up ? mx * c2 : m[tt];
        const float alpha = fast_exp2(m[tt] - mnew);
        m[tt] = mnew;
        thr[tt] = up ? mx + rescale_raw : thr[tt];
        lsum[tt] *= alpha;
#pragma unroll
        for (int c = 0; c < DC; ++c) o[tt][c] *= alpha;
      }
      // V^T for the 32 keys by transposed reads, issued before the exponentials
      bf16x8 va[DC];
#pragma unroll
      for (int c = 0; c < DC; ++c)
        va[c] = join(lds_read_tr_at(tr_addr[c] + stage_off), lds_read_tr_at(tr_addr[c] + stage_off + kTileBytes));
      u32x4 phw, plw;
      float ps[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x2 pr = {fast_exp2(fmaf(sc[2 * k], c2, -m[tt])), fast_exp2(fmaf(sc[2 * k + 1], c2, -m[tt]))};
        ps[k] = pr[0] + pr[1];
        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        const f32x2 lo = {pr[0] - __uint_as_float(h << 16), pr[1] - __uint_as_float(h & 0xFFFF0000u)};
        phw[k] = h;
        plw[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
      }
      lsum[tt] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      const bf16x8 ph = as_bf16x8(phw), pl = as_bf16x8(plw);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        f32x4 t = mfma(va[c], ph, o[tt][c]);
        o[tt][c] = mfma(va[c], pl, t);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  static_assert(kStages == 4 && (kCopies == 1 || kCopies == 2 || kCopies == 4), "wait counts");
  for (int32_t p0 = 0; p0 < npairs; p0 += kStages) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int32_t pp = p0 + st;
      if (pp >= npairs) break;
      // this pair's copies have landed once at most the later issued pairs'
      // copies are outstanding (copies complete in issue order)
      const int32_t ahead = min(kStages - 2, npairs - 1 - pp);
      if (ahead >= 2) {
        if constexpr (kCopies == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if constexpr (kCopies == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      } else if (ahead == 1) {
        if constexpr (kCopies == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else if constexpr (kCopies == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // the pair issued after this one takes the ids loaded a pair ago; the
      // ids of the pair after it are loaded now, with no LDS read pending,
      // and arrive during the barrier
      const int32_t pn = pp + kStages - 1;
      int32_t ids[kBPP];
#pragma unroll
      for (int q = 0; q < kBPP; ++q) ids[q] = nids[q];
      if (pn + 1 < npairs) pair_ids(pn + 1, nids);
      __builtin_amdgcn_s_barrier();
      pair(pp, ring[st]);
      // every wave passed the barrier after it finished the pair before this
      // one, so that pair's stage takes pair pp + kStages - 1
      if (pn < npairs) issue(pn, ids, ring[(st + kStages - 1) % kStages]);
    }
  }

  // a bad block id anywhere in the workgroup's range poisons its rows
  const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    float L = lsum[tt];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const int32_t r = r0 + (wave * kTiles + tt) * 16 + n;
    if (r >= r_end) continue;
    const float inv = any_bad ? __builtin_nanf("") : 1.f / L;
    float* orow = a.out + ((static_cast<int64_t>(q0) + r / G) * Hq + kvh * G + r % G) * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const f32x4 v = o[tt][c] * inv;
      *reinterpret_cast<f32x4*>(orow + 16 * c + 4 * g) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode for wide query-head groups: 17..64 query heads per KV head (down to
// one KV head for all of them).  The group kernel above gives each 16-row
// slice of such a group a workgroup of its own, so every K/V tile crosses
// from L2 into a CU once per slice.  Here one workgroup per (unit, KV head)
// stages the unit's K/V once in LDS -- the prefill kernel's ring of 32-key
// stages, filled by direct global->LDS copies kStages-1 stages ahead -- and
// wave w computes slice w (query heads kvh*G + 16w ..) over every stage with
// the prefill kernel's softmax (the row maximum raised only past a 2^8
// margin, the bf16 probability pair).  Keys past the context are copied from
// key 0 of their pair and masked.  With the cache write, token ctx-1's rows
// are copied from the step's rows when the new slot is token ctx-1's, and
// stored into the pool by the workgroup; any other slot gives NaN rows.
// Each wave writes its rows, or their partials and one step on its slice's
// ticket (the group kernel's ticket layout), merging the slice if it is last.
// Partitions start at multiples of 1024 tokens (wide groups take no shared
// prefix), so every 32-key stage lies in whole blocks.
// ---------------------------------------------------------------------------
constexpr int kWideWaves = 4;
constexpr int kWideThreads = 64 * kWideWaves;

// Direct global->LDS copy of 16 bytes per lane from a per-lane 64-bit address
// (the vector-address form of the instruction), under the same rules as
// copy16_to_lds_at.
__device__ __forceinline__ void copy16_to_lds_va(const char* p, const void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(p), "{m0}"(lds_addr(lds)) : "memory");
}

template <int D, int BS>
__global__ __launch_bounds__(kWideThreads, 2) void decode_wide_group_kernel(pkv_decode_args a) {
  constexpr int KC = D / 32;
  constexpr int DC = D / 16;
  constexpr int RB = D * 2;
  constexpr int kStages = 4;                       // LDS ring depth (32-key stages)
  constexpr int kTileBytes = kBlock * RB;          // 16 keys' K (or V) rows
  constexpr int kTileKiB = kTileBytes / 1024;
  constexpr int kStageBytes = 4 * kTileBytes;      // K0 K1 V0 V1
  constexpr int kCopies = kStageBytes / (16 * kWideThreads);   // 16-byte copies per thread per stage
  static_assert(kStageBytes % (16 * kWideThreads) == 0 && (kCopies == 2 || kCopies == 4), "wide decode shape");
  constexpr int64_t kHeadTile = static_cast<int64_t>(BS) * RB;
  constexpr int kBPP = 2 * kBlock / BS;            // blocks per 32-key stage
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(RB * 8 >= 1024, "a 1 KiB copy covers rows of one 8-token block");
  __shared__ __align__(16) char ring[kStages][kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;

  const int32_t Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  const int32_t nsl = (G + 15) / 16;               // 2..4 slices
  const bool active = wave < nsl;                  // this wave has a slice
  const int32_t R = active ? min(16, G - 16 * wave) : 0;
  const uint32_t bid = blockIdx.x;
  const int32_t u = static_cast<int32_t>(bid / static_cast<uint32_t>(Hkv));
  const int32_t kvh = static_cast<int32_t>(bid - static_cast<uint32_t>(u) * Hkv);
  const int32_t* plan = a.plan;
  if (!plan_matches(plan, a)) {
    // a plan built for other sizes: every row is NaN
    if (u < a.num_seqs)
      for (int idx = threadIdx.x; idx < G * D; idx += kWideThreads)
        a.out[(static_cast<int64_t>(u) * Hq + kvh * G) * D + idx] = __builtin_nanf("");
    return;
  }
  if (u >= plan[0]) return;
  const int32_t* units = pkvd::plan_units(plan);
  const int32_t s = units[2 * u];
  const int32_t p = units[2 * u + 1];
  const int32_t ctx = a.context_lens[s];
  const int64_t grow0 = static_cast<int64_t>(s) * Hq + kvh * G;   // the group's first output row
  if (p < 0) {
    // no attention work: an empty context gives 0, an invalid one NaN
    for (int idx = threadIdx.x; idx < G * D; idx += kWideThreads)
      a.out[grow0 * D + idx] = ctx == 0 ? 0.f : __builtin_nanf("");
    return;
  }
  const int32_t part = a.part_tokens;
  const int32_t np_s = (ctx + part - 1) / part;
  const int32_t k_begin = p * part;
  const int32_t k_end = min(ctx, k_begin + part);
  const int32_t npairs = (k_end - k_begin + 2 * kBlock - 1) / (2 * kBlock);
  const int32_t blk0 = k_begin / BS;               // the unit's first block
  const int32_t nblk = (ctx + BS - 1) / BS;
  const bool direct = np_s == 1;
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const int64_t block_bytes = static_cast<int64_t>(Hkv) * kHeadTile;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache) + kvh * kHeadTile;
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache) + kvh * kHeadTile;
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

  // Copy i of wave w fills KiB kWideWaves*i + w of a stage (0: K0, 1: K1, 2:
  // V0, 3: V1 by tile), rows in lane order, LDS row r's 16-byte slot k from
  // the swizzled source slot; the copy's rows lie in one pool block (block
  // cp_blk[i] of the stage).
  uint32_t cp_off[kCopies], cp_slot[kCopies];
  int32_t cp_key[kCopies], cp_blk[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int kib = kWideWaves * i + wave;
    const int t = kib / kTileKiB;
    const int off = (kib % kTileKiB) * 1024 + 16 * lane;
    const int r = off / RB, k = (off % RB) / 16;
    const int slot = t < 2 ? (k ^ kswz<D>(r)) : (k ^ vswz<D>(r));
    const int key = kBlock * (t & 1) + r;               // key of the row within the stage
    cp_key[i] = key;
    cp_blk[i] = ((kib % kTileKiB) * 1024 / RB + kBlock * (t & 1)) / BS;
    cp_off[i] = static_cast<uint32_t>((key % BS) * RB + 16 * slot);
    cp_slot[i] = static_cast<uint32_t>(16 * slot);
  }
  auto issue = [&](int32_t pp, int32_t (&ids)[kBPP], char* stage) {
#pragma unroll
    for (int q = 0; q < kBPP; ++q)
      if (static_cast<uint32_t>(ids[q]) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; ids[q] = 0; }
    const int32_t key0 = k_begin + pp * 2 * kBlock;
    const bool tail = key0 + 2 * kBlock > ctx;         // some keys of the stage lie past the context
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int kib = kWideWaves * i + wave;
      const int t = kib / kTileKiB;
      const int32_t j = blk0 + kBPP * pp + cp_blk[i];
      const int32_t id = j < nblk ? ids[cp_blk[i]] : ids[0];
      const int32_t key = key0 + cp_key[i];
      const char* src = (t < 2 ? kc : vc) + id * block_bytes + cp_off[i];
      if (tail && key >= ctx) src = (t < 2 ? kc : vc) + id * block_bytes + cp_slot[i];
      if (use_new && key == ctx - 1) src = (t < 2 ? nk : nv) + cp_slot[i];
      copy16_to_lds_va(src, stage + kib * 1024);
    }
  };
  // the stage's block ids (entries past the context's last block are not
  // read: the last one is read again instead)
  auto pair_ids = [&](int32_t pp, int32_t (&ids)[kBPP]) {
#pragma unroll
    for (int q = 0; q < kBPP; ++q)
      ids[q] = load_block_id(table, __builtin_amdgcn_readfirstlane(min(blk0 + kBPP * pp + q, nblk - 1)));
  };
#pragma unroll
  for (int pp = 0; pp < kStages - 1; ++pp)
    if (pp < npairs) {
      int32_t ids[kBPP];
      pair_ids(pp, ids);
      issue(pp, ids, ring[pp]);
    }
  int32_t nids[kBPP];
#pragma unroll
  for (int q = 0; q < kBPP; ++q) nids[q] = 0;
  if (kStages - 1 < npairs) pair_ids(kStages - 1, nids);

  // the wave's query rows as the B operand (rows >= R: q = 0, never written);
  // the scale's sign goes into q so that the exponent factor c2 is positive
  const float sl = a.scale_log2;
  const int q_mode = sl > 0.f ? 0 : sl < 0.f ? 1 : 2;
  const float c2 = q_mode == 2 ? 1.f : fabsf(sl);
  const float rescale_raw = kRescaleLog2 / c2;
  bf16x8 qb[KC];
  {
    // (a wave without a slice reads the group's first row and zeroes it)
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((grow0 + (n < R ? 16 * wave + n : 0)) * D) * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 64 * c + 16 * g);
      if (n >= R || q_mode == 2) w = u32x4{0, 0, 0, 0};
      if (q_mode == 1) w ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};   // -q, exactly
      qb[c] = as_bf16x8(w);
    }
  }

  f32x4 o[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegBig, thr = kNegBig, lsum = 0.f;
  const int k_row = n * RB;
  const int k_sw = kswz<D>(n);
  const int tr_row = 4 * g + (n >> 2);
  const int tr_sw = vswz<D>(tr_row);
  const int tr_k0 = (n & 3) >> 1;
  const uint32_t ring0 = lds_addr(ring[0]);
  uint32_t k_addr[KC], tr_addr[DC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    k_addr[c] = ring0 + k_row + 16 * ((4 * c + g) ^ k_sw);
    asm volatile("" : "+v"(k_addr[c]));
  }
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    tr_addr[c] = ring0 + 2 * kTileBytes + tr_row * RB + 8 * (n & 1) + 16 * ((2 * c + tr_k0) ^ tr_sw);
    asm volatile("" : "+v"(tr_addr[c]));
  }

  // One 32-key stage: S^T = K Q^T, the online softmax, O^T += V^T P^T.
  auto pair = [&](int32_t pp, const char* stage) {
    const int32_t key0 = k_begin + pp * 2 * kBlock;
    const uint32_t stage_off = static_cast<uint32_t>(stage - ring[0]);
    __builtin_amdgcn_s_setprio(1);
    f32x4 acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      bf16x8 ka[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) ka[c] = as_bf16x8(lds_read16_at(k_addr[c] + stage_off + b * kTileBytes));
      acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) acc[b] = mfma(ka[c], qb[c], acc[b]);
    }
    float sc[8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sc[4 * b + jj] = acc[b][jj];
    if (key0 + 2 * kBlock > ctx) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (key0 + b * kBlock + 4 * g + jj >= ctx) sc[4 * b + jj] = -INFINITY;
    }
    __builtin_amdgcn_s_setprio(0);
    const float lane_mx = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[0], sc[1]),
                                      __builtin_elementwise_maximum(sc[2], sc[3])),
        __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[4], sc[5]),
                                      __builtin_elementwise_maximum(sc[6], sc[7])));
    if (__builtin_amdgcn_ballot_w64(lane_mx > thr)) {
      const float mx = max_over_rows(lane_mx);
      const bool up = mx > thr;
      const float mnew = up ? mx * c2 : m;
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      thr = up ? mx + rescale_raw : thr;
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < DC; ++c) o[c] *= alpha;
    }
    bf16x8 va[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c)
      va[c] = join(lds_read_tr_at(tr_addr[c] + stage_off), lds_read_tr_at(tr_addr[c] + stage_off + kTileBytes));
    u32x4 phw, plw;
    float ps[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x2 pr = {fast_exp2(fmaf(sc[2 * k], c2, -m)), fast_exp2(fmaf(sc[2 * k + 1], c2, -m))};
      ps[k] = pr[0] + pr[1];
      const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
      const f32x2 lo = {pr[0] - __uint_as_float(h << 16), pr[1] - __uint_as_float(h & 0xFFFF0000u)};
      phw[k] = h;
      plw[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
    }
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    const bf16x8 ph = as_bf16x8(phw), pl = as_bf16x8(plw);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      f32x4 t = mfma(va[c], ph, o[c]);
      o[c] = mfma(va[c], pl, t);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  for (int32_t p0 = 0; p0 < npairs; p0 += kStages) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int32_t pp = p0 + st;
      if (pp >= npairs) break;
      // this stage's copies have landed once at most the later issued stages'
      // copies are outstanding (copies complete in issue order)
      const int32_t ahead = min(kStages - 2, npairs - 1 - pp);
      if (ahead >= 2) {
        if constexpr (kCopies == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else if (ahead == 1) {
        if constexpr (kCopies == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int32_t pn = pp + kStages - 1;
      int32_t ids[kBPP];
#pragma unroll
      for (int q = 0; q < kBPP; ++q) ids[q] = nids[q];
      if (pn + 1 < npairs) pair_ids(pn + 1, nids);
      __builtin_amdgcn_s_barrier();
      if (active) pair(pp, ring[st]);
      if (pn < npairs) issue(pn, ids, ring[(st + kStages - 1) % kStages]);
    }
  }

  // a bad block id anywhere in the unit's range, or a wrong new slot, poisons its rows
  const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
  if (use_new && threadIdx.x < 2 * RB / 16) {
    // the new token's K and V rows into the pool (16 bytes per thread)
    const int half = threadIdx.x / (RB / 16), piece = threadIdx.x % (RB / 16);
    const char* src = (half == 0 ? nk : nv) + 16 * piece;
    char* dst = const_cast<char*>(half == 0 ? kc : vc) + new_blk * block_bytes + ((ctx - 1) % BS) * RB + 16 * piece;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
  if (!active) return;
  float L = lsum;
  L += __shfl_xor(L, 16);
  L += __shfl_xor(L, 32);
  const int64_t row0 = grow0 + 16 * wave;          // the wave's first row
  if (direct) {
    if (n < R) {
      const float inv = any_bad ? __builtin_nanf("") : 1.f / L;
      float* orow = a.out + (row0 + n) * D;
#pragma unroll
      for (int c = 0; c < DC; ++c) *reinterpret_cast<f32x4*>(orow + 16 * c + 4 * g) = o[c] * inv;
    }
    return;
  }
  // a split context: the wave's partial (the running maximum it scaled by,
  // the sum, the accumulator), then one step on its slice's ticket
  if (n < R) {
    const int64_t pidx = (row0 + n) * a.num_partitions + p;
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        pkvd::store_coherent(a.part_acc + pidx * D + 16 * c + 4 * g + jj,
                             any_bad ? __builtin_nanf("") : o[c][jj]);
    if (g == 0) {
      pkvd::store_coherent(a.part_ml + 2 * pidx, m);
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

}  // namespace

namespace {
// A kernel instance for the launch's head_dim and block size.
template <template <int, int> class K, typename... Args>
void launch_d_bs(int head_dim, int block_size, dim3 grid, hipStream_t st, Args... args) {
  if (head_dim == 128) {
    if (block_size == 8) K<128, 8>::launch(grid, st, args...);
    else if (block_size == 32) K<128, 32>::launch(grid, st, args...);
    else K<128, 16>::launch(grid, st, args...);
  } else {
    if (block_size == 8) K<64, 8>::launch(grid, st, args...);
    else if (block_size == 32) K<64, 32>::launch(grid, st, args...);
    else K<64, 16>::launch(grid, st, args...);
  }
}
template <int D, int BS>
struct GroupDecode {
  static void launch(dim3 grid, hipStream_t st, const pkv_decode_args& a) {
    hipLaunchKernelGGL((decode_group_mfma_kernel<D, BS>), grid, dim3(kGroupThreads), 0, st, a);
  }
};
template <int D, int BS>
struct WideGroupDecode {
  static void launch(dim3 grid, hipStream_t st, const pkv_decode_args& a) {
    hipLaunchKernelGGL((decode_wide_group_kernel<D, BS>), grid, dim3(kWideThreads), 0, st, a);
  }
};
template <int D, int BS>
struct SharedUnits {
  static void launch(dim3 grid, hipStream_t st, const pkv_decode_args& a) {
    hipLaunchKernelGGL((decode_shared_mfma_kernel<D, BS>), grid, dim3(kGroupThreads), 0, st, a);
  }
};
}  // namespace

int pkv_launch_decode_group(const pkv_decode_args& a, void* stream) {
  const int64_t np = (a.max_context_len + a.part_tokens - 1) / a.part_tokens;
  if (pkv_wide_group(a.dtype, a.num_heads, a.num_kv_heads)) {
    // one workgroup per (unit, KV head) for all the group's slices
    const int64_t units = static_cast<int64_t>(a.num_seqs) * (np < 1 ? 1 : np) * a.num_kv_heads;
    launch_d_bs<WideGroupDecode>(a.head_dim, a.block_size, dim3(static_cast<uint32_t>(units)),
                                 static_cast<hipStream_t>(stream), a);
    return hipGetLastError();
  }
  const int32_t slices = (a.num_heads / a.num_kv_heads + kMaxMfmaGroup - 1) / kMaxMfmaGroup;
  const int64_t units = static_cast<int64_t>(a.num_seqs) * (np < 1 ? 1 : np) * a.num_kv_heads;
  const int64_t grid = slices == 1 ? units : (units + 7) / 8 * 8 * slices;
  launch_d_bs<GroupDecode>(a.head_dim, a.block_size, dim3(static_cast<uint32_t>(grid)),
                           static_cast<hipStream_t>(stream), a);
  return hipGetLastError();
}

int pkv_launch_shared_plans(const pkv_decode_args& a, const int32_t* group_start, int32_t num_groups,
                            int32_t* seq_start, int32_t* shared_plan, int32_t* plan, void* stream) {
  hipLaunchKernelGGL(shared_plans_kernel, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), a, group_start,
                     num_groups, seq_start, shared_plan, plan);
  return hipGetLastError();
}

int pkv_launch_shared_units(const pkv_decode_args& a, void* stream) {
  // at most num_seqs sub-groups, each with ceil(max_context_len / partition) units
  const int64_t npp = (a.max_context_len + a.prefix_part_tokens - 1) / a.prefix_part_tokens;
  const int64_t shared = static_cast<int64_t>(a.num_seqs) * (npp < 1 ? 1 : npp) * a.num_kv_heads;
  launch_d_bs<SharedUnits>(a.head_dim, a.block_size, dim3(static_cast<uint32_t>(shared)),
                           static_cast<hipStream_t>(stream), a);
  return hipGetLastError();
}

namespace {
template <int D, int BS>
struct Prefill {
  static void launch(dim3 grid, hipStream_t st, const pkv_prefill_args& a) {
    hipLaunchKernelGGL((prefill_chunk_mfma_kernel<D, BS>), grid, dim3(kPrefillThreads), 0, st, a);
  }
};
}  // namespace

int pkv_launch_prefill(const pkv_prefill_args& a, void* stream) {
  const int32_t group = a.num_heads / a.num_kv_heads;
  const int64_t tiles = (static_cast<int64_t>(a.max_query_len) * group + kPrefillRowsPerWg - 1) / kPrefillRowsPerWg;
  const int64_t grid = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * tiles;
  if (grid == 0) return hipSuccess;
  launch_d_bs<Prefill>(a.head_dim, a.block_size, dim3(static_cast<uint32_t>(grid)), static_cast<hipStream_t>(stream),
                       a);
  return hipGetLastError();
}

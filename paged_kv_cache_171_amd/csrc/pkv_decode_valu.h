// Vector-ALU paged decode (one query per (sequence, head)) as a device
// function run by the decode kernel, also for the sequences' own tokens of a
// shared-prefix decode (units from a per-sequence start).
#pragma once

#include "pkv_device.h"

namespace {

using pkvd::u32x4;
using pkvd::kNegBig;
using pkvd::kPlanHdr;
using pkvd::fast_exp2;
using pkvd::len_ok;
using pkvd::plan_matches;

constexpr int kValuWaves = 4;     // waves per VALU decode workgroup

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
// partial (max, sum, unnormalised accumulator), and the row's last unit to
// finish merges the row.
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

template <typename T, int D, int BS>
__device__ __forceinline__ void decode_valu_body(const pkv_decode_args& a, uint32_t bid) {
  using S = DecodeShape<T, D, BS>;
  constexpr int kBlock = BS;          // tokens per block of this instance
  constexpr int EPL = S::kEpl, LPR = S::kLpr, TPL = S::kTpl, NLD = S::kNld, BPI = S::kBpi;

  __shared__ float sm_acc[kValuWaves][D];
  __shared__ float sm_ml[kValuWaves][2];
  __shared__ int sm_bad[kValuWaves];
  __shared__ int sm_last;
  __shared__ int sm_peek;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int row = lane / LPR;
  const int col = lane % LPR;

  const int32_t Hq = a.num_heads;
  const int32_t u = static_cast<int32_t>(bid / Hq);
  const int32_t h = static_cast<int32_t>(bid - static_cast<uint32_t>(u) * Hq);
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
  constexpr int kRowBytes = D * sizeof(T);
  const int32_t G = Hq / a.num_kv_heads;
  const int32_t kvh = h / G;
  const int64_t block_bytes = static_cast<int64_t>(a.num_kv_heads) * kTileBytes;
  const int64_t head_off = static_cast<int64_t>(kvh) * kTileBytes;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache);
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  bool bad = false;

  // The step's new token (decode with the cache write): in the unit that holds
  // the sequence's last token, the block loop covers tokens 0 .. ctx-2 only,
  // and wave 0 adds token ctx-1 afterwards -- from the new K/V, loaded here
  // into registers, when the slot is token ctx-1's (one workgroup per KV head
  // then stores the row into the pool), else from the pool (no new token this
  // step).  So the loop neither stores nor waits on anything extra.
  const bool with_new = a.new_slots != nullptr && blk_end == nblk;
  const int32_t ctx_loop = with_new ? ctx - 1 : ctx;
  const int32_t loop_end = with_new ? min(blk_end, (ctx_loop + kBlock - 1) / kBlock) : blk_end;
  int64_t new_slot = -1;
  int32_t last_id = 0;
  u32x4 nk_row{0, 0, 0, 0}, nv_row{0, 0, 0, 0};
  if (with_new && wave == 0) {
    new_slot = a.new_slots[s];
    last_id = table[nblk - 1];
    const int64_t src = (static_cast<int64_t>(s) * a.num_kv_heads + kvh) * kRowBytes + 16 * col;
    nk_row = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.new_k) + src);
    nv_row = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.new_v) + src);
  }

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

  // Online-softmax update with the tile of tokens t0 .. t0+kBlock-1 (rows past
  // the context are masked).
  auto update = [&](const u32x4 (&kt)[NLD], const u32x4 (&vt)[NLD], int32_t t0) {
    const bool full = t0 + kBlock <= ctx_loop;
    float sc[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float kf[EPL];
      Elem<T>::unpack(kt[i], kf);
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
        const bool valid = t0 + i * TPL + row < ctx_loop;
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
      Elem<T>::unpack(vt[i], vf);
      if (!full) {
        const bool valid = t0 + i * TPL + row < ctx_loop;
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = valid ? vf[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pr, vf[e], acc[e]);
    }
  };

  // The block ids of the next iteration are fetched (scalar loads) while the
  // current iteration's tiles are in flight.
  int32_t nxt[BPI];
#pragma unroll
  for (int bi = 0; bi < BPI; ++bi) {
    const int32_t j = blk_begin + wave + bi * kValuWaves;
    nxt[bi] = j < loop_end ? table[j] : 0;
  }
  for (int32_t j0 = blk_begin + wave; j0 < loop_end; j0 += kValuWaves * BPI) {
    u32x4 kt[BPI][NLD], vt[BPI][NLD];
    int32_t tb[BPI];
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
      const int32_t j = j0 + bi * kValuWaves;
      int32_t b = nxt[bi];
      tb[bi] = -1;
      if (j < loop_end) {
        if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; b = 0; }
        tb[bi] = j * kBlock;
        const u32x4* kp = reinterpret_cast<const u32x4*>(kc + b * block_bytes + head_off);
        const u32x4* vp = reinterpret_cast<const u32x4*>(vc + b * block_bytes + head_off);
        // rows past the context (the tail of a sequence's last block) are not
        // loaded: those lanes read nothing and hold 0
        const int32_t valid = ctx_loop - j * kBlock;
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
      const int32_t j = j0 + kValuWaves * BPI + bi * kValuWaves;
      nxt[bi] = j < loop_end ? table[j] : 0;
    }
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
      if (tb[bi] < 0) break;
      update(kt[bi], vt[bi], tb[bi]);
    }
  }

  if (with_new && wave == 0) {
    // token ctx-1: one more key for the lanes of row 0 (the other rows mask it)
    const int32_t last_row = (ctx - 1) % kBlock;
    int32_t b = last_id;
    const bool id_bad = static_cast<uint32_t>(b) >= static_cast<uint32_t>(a.num_blocks);
    if (id_bad) { bad = true; b = 0; }
    char* krow = const_cast<char*>(kc) + b * block_bytes + head_off + last_row * kRowBytes + 16 * col;
    char* vrow = const_cast<char*>(vc) + b * block_bytes + head_off + last_row * kRowBytes + 16 * col;
    u32x4 kn = nk_row, vn = nv_row;
    if (new_slot < 0) {
      // no new token this step: the token is in the pool
      kn = *reinterpret_cast<const u32x4*>(krow);
      vn = *reinterpret_cast<const u32x4*>(vrow);
    } else if (id_bad || new_slot != static_cast<int64_t>(b) * kBlock + last_row) {
      bad = true;       // not token ctx-1's slot: NaN rows, nothing stored
    } else if (h % G == 0 && row == 0) {
      *reinterpret_cast<u32x4*>(krow) = kn;
      *reinterpret_cast<u32x4*>(vrow) = vn;
    }
    float kf[EPL], vf[EPL];
    Elem<T>::unpack(kn, kf);
    Elem<T>::unpack(vn, vf);
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) part = fmaf(qv[e], kf[e], part);
    const float dot = group_sum<LPR>(part);      // every lane takes part in the row sums
    const float sc = row == 0 ? dot : -INFINITY;
    const float mt = fmaxf(m, sc);
    const float alpha = fast_exp2(m - mt);
    m = mt;
    const float pr = fast_exp2(sc - m);
    l = l * alpha + pr;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pr, vf[e], acc[e] * alpha);
  }

  // A split row: one thread looks at the row's ticket now, so that the load
  // is in flight while the rows and waves merge.
  const bool split = np_s != 1 || base != 0;
  uint64_t* const ticket = split ? a.merge_tickets + static_cast<int64_t>(s) * Hq + h : nullptr;
  uint64_t seen = 0;
  if (split && threadIdx.x == 0) seen = pkvd::peek_ticket(ticket);

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
  if (threadIdx.x == 0) sm_peek = split && pkvd::ticket_all_others(seen, a.merge_epoch, base + np_s) ? 1 : 0;
  __syncthreads();
  float M = 0.f, L = 0.f, o = 0.f;
  const int t = threadIdx.x;
  if (t < D) {
    M = sm_ml[0][0];
#pragma unroll
    for (int v = 1; v < kValuWaves; ++v) M = fmaxf(M, sm_ml[v][0]);
#pragma unroll
    for (int v = 0; v < kValuWaves; ++v) {
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
  // a split context: this partition's (max, sum, accumulator), merged by the
  // row's last unit to finish -- at once, from registers, when every other
  // unit of the row had arrived before this one looked
  const int64_t prow = (static_cast<int64_t>(s) * Hq + h) * a.num_partitions;
  const int64_t pidx = prow + base + p;
  if (sm_peek) {
    if (t == 0) pkvd::reset_ticket(ticket);
    if (t < D)
      a.out[orow + t] = pkvd::merge_partials_coherent_self(a.part_ml + 2 * prow, a.part_acc + prow * D + t,
                                                           base + np_s, D, base + p, M, L, o);
    return;
  }
  if (t < D) {
    pkvd::store_coherent(a.part_acc + pidx * D + t, o);
    if (t == 0) { pkvd::store_coherent(a.part_ml + 2 * pidx, M); pkvd::store_coherent(a.part_ml + 2 * pidx + 1, L); }
  }
  if (!pkvd::arrive_last(ticket, a.merge_epoch, base + np_s, &sm_last)) return;
  if (t < D)
    a.out[orow + t] = pkvd::merge_partials_coherent(a.part_ml + 2 * prow, a.part_acc + prow * D + t, base + np_s, D);
}

}  // namespace

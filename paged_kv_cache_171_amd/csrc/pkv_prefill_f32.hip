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
// 32-token block); a workgroup's four waves take neighbouring tiles of one
// (sequence, KV head), so they read the same K/V rows close together in time
// and the repeats hit the CU's cache.  The waves share nothing else: no LDS,
// no barrier.
//
// Matrix-core layout of v_mfma_f32_16x16x4_f32: lane l, n = l % 16,
// g = l / 16, supplies A[n][g] and B[g][n] and receives D[4g + j][n] in
// register j.  The k index of a product can be any bijection shared by A and
// B; this kernel picks them so that every lane loads whole 16-byte pieces:
//     S^T = K Q^T   k = 4m + t  <->  dim 16m + 4g + t  (lane (n, g) loads
//                   K[key n] and Q[row n] at dims 16m + 4g .. +3)
//     O^T += V^T P^T  k = kk  <->  key 4g + kk, and output row i of tile dt
//                   <->  dim DT i + dt (lane n loads dims DT n .. DT n + DT-1
//                   of the four V rows 4g .. 4g+3)
// so the S^T result, lane (n, g) holding S[row n][key 4g + j], is already the
// P^T operand, and every per-row quantity lives in the lanes whose n is the
// row.  The softmax is the online one in base 2 with the maximum taken every
// tile: P is exact fp32, so there is nothing to gain from raising it lazily.
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

template <int D, int BS>
// Two waves per SIMD: each wave holds the K and V rows of two tiles (the next
// one loads while this one is on the matrix cores), 256 registers.
__global__ __launch_bounds__(64 * kF32Waves, 2) void prefill_chunk_f32_kernel(pkv_prefill_args a) {
  constexpr int KQ = D / 16;   // 16-byte pieces of a K or q row per lane
  constexpr int DT = D / 16;   // 16-dim output tiles; a lane holds DT dims of each of its V rows
  constexpr int DV = DT / 4;   // 16-byte pieces of those
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int64_t kHeadTile = static_cast<int64_t>(BS) * D;   // floats of one (block, head) tile

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
  const int32_t rbase = rt * kPrefillF32RowsPerWg + wave * 16;
  if (rbase >= rows) return;                   // no barrier below: an idle wave just leaves
  const int32_t r_end = min(rows, rbase + 16);
  const int32_t ctx = a.context_lens[s];
  if (ctx < nq || !len_ok(ctx, a.max_context_len, a.max_blocks_per_seq, BS)) {
    for (int idx = lane; idx < (r_end - rbase) * D; idx += 64) {
      const int32_t r = rbase + idx / D, d = idx % D;
      a.out[((static_cast<int64_t>(q0) + r / G) * Hq + kvh * G + r % G) * D + d] = __builtin_nanf("");
    }
    return;
  }
  const int32_t first_pos = ctx - nq;          // position of query 0
  const int32_t* __restrict__ table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const int64_t block_stride = static_cast<int64_t>(Hkv) * kHeadTile;
  const float* __restrict__ kc = static_cast<const float*>(a.k_cache) + kvh * kHeadTile;
  const float* __restrict__ vc = static_cast<const float*>(a.v_cache) + kvh * kHeadTile;
  const int32_t nblk = (ctx + BS - 1) / BS;

  // this lane's row; rows past the tile's end get key limit 0 and q = 0 (their
  // results are never written)
  const int32_t r = rbase + n;
  const bool valid = r < r_end;
  const int32_t i = valid ? r / G : 0;
  const int32_t lim = valid ? first_pos + i + 1 : 0;
  const int32_t tile_lim = first_pos + (r_end - 1) / G + 1;    // keys any row of the tile needs
  const int32_t nomask_lim = first_pos + rbase / G + 1;          // keys every row of the tile sees

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
  float m_run = kNegBig, lsum = 0.f;
  bool bad = false;

  const int32_t ntiles = (tile_lim + 15) / 16;
  // the tile's block ids (wave-uniform): its block, or with 8-token blocks its
  // two (the second clamped to the context's last block: keys past the context
  // are never read from it); a key past the context reads the tile's first key
  // instead (a cached token: finite data, masked to probability 0)
  auto load_tile = [&](int32_t t, f32x4 (&kv)[KQ], f32x4 (&vv)[4][DV]) {
    const int32_t key0 = 16 * t;
    const int32_t j0 = key0 / BS;
    int32_t id_a = load_block_id(table, __builtin_amdgcn_readfirstlane(j0));
    int32_t id_b = id_a;
    if constexpr (BS == 8) id_b = load_block_id(table, __builtin_amdgcn_readfirstlane(min(j0 + 1, nblk - 1)));
    if (static_cast<uint32_t>(id_a) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; id_a = 0; }
    if (static_cast<uint32_t>(id_b) >= static_cast<uint32_t>(a.num_blocks)) { bad = true; id_b = 0; }
    auto row_ptr = [&](const float* base, int32_t off) {
      const int32_t o2 = key0 + off < ctx ? off : 0;
      const int32_t id = (BS == 8 && o2 >= 8) ? id_b : id_a;
      return base + id * block_stride + ((key0 + o2) % BS) * D;
    };
    {
      const float* krow = row_ptr(kc, n);
#pragma unroll
      for (int m = 0; m < KQ; ++m) kv[m] = *reinterpret_cast<const f32x4*>(krow + 16 * m + 4 * g);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float* vrow = row_ptr(vc, 4 * g + kk) + DT * n;
#pragma unroll
      for (int c = 0; c < DV; ++c) vv[kk][c] = *reinterpret_cast<const f32x4*>(vrow + 4 * c);
    }
  };
  // S^T = K Q^T (two accumulator chains), the online softmax over the tile's
  // 16 keys (base 2, maximum taken every tile), then O^T += V^T P^T
  auto compute_tile = [&](int32_t t, const f32x4 (&kv)[KQ], const f32x4 (&vv)[4][DV]) {
    const int32_t key0 = 16 * t;
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
    for (int m = 0; m < KQ; ++m)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (m & 1) acc1 = mfma4(kv[m][tt], qv[m][tt], acc1);
        else acc0 = mfma4(kv[m][tt], qv[m][tt], acc0);
      }
    f32x4 sc = acc0 + acc1;
    if (key0 + 16 > nomask_lim) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (key0 + 4 * g + j >= lim) sc[j] = -INFINITY;
    }
    const float mx = max_over_rows(max4(sc));
    const float mnew = __builtin_elementwise_maximum(m_run, mx * c2);
    const float alpha = fast_exp2(m_run - mnew);
    m_run = mnew;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(fmaf(sc[j], c2, -m_run));
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) o[dt] = mfma4(vv[kk][dt / 4][dt % 4], p[kk], o[dt]);
  };
  // two register sets, the loop unrolled by two so that each stays in place
  f32x4 kA[KQ], vA[4][DV], kB[KQ], vB[4][DV];
  if (ntiles > 0) load_tile(0, kA, vA);
  for (int32_t t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) load_tile(t + 1, kB, vB);
    compute_tile(t, kA, vA);
    if (t + 1 >= ntiles) break;
    if (t + 2 < ntiles) load_tile(t + 2, kA, vA);
    compute_tile(t + 1, kB, vB);
  }

  float L = lsum;
  L += __shfl_xor(L, 16);
  L += __shfl_xor(L, 32);
  if (!valid) return;
  // a bad block id in the tile's range poisons its rows
  const float inv = bad ? __builtin_nanf("") : 1.f / L;
  float* orow = a.out + ((static_cast<int64_t>(q0) + i) * Hq + kvh * G + r % G) * D;
  // lane (n, g) holds dims DT (4g + j) + dt of row n in o[dt][j]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < DV; ++c) {
      const f32x4 v = f32x4{o[4 * c][j], o[4 * c + 1][j], o[4 * c + 2][j], o[4 * c + 3][j]} * inv;
      *reinterpret_cast<f32x4*>(orow + DT * (4 * g + j) + 4 * c) = v;
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

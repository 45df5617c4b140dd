// Read-bandwidth probes for the bench (libpkv_probes.so, not part of the
// library's ABI): how fast this GPU reads HBM when nothing but reading is
// done, as a measured ceiling beside the 8 TB/s specification.
//
//   stream_read_kernel  -- one contiguous buffer streamed once with 16-byte
//                          loads (non-temporal or ordinary), UNROLL loads in
//                          flight per thread, a grid-stride loop over
//                          workgroup-sized chunks
//   tile_read_kernel    -- the paged decode access pattern and nothing else:
//                          whole (block, head) K and V tiles reached through
//                          block tables, one workgroup per (16-block chunk of a
//                          sequence, head), its four waves taking blocks in turn
//   mfma_rate_kernel    -- the bf16 matrix-core rate with no memory traffic:
//                          chains of v_mfma_f32_16x16x32_bf16 per wave (the
//                          instruction the prefill kernel is built on)
//   mfma32_rate_kernel  -- the same with the 32 x 32 x 16 bf16 instruction
//                          (v_mfma_f32_32x32x16_bf16: twice the work per
//                          instruction, half the operand reads per flop)
//   mfma_f32_rate_kernel -- the same for the fp32 matrix cores
//                          (v_mfma_f32_16x16x4_f32, the float32 prefill's)
//   overlap_kernel      -- how far matrix-core work of some waves and vector
//                          work (fma and exp2, the softmax's kind) of other
//                          waves on the same SIMD run at the same time: each
//                          wave takes its role from its slot on its SIMD (the
//                          HW_ID register), so every SIMD holds both kinds
//
// Every load feeds an XOR that is written only if it equals a constant, so
// the loads cannot be removed and nothing is stored in practice.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kMagic = 0x9E3779B9u;

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  constexpr int64_t kChunk = 256 * UNROLL;      // 16-byte units per workgroup per iteration
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk; base < n16;
       base += static_cast<int64_t>(gridDim.x) * kChunk) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) {
      const int64_t idx = base + i * 256 + threadIdx.x;
      if (idx < n16) v[i] = NT ? __builtin_nontemporal_load(buf + idx) : buf[idx];
      else v[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (acc == kMagic) sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

// One (block, head) tile of TILE16 16-byte units read by one wave.
template <int TILE16>
__device__ __forceinline__ uint32_t tile_xor(const u32x4* p, int lane) {
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < TILE16 / 64; ++i) {
    const u32x4 v = __builtin_nontemporal_load(p + i * 64 + lane);
    a ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  return a;
}

// work: (sequence, chunk) pairs; chunk c covers blocks 16c .. 16c+15 of the
// sequence's table (clipped to its context).  Tiles of tile_bytes bytes, a
// block holding num_heads of them.
template <int TILE16>
__global__ __launch_bounds__(256) void tile_read_kernel(const char* __restrict__ kc, const char* __restrict__ vc,
                                                        const int32_t* __restrict__ tables, int32_t max_blocks,
                                                        const int32_t* __restrict__ lens, int32_t block_size,
                                                        const int32_t* __restrict__ work, int32_t num_heads,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t wi = blockIdx.x / num_heads, h = blockIdx.x - (blockIdx.x / num_heads) * num_heads;
  const int32_t s = work[2 * wi], c = work[2 * wi + 1];
  const int32_t nblk = (lens[s] + block_size - 1) / block_size;
  const int32_t j0 = 16 * c, j1 = min(nblk, j0 + 16);
  const int32_t* t = tables + static_cast<int64_t>(s) * max_blocks;
  constexpr int64_t kTile = static_cast<int64_t>(TILE16) * 16;
  uint32_t acc = 0;
  for (int32_t j = j0 + wave; j < j1; j += 8) {
    const int64_t o1 = (static_cast<int64_t>(t[j]) * num_heads + h) * kTile;
    uint32_t a = tile_xor<TILE16>(reinterpret_cast<const u32x4*>(kc + o1), lane) ^
                 tile_xor<TILE16>(reinterpret_cast<const u32x4*>(vc + o1), lane);
    if (j + 4 < j1) {
      const int64_t o2 = (static_cast<int64_t>(t[j + 4]) * num_heads + h) * kTile;
      a ^= tile_xor<TILE16>(reinterpret_cast<const u32x4*>(kc + o2), lane) ^
           tile_xor<TILE16>(reinterpret_cast<const u32x4*>(vc + o2), lane);
    }
    acc ^= a;
  }
  if (acc == kMagic) sink[static_cast<int64_t>(blockIdx.x) * 4 + wave] = acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// CH independent accumulator chains per wave, iters MFMAs on each.
template <int CH>
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* __restrict__ out, int32_t iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(threadIdx.x * 0.001f + i);
    b[i] = static_cast<__bf16>(i * 0.5f);
  }
  f32x4 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = sum;
}

// CH independent accumulator chains per wave, iters 32 x 32 x 16 MFMAs on each.
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int CH>
__global__ __launch_bounds__(256) void mfma32_rate_kernel(float* __restrict__ out, int32_t iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(threadIdx.x * 0.001f + i);
    b[i] = static_cast<__bf16>(i * 0.5f);
  }
  f32x16 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += acc[c][j];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = sum;
}

// CH independent accumulator chains per wave, iters fp32 MFMAs on each.
template <int CH>
__global__ __launch_bounds__(256) void mfma_f32_rate_kernel(float* __restrict__ out, int32_t iters) {
  const float a = threadIdx.x * 1e-3f, b = 0.5f;
  f32x4 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = sum;
}

__device__ __forceinline__ float overlap_mfma(int32_t iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(threadIdx.x * 0.001f + i);
    b[i] = static_cast<__bf16>(i * 0.5f);
  }
  f32x4 c0 = f32x4{0.f, 0.f, 0.f, 0.f}, c1 = c0;
  for (int32_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
  }
  return c0[0] + c1[1];
}
// four independent chains, per step 4 fma, 4 exp2 and 4 adds
__device__ __forceinline__ float overlap_valu(int32_t iters) {
  float x0 = threadIdx.x * 1e-3f, x1 = x0 + 0.5f, x2 = x0 + 0.25f, x3 = x0 + 0.125f;
  float s = 0.f;
  for (int32_t it = 0; it < iters; ++it) {
    x0 = fmaf(x0, 0.999f, -0.001f);
    x1 = fmaf(x1, 0.999f, -0.001f);
    x2 = fmaf(x2, 0.999f, -0.001f);
    x3 = fmaf(x3, 0.999f, -0.001f);
    const float e0 = __builtin_amdgcn_exp2f(x0), e1 = __builtin_amdgcn_exp2f(x1);
    const float e2 = __builtin_amdgcn_exp2f(x2), e3 = __builtin_amdgcn_exp2f(x3);
    s += (e0 + e1) + (e2 + e3);
  }
  return s + x0 + x1 + x2 + x3;
}

// mode 0: every wave matrix work; 1: every wave vector work; 2: waves in odd
// slots vector work, the others matrix work; 3: only the matrix-role waves of
// mode 2 work; 4: only its vector-role ones.  out[i] gets the wave's result,
// plus 1e30 for a vector-role wave (so the host can count the roles).
__global__ __launch_bounds__(256) void overlap_kernel(float* __restrict__ out, int32_t mode, int32_t mfma_iters,
                                                      int32_t valu_iters) {
  const uint32_t hw_id = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);   // HW_ID, bits 31:0
  const bool odd = (hw_id & 1u) != 0;                                           // wave slot parity
  float r = 0.f;
  if (mode == 0) r = overlap_mfma(mfma_iters);
  else if (mode == 1) r = overlap_valu(valu_iters);
  else if (mode == 2) r = odd ? overlap_valu(valu_iters) : overlap_mfma(mfma_iters);
  else if (mode == 3) r = odd ? 0.f : overlap_mfma(mfma_iters);
  else r = odd ? overlap_valu(valu_iters) : 0.f;
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = odd ? r + 1e30f : r;
}

}  // namespace

// out: grid * 256 floats.  chains: 1 or 2 (each MFMA 16 x 16 x 4 x 2 = 2048
// flops).  Returns the launch status.
extern "C" int pkvprobe_mfma_f32_rate(float* out, int32_t grid, int32_t iters, int32_t chains, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (chains == 1)
    hipLaunchKernelGGL((mfma_f32_rate_kernel<1>), dim3(grid), dim3(256), 0, st, out, iters);
  else
    hipLaunchKernelGGL((mfma_f32_rate_kernel<2>), dim3(grid), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

// out: grid * 256 floats.  mode as overlap_kernel's (0..4).  Returns the
// launch status.
extern "C" int pkvprobe_overlap(float* out, int32_t grid, int32_t mode, int32_t mfma_iters, int32_t valu_iters,
                                void* stream) {
  hipLaunchKernelGGL(overlap_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), out, mode,
                     mfma_iters, valu_iters);
  return hipGetLastError();
}

// out: grid * 256 floats.  chains: 1 or 2 accumulator chains per wave (each
// MFMA 32 x 32 x 16 x 2 = 32768 flops).  Returns the launch status.
extern "C" int pkvprobe_mfma32_rate(float* out, int32_t grid, int32_t iters, int32_t chains, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (chains == 1)
    hipLaunchKernelGGL((mfma32_rate_kernel<1>), dim3(grid), dim3(256), 0, st, out, iters);
  else
    hipLaunchKernelGGL((mfma32_rate_kernel<2>), dim3(grid), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

// out: grid * 256 floats.  chains: 1 or 2 accumulator chains per wave (each
// MFMA 16 x 16 x 32 x 2 = 16384 flops).  Returns the launch status.
extern "C" int pkvprobe_mfma_rate(float* out, int32_t grid, int32_t iters, int32_t chains, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (chains == 1)
    hipLaunchKernelGGL((mfma_rate_kernel<1>), dim3(grid), dim3(256), 0, st, out, iters);
  else
    hipLaunchKernelGGL((mfma_rate_kernel<2>), dim3(grid), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

// bytes: a multiple of 16.  sink: at least grid * 256 uint32 words.  mode:
// UNROLL 4 / 8 / 16 with non-temporal loads (0 / 1 / 2) or ordinary loads (3 /
// 4 / 5).  Returns the launch status.
extern "C" int pkvprobe_stream_read(const void* buf, int64_t bytes, int32_t grid, int32_t mode, uint32_t* sink,
                                    void* stream) {
  const int64_t n16 = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(buf);
  switch (mode) {
    case 0: hipLaunchKernelGGL((stream_read_kernel<4, true>), dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    case 1: hipLaunchKernelGGL((stream_read_kernel<8, true>), dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<16, true>), dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    case 3: hipLaunchKernelGGL((stream_read_kernel<4, false>), dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    case 4: hipLaunchKernelGGL((stream_read_kernel<8, false>), dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    default: hipLaunchKernelGGL((stream_read_kernel<16, false>), dim3(grid), dim3(256), 0, st, p, n16, sink); break;
  }
  return hipGetLastError();
}

// tile_bytes: 4096 (16 tokens x 128 dims bf16) or 2048.  Every table entry of
// tokens below lens[s] must lie in the pools.  sink: num_work * num_heads * 4
// words.
extern "C" int pkvprobe_tile_read(const void* k_cache, const void* v_cache, const int32_t* tables,
                                  int32_t max_blocks, const int32_t* lens, int32_t block_size, const int32_t* work,
                                  int32_t num_work, int32_t num_heads, int32_t tile_bytes, uint32_t* sink,
                                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(num_work) * num_heads));
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);
  if (tile_bytes == 2048)
    hipLaunchKernelGGL((tile_read_kernel<128>), grid, dim3(256), 0, st, kc, vc, tables, max_blocks, lens, block_size,
                       work, num_heads, sink);
  else
    hipLaunchKernelGGL((tile_read_kernel<256>), grid, dim3(256), 0, st, kc, vc, tables, max_blocks, lens, block_size,
                       work, num_heads, sink);
  return hipGetLastError();
}

// pkv_attention_decode_noalloc: paged decode attention for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops).
// It runs exactly the kernels of pkv_attention_decode; the workspace those
// kernels need (the decode plan, split-context partials, merge tickets) is a
// file-scope device array instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

namespace {

// The scratch array: PKV_NOALLOC_SCRATCH_BYTES per GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device array: kernels and copies get the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, looked up once per device
// with that device current (each GPU holds its own copy at its own address).
pkv_status scratch_on(int dev, void** out) {
  const char* fn = "pkv_attention_decode_noalloc";
  if (dev < 0 || dev >= kMaxDevices) return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return pkv_failf(PKV_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return pkv_failf(PKV_ERR_HIP, "%s: hipSetDevice(%d): %s", fn, dev, hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr)
      return pkv_failf(PKV_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                       hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_attention_decode_noalloc(float* out, const void* q, const void* k_cache,
                                                   const void* v_cache, const int32_t* block_tables,
                                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                                   int32_t max_context_len, float scale, pkv_dtype dtype,
                                                   void* stream) {
  const char* fn = "pkv_attention_decode_noalloc";
  if (num_seqs <= 0) {
    // nothing to launch: argument checks only
    return pkv_decode_impl(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                           num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, dtype,
                           nullptr, 0, nullptr, 0, true, stream);
  }
  const size_t need = pkv_attention_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len);
  if (need > PKV_NOALLOC_SCRATCH_BYTES)
    return pkv_failf(PKV_ERR_INVALID_ARG,
                     "%s: these sizes need %zu bytes of workspace, more than the %zu-byte scratch array; call "
                     "pkv_attention_decode with a workspace of your own",
                     fn, need, static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES));
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return pkv_failf(PKV_ERR_HIP, "%s: device of the stream: %s", fn, hipGetErrorString(e));
  void* ws = nullptr;
  const pkv_status st = scratch_on(dev, &ws);
  if (st != PKV_OK) return st;
  return pkv_decode_impl(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                         num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, dtype,
                         nullptr, 0, ws, PKV_NOALLOC_SCRATCH_BYTES, true, stream);
}

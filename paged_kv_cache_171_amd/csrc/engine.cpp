// Step executor: the continuous-batching loop run natively.  [UL] "Continuous
// Batching", section "Cómo funciona la planificación a nivel de iteración":
// each iteration the scheduler decides who runs, then one forward step serves
// the admitted prompts and the running requests together.  Here one call per
// step turns the scheduler's decisions into device index arrays and the
// decode plan (built on the host; one host->device copy from pinned staging),
// and one call per layer enqueues that layer's swap copies, cache write,
// prefill and decode.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "pkv_internal.h"

namespace {

// The longest context a table of MB blocks can describe (any supported
// block size; the sizes below are bounds for all of them).
constexpr int32_t kMaxBatchBlock = 32;

// Largest possible index region of one step (every array at its maximum,
// the decode plan included).
size_t meta_bytes(int32_t S, int32_t T, int32_t MB, int32_t NB) {
  using pkv_ws::align256;
  const size_t s = static_cast<size_t>(S), mb = static_cast<size_t>(MB), nb = static_cast<size_t>(NB);
  return align256(static_cast<size_t>(T) * 8) + align256((s + 1) * 4) + align256(s * 4) + align256(s * mb * 4) +
         align256(s * 4) + align256(s * mb * 4) + 2 * align256(nb * 2 * 4) +
         align256(pkv_ws::plan_bytes(S, MB * kMaxBatchBlock));
}

size_t workspace_bytes(int32_t S, int32_t MB, int32_t Hq, int32_t d) {
  return pkv_ws::partial_bytes(S, Hq, d, MB * kMaxBatchBlock);
}

// The decode plan built on the host from the step's lengths: the unit list
// the plan kernel builds (plan_body) -- header (n_units, num_seqs,
// max_context_len, max_blocks_per_seq, partition tokens, block size, 0, 0),
// every full partition in sequence order, the remainders by decreasing size,
// then one (s, -1) unit per sequence with an empty or invalid context.  Units
// of one remainder size keep sequence order (any order gives the same
// results: each unit writes its own partial slot).
void host_plan(int32_t* plan, const int32_t* lens, int32_t S, int32_t MB, int32_t BS, int32_t mcl, int32_t part,
               std::vector<int32_t>& count) {
  int32_t* units = plan + pkv_ws::kPlanHdrWords;
  auto ok = [&](int32_t ctx) {
    return ctx > 0 && ctx <= mcl && static_cast<int64_t>(ctx) <= static_cast<int64_t>(MB) * BS;
  };
  int32_t n = 0;
  count.assign(static_cast<size_t>(part), 0);
  for (int32_t s = 0; s < S; ++s) {
    if (!ok(lens[s])) continue;
    for (int32_t q = 0; q < lens[s] / part; ++q) {
      units[2 * n] = s;
      units[2 * n + 1] = q;
      ++n;
    }
    if (lens[s] % part) ++count[static_cast<size_t>(lens[s] % part)];
  }
  // first slot of each remainder size, largest first
  for (int32_t r = part - 1; r >= 1; --r) {
    const int32_t c = count[static_cast<size_t>(r)];
    count[static_cast<size_t>(r)] = n;
    n += c;
  }
  for (int32_t s = 0; s < S; ++s) {
    if (!ok(lens[s]) || lens[s] % part == 0) continue;
    const int32_t slot = count[static_cast<size_t>(lens[s] % part)]++;
    units[2 * slot] = s;
    units[2 * slot + 1] = lens[s] / part;
  }
  for (int32_t s = 0; s < S; ++s) {
    if (ok(lens[s])) continue;
    units[2 * n] = s;
    units[2 * n + 1] = -1;
    ++n;
  }
  plan[0] = n;
  plan[1] = S;
  plan[2] = mcl;
  plan[3] = MB;
  plan[4] = part;
  plan[5] = BS;
  plan[6] = 0;
  plan[7] = 0;
}

}  // namespace

struct pkv_batch {
  pkv_scheduler* sched = nullptr;
  pkv_allocator* alloc = nullptr;
  int32_t S = 0, T = 0, MB = 0, NB = 0, NH = 0, Hq = 0, Hkv = 0, d = 0, BS = 16;
  pkv_dtype dtype = PKV_BF16;
  char* staging = nullptr;          // two halves of meta bytes, pinned host
  char* dev = nullptr;              // meta (indices and the decode plan) | partials
  size_t meta = 0, ws_cap = 0;
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool ev_used[2] = {false, false};
  int parity = 0;
  // the last step
  pkv_step_info info{};
  int32_t n_tokens = 0, mbp = 0, mbd = 0, mql = 0, mcl_d = 0;
  const int64_t* slots = nullptr;
  const int32_t *pf_qsl = nullptr, *pf_lens = nullptr, *pf_tables = nullptr;
  const int32_t *dc_lens = nullptr, *dc_tables = nullptr, *so_pairs = nullptr, *si_pairs = nullptr;
  const int32_t* dc_plan = nullptr;
  // host scratch of the last step
  std::vector<int64_t> pf_ids, dc_ids, pf_seqs, dc_seqs, slot_v;
  std::vector<int32_t> qsl_v, so_v, si_v, plan_count;
};

extern "C" {

size_t pkv_batch_host_bytes(int32_t max_num_seqs, int32_t max_num_batched_tokens, int32_t max_blocks_per_seq,
                            int32_t num_blocks) {
  if (max_num_seqs <= 0 || max_num_batched_tokens <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0) return 0;
  return 2 * meta_bytes(max_num_seqs, max_num_batched_tokens, max_blocks_per_seq, num_blocks);
}

size_t pkv_batch_device_bytes(int32_t max_num_seqs, int32_t max_num_batched_tokens, int32_t max_blocks_per_seq,
                              int32_t num_blocks, int32_t num_heads, int32_t head_dim) {
  if (max_num_seqs <= 0 || max_num_batched_tokens <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      num_heads <= 0 || head_dim <= 0)
    return 0;
  return meta_bytes(max_num_seqs, max_num_batched_tokens, max_blocks_per_seq, num_blocks) +
         workspace_bytes(max_num_seqs, max_blocks_per_seq, num_heads, head_dim);
}

pkv_status pkv_batch_create(pkv_scheduler* sched, int32_t max_blocks_per_seq, int32_t num_blocks,
                            int32_t num_host_blocks, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            pkv_dtype dtype, void* host_staging, size_t host_bytes, void* device_buffer,
                            size_t device_bytes, pkv_batch** out) {
  const char* fn = "pkv_batch_create";
  if (!sched || !out) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL argument", fn);
  pkv_allocator* alloc = pkv_scheduler_allocator(sched);
  const int32_t bs = pkv_allocator_block_size(alloc);
  if (bs != 8 && bs != 16 && bs != 32)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: the allocator's block size must be 8, 16 or 32", fn);
  if (dtype != PKV_BF16 && dtype != PKV_F32) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (head_dim != 64 && head_dim != 128)
    return pkv_failf(PKV_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128", fn);
  if (num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads != 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: num_heads must be a positive multiple of num_kv_heads", fn);
  if (max_blocks_per_seq <= 0 || num_host_blocks < 0 || num_blocks != pkv_allocator_num_blocks(alloc))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: bad sizes (num_blocks must be the allocator's pool size)", fn);
  const int32_t S = pkv_scheduler_max_num_seqs(sched), T = pkv_scheduler_max_num_batched_tokens(sched);
  const size_t hb = pkv_batch_host_bytes(S, T, max_blocks_per_seq, num_blocks);
  const size_t db = pkv_batch_device_bytes(S, T, max_blocks_per_seq, num_blocks, num_heads, head_dim);
  if (!host_staging || host_bytes < hb)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: host staging of %zu bytes is smaller than the %zu needed", fn,
                     host_bytes, hb);
  if (!device_buffer || device_bytes < db || (reinterpret_cast<uintptr_t>(device_buffer) & 255u))
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: device buffer must hold %zu bytes, 256-byte aligned", fn, db);
  if (reinterpret_cast<uintptr_t>(host_staging) & 255u)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: host staging must be 256-byte aligned", fn);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_staging) != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: host staging must be pinned host memory", fn);
  }
  pkv_batch* b = new (std::nothrow) pkv_batch();
  if (!b) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: out of host memory", fn);
  b->sched = sched;
  b->alloc = alloc;
  b->S = S;
  b->T = T;
  b->MB = max_blocks_per_seq;
  b->NB = num_blocks;
  b->NH = num_host_blocks;
  b->Hq = num_heads;
  b->Hkv = num_kv_heads;
  b->d = head_dim;
  b->BS = bs;
  b->dtype = dtype;
  b->staging = static_cast<char*>(host_staging);
  b->dev = static_cast<char*>(device_buffer);
  b->meta = meta_bytes(S, T, max_blocks_per_seq, num_blocks);
  b->ws_cap = pkv_ws::partial_bytes(S, num_heads, head_dim, max_blocks_per_seq * bs);
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(&b->ev[i], hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      pkv_batch_destroy(b);
      return pkv_failf(PKV_ERR_HIP, "%s: hipEventCreate failed", fn);
    }
  }
  *out = b;
  return PKV_OK;
}

void pkv_batch_destroy(pkv_batch* b) {
  if (!b) return;
  for (int i = 0; i < 2; ++i)
    if (b->ev[i]) {
      if (b->ev_used[i]) (void)hipEventSynchronize(b->ev[i]);
      (void)hipEventDestroy(b->ev[i]);
    }
  delete b;
}

pkv_status pkv_batch_schedule(pkv_batch* b, void* stream, pkv_step_info* info) {
  const char* fn = "pkv_batch_schedule";
  if (!b || !info) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL argument", fn);
  b->n_tokens = 0;
  b->info = pkv_step_info{};
  pkv_status st = pkv_scheduler_step(b->sched, info);
  if (st != PKV_OK) return st;
  b->info = *info;
  const int32_t np = info->num_prefill, nd = info->num_decode;
  const int32_t nso = info->num_swap_out_pairs, nsi = info->num_swap_in_pairs;
  const int32_t T = info->num_prefill_tokens + nd;
  if (T == 0 && nso == 0 && nsi == 0) return PKV_OK;
  b->pf_ids.resize(np);
  b->dc_ids.resize(nd);
  b->qsl_v.resize(np + 1);
  b->slot_v.resize(T);
  b->so_v.resize(2 * static_cast<size_t>(nso));
  b->si_v.resize(2 * static_cast<size_t>(nsi));
  st = pkv_scheduler_step_output(b->sched, nullptr, nullptr, b->so_v.data(), nullptr, b->si_v.data(),
                                 b->pf_ids.data(), b->qsl_v.data(), b->dc_ids.data(), b->slot_v.data());
  if (st != PKV_OK) return st;
  // sequences and lengths of the step's requests
  b->pf_seqs.resize(np);
  b->dc_seqs.resize(nd);
  int32_t mql = 0, mcl_d = 0;
  for (int32_t i = 0; i < np; ++i) {
    int32_t ctx = 0;
    pkv_scheduler_request(b->sched, b->pf_ids[i], nullptr, &b->pf_seqs[i], nullptr, &ctx);
    mql = std::max(mql, ctx);
  }
  for (int32_t i = 0; i < nd; ++i) {
    int32_t ctx = 0;
    pkv_scheduler_request(b->sched, b->dc_ids[i], nullptr, &b->dc_seqs[i], nullptr, &ctx);
    mcl_d = std::max(mcl_d, ctx);
  }
  const int32_t BS = b->BS;
  const int32_t mbp = std::max(1, (mql + BS - 1) / BS);
  const int32_t mbd = std::max(1, (mcl_d + BS - 1) / BS);
  if (mbp > b->MB || mbd > b->MB)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: a block table of %d blocks exceeds max_blocks_per_seq %d", fn,
                     std::max(mbp, mbd), b->MB);
  // the staging half read by the copy two steps ago must be free again
  const int h = b->parity;
  if (b->ev_used[h] && hipEventSynchronize(b->ev[h]) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    return pkv_failf(PKV_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  }
  char* hs = b->staging + static_cast<size_t>(h) * b->meta;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += pkv_ws::align256(bytes); return o; };
  const size_t o_slots = take(static_cast<size_t>(T) * 8);
  const size_t o_qsl = take(static_cast<size_t>(np + 1) * 4);
  const size_t o_pfl = take(static_cast<size_t>(np) * 4);
  const size_t o_pft = take(static_cast<size_t>(np) * mbp * 4);
  const size_t o_dcl = take(static_cast<size_t>(nd) * 4);
  const size_t o_dct = take(static_cast<size_t>(nd) * mbd * 4);
  const size_t o_so = take(static_cast<size_t>(nso) * 8);
  const size_t o_si = take(static_cast<size_t>(nsi) * 8);
  const size_t o_plan = take(nd > 0 ? pkv_ws::plan_bytes(nd, mcl_d) : 0);
  std::memcpy(hs + o_slots, b->slot_v.data(), static_cast<size_t>(T) * 8);
  std::memcpy(hs + o_qsl, b->qsl_v.data(), static_cast<size_t>(np + 1) * 4);
  if (np > 0) {
    st = pkv_block_tables(b->alloc, b->pf_seqs.data(), np, mbp, reinterpret_cast<int32_t*>(hs + o_pft),
                          reinterpret_cast<int32_t*>(hs + o_pfl));
    if (st != PKV_OK) return st;
  }
  if (nd > 0) {
    st = pkv_block_tables(b->alloc, b->dc_seqs.data(), nd, mbd, reinterpret_cast<int32_t*>(hs + o_dct),
                          reinterpret_cast<int32_t*>(hs + o_dcl));
    if (st != PKV_OK) return st;
  }
  std::memcpy(hs + o_so, b->so_v.data(), static_cast<size_t>(nso) * 8);
  std::memcpy(hs + o_si, b->si_v.data(), static_cast<size_t>(nsi) * 8);
  // the decode plan, built here from the lengths just staged: it travels in
  // the same copy, so the step needs no plan kernel
  if (nd > 0)
    host_plan(reinterpret_cast<int32_t*>(hs + o_plan), reinterpret_cast<const int32_t*>(hs + o_dcl), nd, mbd, BS,
              mcl_d, pkv_part_tokens(b->dtype, nd, b->Hq, b->Hkv, BS, mcl_d), b->plan_count);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(b->dev, hs, off, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipEventRecord(b->ev[h], s) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    return pkv_failf(PKV_ERR_HIP, "%s: index copy failed: %s", fn, hipGetErrorString(e));
  }
  b->ev_used[h] = true;
  b->parity ^= 1;
  b->n_tokens = T;
  b->mbp = mbp;
  b->mbd = mbd;
  b->mql = mql;
  b->mcl_d = mcl_d;
  b->slots = reinterpret_cast<const int64_t*>(b->dev + o_slots);
  b->pf_qsl = reinterpret_cast<const int32_t*>(b->dev + o_qsl);
  b->pf_lens = reinterpret_cast<const int32_t*>(b->dev + o_pfl);
  b->pf_tables = reinterpret_cast<const int32_t*>(b->dev + o_pft);
  b->dc_lens = reinterpret_cast<const int32_t*>(b->dev + o_dcl);
  b->dc_tables = reinterpret_cast<const int32_t*>(b->dev + o_dct);
  b->so_pairs = reinterpret_cast<const int32_t*>(b->dev + o_so);
  b->si_pairs = reinterpret_cast<const int32_t*>(b->dev + o_si);
  b->dc_plan = reinterpret_cast<const int32_t*>(b->dev + o_plan);
  return PKV_OK;
}

pkv_status pkv_batch_layer(pkv_batch* b, void* k_cache, void* v_cache, void* k_host, void* v_host, const void* q,
                           const void* k, const void* v, float* out, float scale, void* stream) {
  const char* fn = "pkv_batch_layer";
  if (!b) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL batch", fn);
  const pkv_step_info& in = b->info;
  pkv_status st = PKV_OK;
  if (in.num_swap_out_pairs > 0 || in.num_swap_in_pairs > 0) {
    if (!k_host || !v_host) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: this step swaps but no host pools", fn);
    if (in.num_swap_out_pairs > 0)
      st = pkv_swap_blocks(k_host, v_host, b->NH, k_cache, v_cache, b->NB, b->so_pairs, in.num_swap_out_pairs,
                           b->Hkv, b->d, b->BS, b->dtype, stream);
    if (st == PKV_OK && in.num_swap_in_pairs > 0)
      st = pkv_swap_blocks(k_cache, v_cache, b->NB, k_host, v_host, b->NH, b->si_pairs, in.num_swap_in_pairs,
                           b->Hkv, b->d, b->BS, b->dtype, stream);
    if (st != PKV_OK) return st;
  }
  if (b->n_tokens == 0) return PKV_OK;
  const int32_t npt = in.num_prefill_tokens;
  if (npt > 0) {
    // the prompts' K/V rows; each decode token's row is written by the decode launch
    st = pkv_append(k_cache, v_cache, k, v, b->slots, npt, b->NB, b->Hkv, b->d, b->BS, b->dtype, stream);
    if (st != PKV_OK) return st;
  }
  if (in.num_prefill > 0) {
    st = pkv_attention_prefill_chunk(out, q, b->pf_qsl, npt, b->mql, k_cache, v_cache, b->pf_tables, b->mbp,
                                     b->pf_lens, in.num_prefill, b->Hq, b->Hkv, b->d, b->BS, b->NB, b->mql,
                                     scale, b->dtype, stream);
    if (st != PKV_OK) return st;
  }
  if (in.num_decode > 0) {
    const size_t elem = b->dtype == PKV_BF16 ? 2 : 4;                // bytes of a pool element
    const size_t row = static_cast<size_t>(b->Hq) * b->d;            // q / out elements per token
    const size_t kv_row = static_cast<size_t>(b->Hkv) * b->d * elem;  // bytes of a K or V row
    char* ws = b->dev + b->meta;
    st = pkv_attention_decode_append(out + npt * row, static_cast<const char*>(q) + npt * row * elem,
                                     static_cast<const char*>(k) + npt * kv_row,
                                     static_cast<const char*>(v) + npt * kv_row, b->slots + npt, k_cache, v_cache,
                                     b->dc_tables, b->mbd, b->dc_lens, in.num_decode, b->Hq, b->Hkv, b->d, b->BS,
                                     b->NB, b->mcl_d, scale, b->dtype, b->dc_plan,
                                     pkv_ws::plan_bytes(in.num_decode, b->mcl_d), ws, b->ws_cap, stream);
  }
  return st;
}

}  // extern "C"

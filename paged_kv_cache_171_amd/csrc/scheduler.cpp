// Host scheduler: iteration-level (continuous) batching over the block
// allocator, with swap-out / swap-in of whole sequences under memory pressure.
//
// [UL] "Continuous Batching" (Ultralytics glossary), "Cómo funciona la
// planificación a nivel de iteración": every step the scheduler lets each
// active sequence produce one token, returns the finished ones and frees their
// memory, and admits queued requests if they fit in the KV cache; a new
// request's prefill runs in the same step as the others' decode.  "Límites y
// técnicas complementarias": a step is capped in sequences and tokens
// (max_num_seqs, max_num_batched_tokens).  [CB] "Batching Continuo y
// PagedAttention", "Juntándolo todo: Arquitectura de vLLM": admission needs
// enough free blocks; under memory pressure a low-priority request's blocks are
// copied to CPU memory and freed, and copied back when memory allows.
//
// One step, in this order:
//   1. requests that have produced all their tokens leave (blocks freed);
//   2. running requests, in admission order, take one decode slot each; while
//      the pool is short, the most recently admitted running request is swapped
//      out (whole table to host blocks, taken first in first out); with no host
//      space, that request and the later ones wait this step;
//   3. if nothing was swapped out or stalled, swapped requests come back first
//      in first out: a fresh table (blocks in pool order), one host->device copy
//      per block, then their decode slot;
//   4. queued requests are admitted first in first out (never past a swapped
//      one) while a sequence slot, the token budget and free blocks for the
//      whole prompt allow -- static batching only when nothing runs or waits in
//      host memory -- and their prompts take slots (the prefill);
//   5. every scheduled request counts one more generated token.
// Slots of a step: prefill tokens (admission order), then decode tokens.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <vector>

#include "pkv_internal.h"

namespace {

enum : int32_t { kWaiting = 0, kRunning = 1, kSwapped = 2, kFinished = 3 };

struct Request {
  int32_t prompt = 0;
  int32_t output = 0;
  int32_t generated = 0;
  int32_t state = kWaiting;
  int64_t seq = -1;                    // allocator sequence while running
  int64_t length = 0;                  // cached tokens (kept while swapped)
  std::vector<int32_t> host_table;     // host blocks while swapped
};

}  // namespace

struct pkv_scheduler {
  pkv_allocator* alloc = nullptr;
  int32_t max_num_seqs = 0;
  int32_t max_tokens = 0;
  int32_t policy = PKV_SCHED_CONTINUOUS;
  int32_t num_host_blocks = 0;
  std::vector<Request> req;
  std::deque<int64_t> queue;           // waiting requests
  std::vector<int64_t> running;        // admission order
  std::deque<int64_t> swapped;         // swap-out order
  std::deque<int32_t> host_free;
  int64_t steps = 0, busy = 0;
  // output of the last step
  std::vector<int64_t> finished, swapped_out, swapped_in, prefill, decode, slots;
  std::vector<int32_t> swap_out_pairs, swap_in_pairs, prefill_qsl;

  bool done() const { return queue.empty() && running.empty() && swapped.empty(); }

  int64_t block_size() const { return pkv_allocator_block_size(alloc); }
  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size() - 1) / block_size(); }

  int32_t free_blocks() const { return pkv_allocator_num_free(alloc); }

  // Table of a running request (its length is known here, so the size is too).
  std::vector<int32_t> table_of(const Request& r) const {
    std::vector<int32_t> t(static_cast<size_t>(blocks_for(r.length)));
    int32_t nb = 0, nt = 0;
    pkv_seq_block_table(alloc, r.seq, t.data(), static_cast<int32_t>(t.size()), &nb, &nt);
    t.resize(nb);
    return t;
  }

  bool swap_out(int64_t id) {
    Request& r = req[id];
    const std::vector<int32_t> t = table_of(r);
    if (t.size() > host_free.size()) return false;
    r.host_table.clear();
    for (int32_t b : t) {
      const int32_t h = host_free.front();
      host_free.pop_front();
      r.host_table.push_back(h);
      swap_out_pairs.push_back(b);
      swap_out_pairs.push_back(h);
    }
    pkv_seq_free(alloc, r.seq);
    r.seq = -1;
    r.state = kSwapped;
    swapped.push_back(id);
    running.erase(std::find(running.begin(), running.end(), id));
    swapped_out.push_back(id);
    return true;
  }

  // One slot for request r (its decode token); the caller checked the blocks.
  void take_decode_slot(Request& r, int64_t id) {
    int64_t slot = 0;
    int32_t cow[2], n_cow = 0;
    pkv_seq_append_slots(alloc, r.seq, 1, &slot, cow, &n_cow);
    r.length += 1;
    slots.push_back(slot);
    decode.push_back(id);
  }

  int32_t decode_blocks(const Request& r) const {
    int32_t need = 0;
    pkv_seq_blocks_needed(alloc, r.seq, 1, &need);
    return need;
  }

  pkv_status step(pkv_step_info* info) {
    finished.clear(); swapped_out.clear(); swapped_in.clear(); prefill.clear(); decode.clear();
    slots.clear(); swap_out_pairs.clear(); swap_in_pairs.clear(); prefill_qsl.assign(1, 0);
    std::vector<int64_t> decode_slots;

    // 1. finished requests leave
    for (size_t i = 0; i < running.size();) {
      Request& r = req[running[i]];
      if (r.generated == r.output) {
        pkv_seq_free(alloc, r.seq);
        r.seq = -1;
        r.state = kFinished;
        finished.push_back(running[i]);
        running.erase(running.begin() + static_cast<std::ptrdiff_t>(i));
      } else {
        ++i;
      }
    }
    int64_t budget = max_tokens;
    bool stalled = false;
    if (!done()) {
      // 2. decode slots of running requests, swapping out from the back
      for (size_t i = 0; i < running.size();) {
        const int64_t id = running[i];
        Request& r = req[id];
        while (decode_blocks(r) > free_blocks()) {
          if (!swap_out(running.back())) {
            stalled = true;
            break;
          }
          if (r.state == kSwapped) break;
        }
        if (stalled || r.state != kRunning) break;
        take_decode_slot(r, id);
        budget -= 1;
        ++i;
      }
      // 3. swapped requests return
      if (swapped_out.empty() && !stalled) {
        while (!swapped.empty() && static_cast<int32_t>(running.size()) < max_num_seqs && budget >= 1) {
          const int64_t id = swapped.front();
          Request& r = req[id];
          const int64_t need = blocks_for(r.length) + (r.length % block_size() == 0 ? 1 : 0);
          if (need > free_blocks()) break;
          swapped.pop_front();
          pkv_seq_create(alloc, &r.seq);
          std::vector<int64_t> tmp(static_cast<size_t>(r.length));
          int32_t cow[2], n_cow = 0;
          pkv_seq_append_slots(alloc, r.seq, static_cast<int32_t>(r.length), tmp.data(), cow, &n_cow);
          const std::vector<int32_t> t = table_of(r);
          for (size_t k = 0; k < t.size(); ++k) {
            swap_in_pairs.push_back(r.host_table[k]);
            swap_in_pairs.push_back(t[k]);
            host_free.push_back(r.host_table[k]);
          }
          r.host_table.clear();
          r.state = kRunning;
          running.push_back(id);
          swapped_in.push_back(id);
          take_decode_slot(r, id);
          budget -= 1;
        }
      }
      decode_slots.swap(slots);
      // 4. admission and prefill of queued requests
      const bool may_admit =
          !stalled && (policy == PKV_SCHED_CONTINUOUS || (running.empty() && swapped.empty()));
      while (may_admit && !queue.empty() && swapped.empty() &&
             static_cast<int32_t>(running.size()) < max_num_seqs) {
        const int64_t id = queue.front();
        Request& r = req[id];
        if (r.prompt > budget || blocks_for(r.prompt) > free_blocks()) break;
        queue.pop_front();
        pkv_seq_create(alloc, &r.seq);
        const size_t at = slots.size();
        slots.resize(at + static_cast<size_t>(r.prompt));
        int32_t cow[2], n_cow = 0;
        pkv_seq_append_slots(alloc, r.seq, r.prompt, slots.data() + at, cow, &n_cow);
        r.length = r.prompt;
        r.state = kRunning;
        running.push_back(id);
        prefill.push_back(id);
        prefill_qsl.push_back(prefill_qsl.back() + r.prompt);
        budget -= r.prompt;
      }
      slots.insert(slots.end(), decode_slots.begin(), decode_slots.end());
    }
    // 5. one token for every scheduled request
    for (int64_t id : prefill) req[id].generated += 1;
    for (int64_t id : decode) req[id].generated += 1;
    const int64_t n = static_cast<int64_t>(prefill.size() + decode.size());
    if (n > 0) {
      steps += 1;
      busy += n;
    }
    info->num_finished = static_cast<int32_t>(finished.size());
    info->num_swapped_out = static_cast<int32_t>(swapped_out.size());
    info->num_swap_out_pairs = static_cast<int32_t>(swap_out_pairs.size() / 2);
    info->num_swapped_in = static_cast<int32_t>(swapped_in.size());
    info->num_swap_in_pairs = static_cast<int32_t>(swap_in_pairs.size() / 2);
    info->num_prefill = static_cast<int32_t>(prefill.size());
    info->num_prefill_tokens = prefill_qsl.back();
    info->num_decode = static_cast<int32_t>(decode.size());
    if (n == 0 && !done())
      return pkv_fail(PKV_ERR_OUT_OF_BLOCKS, "pkv_scheduler_step: no request can run (host swap space exhausted)");
    return PKV_OK;
  }
};

extern "C" {

pkv_status pkv_scheduler_create(pkv_allocator* alloc, int32_t max_num_seqs, int32_t max_num_batched_tokens,
                                pkv_sched_policy policy, int32_t num_host_blocks, pkv_scheduler** out) {
  const char* fn = "pkv_scheduler_create";
  if (!alloc || !out) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL argument", fn);
  if (max_num_seqs <= 0 || max_num_batched_tokens <= 0 || num_host_blocks < 0)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
  if (policy != PKV_SCHED_CONTINUOUS && policy != PKV_SCHED_STATIC)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: unknown policy %d", fn, static_cast<int>(policy));
  pkv_scheduler* s = new (std::nothrow) pkv_scheduler();
  if (!s) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: out of host memory", fn);
  s->alloc = alloc;
  s->max_num_seqs = max_num_seqs;
  s->max_tokens = max_num_batched_tokens;
  s->policy = policy;
  s->num_host_blocks = num_host_blocks;
  for (int32_t h = 0; h < num_host_blocks; ++h) s->host_free.push_back(h);
  *out = s;
  return PKV_OK;
}

void pkv_scheduler_destroy(pkv_scheduler* s) { delete s; }

pkv_status pkv_scheduler_add_request(pkv_scheduler* s, int32_t prompt_len, int32_t output_len,
                                     int64_t* request_id) {
  const char* fn = "pkv_scheduler_add_request";
  if (!s || !request_id) return pkv_failf(PKV_ERR_INVALID_ARG, "%s: NULL argument", fn);
  if (prompt_len < 1 || output_len < 1 || prompt_len > s->max_tokens)
    return pkv_failf(PKV_ERR_INVALID_ARG, "%s: prompt must be in [1, %d] and output >= 1", fn, s->max_tokens);
  if (s->blocks_for(static_cast<int64_t>(prompt_len) + output_len) > pkv_allocator_num_blocks(s->alloc))
    return pkv_failf(PKV_ERR_OUT_OF_BLOCKS, "%s: the request would not fit the pool even alone", fn);
  Request r;
  r.prompt = prompt_len;
  r.output = output_len;
  s->req.push_back(r);
  *request_id = static_cast<int64_t>(s->req.size()) - 1;
  s->queue.push_back(*request_id);
  return PKV_OK;
}

pkv_status pkv_scheduler_step(pkv_scheduler* s, pkv_step_info* info) {
  if (!s || !info) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_scheduler_step: NULL argument");
  return s->step(info);
}

pkv_status pkv_scheduler_step_output(const pkv_scheduler* s, int64_t* finished, int64_t* swapped_out,
                                     int32_t* swap_out_pairs, int64_t* swapped_in, int32_t* swap_in_pairs,
                                     int64_t* prefill, int32_t* prefill_query_start_loc, int64_t* decode,
                                     int64_t* slot_mapping) {
  if (!s) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_scheduler_step_output: NULL scheduler");
  auto put64 = [](int64_t* dst, const std::vector<int64_t>& v) { if (dst) std::copy(v.begin(), v.end(), dst); };
  auto put32 = [](int32_t* dst, const std::vector<int32_t>& v) { if (dst) std::copy(v.begin(), v.end(), dst); };
  put64(finished, s->finished);
  put64(swapped_out, s->swapped_out);
  put32(swap_out_pairs, s->swap_out_pairs);
  put64(swapped_in, s->swapped_in);
  put32(swap_in_pairs, s->swap_in_pairs);
  put64(prefill, s->prefill);
  put32(prefill_query_start_loc, s->prefill_qsl);
  put64(decode, s->decode);
  put64(slot_mapping, s->slots);
  return PKV_OK;
}

pkv_status pkv_scheduler_request(const pkv_scheduler* s, int64_t request_id, int32_t* state, int64_t* seq_id,
                                 int32_t* generated, int32_t* context_len) {
  if (!s) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_scheduler_request: NULL scheduler");
  if (request_id < 0 || request_id >= static_cast<int64_t>(s->req.size()))
    return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_scheduler_request: unknown request");
  const Request& r = s->req[request_id];
  if (state) *state = r.state;
  if (seq_id) *seq_id = r.seq;
  if (generated) *generated = r.generated;
  if (context_len) *context_len = static_cast<int32_t>(r.length);
  return PKV_OK;
}

pkv_allocator* pkv_scheduler_allocator(const pkv_scheduler* s) { return s ? s->alloc : nullptr; }
int32_t pkv_scheduler_max_num_seqs(const pkv_scheduler* s) { return s ? s->max_num_seqs : 0; }
int32_t pkv_scheduler_max_num_batched_tokens(const pkv_scheduler* s) { return s ? s->max_tokens : 0; }

pkv_status pkv_scheduler_stats(const pkv_scheduler* s, int64_t* steps, int64_t* busy_slot_steps,
                               int32_t* num_waiting, int32_t* num_running, int32_t* num_swapped) {
  if (!s) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_scheduler_stats: NULL scheduler");
  if (steps) *steps = s->steps;
  if (busy_slot_steps) *busy_slot_steps = s->busy;
  if (num_waiting) *num_waiting = static_cast<int32_t>(s->queue.size());
  if (num_running) *num_running = static_cast<int32_t>(s->running.size());
  if (num_swapped) *num_swapped = static_cast<int32_t>(s->swapped.size());
  return PKV_OK;
}

}  // extern "C"

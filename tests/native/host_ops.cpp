// Random operation sequences on the host block allocator and the
// continuous-batching scheduler, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py compiles and runs
// it).  After every operation the pool invariants are checked: every table
// entry is a pool block, free + distinct blocks in use = pool size, and each
// block's refcount equals the number of tables that hold it.
//
//   usage: host_ops <seed> <rounds>
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "../../include/pkv.h"

// The library's error reporters live with the HIP runtime code in the full
// build; these keep the status and drop the text.
pkv_status pkv_fail(pkv_status st, const char*) { return st; }
pkv_status pkv_failf(pkv_status st, const char*, ...) { return st; }

#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #c); \
      std::exit(1);                                                       \
    }                                                                     \
  } while (0)

static void check_pool(const pkv_allocator* a, const std::vector<int64_t>& live, int32_t nb, int32_t bs) {
  std::map<int32_t, int32_t> uses;
  std::vector<int32_t> t(8192);
  for (int64_t s : live) {
    int32_t n = -1, len = -1;
    CHECK(pkv_seq_block_table(a, s, t.data(), static_cast<int32_t>(t.size()), &n, &len) == PKV_OK);
    CHECK(n == (len + bs - 1) / bs);
    for (int32_t i = 0; i < n; ++i) {
      CHECK(t[i] >= 0 && t[i] < nb);
      ++uses[t[i]];
    }
  }
  CHECK(pkv_allocator_num_free(a) + static_cast<int32_t>(uses.size()) == nb);
  for (const auto& bu : uses) {
    int32_t rc = -1;
    CHECK(pkv_block_refcount(a, bu.first, &rc) == PKV_OK);
    CHECK(rc == bu.second);
  }
}

static void allocator_round(std::mt19937& rng) {
  const int32_t nb = 8 + static_cast<int32_t>(rng() % 57);
  const int32_t sizes[3] = {8, 16, 32};
  const int32_t bs = sizes[rng() % 3];
  std::vector<int32_t> order(nb);
  for (int32_t i = 0; i < nb; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_allocator* a = nullptr;
  CHECK(pkv_allocator_create(nb, bs, (rng() & 1) ? order.data() : nullptr, &a) == PKV_OK);
  CHECK(pkv_allocator_num_blocks(a) == nb && pkv_allocator_block_size(a) == bs);
  std::vector<int64_t> live;
  std::vector<int64_t> slots(4096);
  std::vector<int32_t> cow(2 * 64);
  for (int op = 0; op < 300; ++op) {
    const uint32_t r = rng() % 12;
    if (r < 2 || live.empty()) {
      int64_t s = -1;
      CHECK(pkv_seq_create(a, &s) == PKV_OK);
      live.push_back(s);
    } else if (r < 6) {
      const int64_t s = live[rng() % live.size()];
      const int32_t n = static_cast<int32_t>(rng() % 48);
      int32_t ncow = -1, need = -1;
      CHECK(pkv_seq_blocks_needed(a, s, n, &need) == PKV_OK);
      const int32_t free_before = pkv_allocator_num_free(a);
      const pkv_status st = pkv_seq_append_slots(a, s, n, slots.data(), cow.data(), &ncow);
      // granted exactly when the blocks it needs are free; a refusal changes nothing
      CHECK(st == (need <= free_before ? PKV_OK : PKV_ERR_OUT_OF_BLOCKS));
      if (st != PKV_OK) CHECK(pkv_allocator_num_free(a) == free_before);
      if (st == PKV_OK) {
        CHECK(ncow == 0 || ncow == 1);
        for (int32_t i = 0; i < n; ++i) CHECK(slots[i] >= 0 && slots[i] < static_cast<int64_t>(nb) * bs);
      }
    } else if (r < 7) {
      // one batched reservation over up to four live sequences
      const int32_t count = 1 + static_cast<int32_t>(rng() % (live.size() < 4 ? live.size() : 4));
      std::vector<int64_t> seqs(count);
      std::vector<int32_t> ns(count);
      int32_t total = 0;
      for (int32_t i = 0; i < count; ++i) {
        seqs[i] = live[(rng() % live.size())];
        ns[i] = static_cast<int32_t>(rng() % 20);
        total += ns[i];
      }
      int32_t ncow = -1;
      const pkv_status st =
          pkv_seq_append_slots_batch(a, seqs.data(), ns.data(), count, slots.data(), cow.data(), &ncow);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_INVALID_ARG);
      if (st == PKV_OK)
        for (int32_t i = 0; i < total; ++i) CHECK(slots[i] >= 0 && slots[i] < static_cast<int64_t>(nb) * bs);
    } else if (r < 9) {
      int64_t c = -1;
      CHECK(pkv_seq_fork(a, live[rng() % live.size()], &c) == PKV_OK);
      live.push_back(c);
    } else if (r < 11) {
      const size_t i = rng() % live.size();
      CHECK(pkv_seq_free(a, live[i]) == PKV_OK);
      live.erase(live.begin() + static_cast<long>(i));
    } else {
      // invalid arguments are refused without changing anything
      int32_t n = 0, len = 0, rc = 0, ncow = 0;
      CHECK(pkv_seq_free(a, -5) == PKV_ERR_UNKNOWN_SEQ);
      CHECK(pkv_seq_append_slots(a, 1 << 30, 1, slots.data(), cow.data(), &ncow) == PKV_ERR_UNKNOWN_SEQ);
      CHECK(pkv_block_refcount(a, nb, &rc) == PKV_ERR_INVALID_ARG);
      CHECK(pkv_block_refcount(a, -1, &rc) == PKV_ERR_INVALID_ARG);
      CHECK(pkv_seq_block_table(a, live[0], nullptr, -1, &n, &len) == PKV_ERR_INVALID_ARG);
    }
    check_pool(a, live, nb, bs);
  }
  for (int64_t s : live) CHECK(pkv_seq_free(a, s) == PKV_OK);
  CHECK(pkv_allocator_num_free(a) == nb);
  pkv_allocator_destroy(a);
}

static int64_t scheduler_round(std::mt19937& rng) {
  const int32_t nb = 6 + static_cast<int32_t>(rng() % 43);
  const int32_t sizes[3] = {8, 16, 32};
  const int32_t bs = sizes[rng() % 3];
  const int32_t tokens = 24 + static_cast<int32_t>(rng() % 137);
  pkv_allocator* a = nullptr;
  CHECK(pkv_allocator_create(nb, bs, nullptr, &a) == PKV_OK);
  pkv_scheduler* s = nullptr;
  const pkv_sched_policy policy = (rng() & 1) ? PKV_SCHED_STATIC : PKV_SCHED_CONTINUOUS;
  const int32_t host_blocks = (rng() % 4 == 0) ? 0 : 4 * nb;
  CHECK(pkv_scheduler_create(a, 1 + static_cast<int32_t>(rng() % 9), tokens, policy, host_blocks, &s) == PKV_OK);
  const int32_t nreq = 1 + static_cast<int32_t>(rng() % 16);
  for (int32_t i = 0; i < nreq; ++i) {
    const int32_t p = 1 + static_cast<int32_t>(rng() % (tokens < 70 ? tokens : 70));
    const int32_t o = 1 + static_cast<int32_t>(rng() % 90);
    int64_t id = -1;
    const pkv_status st = pkv_scheduler_add_request(s, p, o, &id);
    CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
  }
  int64_t bad_id = 0;
  CHECK(pkv_scheduler_add_request(s, 0, 1, &bad_id) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_scheduler_add_request(s, tokens + 1, 1, &bad_id) == PKV_ERR_INVALID_ARG);
  for (int step = 0; step < 20000; ++step) {
    pkv_step_info info{};
    const pkv_status st = pkv_scheduler_step(s, &info);
    if (st == PKV_ERR_OUT_OF_BLOCKS) break;       // no host space to swap into: the step is refused
    CHECK(st == PKV_OK);
    std::vector<int64_t> fin(info.num_finished + 1), sout(info.num_swapped_out + 1), sin(info.num_swapped_in + 1);
    std::vector<int32_t> sop(2 * info.num_swap_out_pairs + 2), sip(2 * info.num_swap_in_pairs + 2);
    std::vector<int64_t> pre(info.num_prefill + 1), dec(info.num_decode + 1);
    std::vector<int32_t> qsl(info.num_prefill + 2);
    std::vector<int64_t> slot(info.num_prefill_tokens + info.num_decode + 1);
    CHECK(pkv_scheduler_step_output(s, fin.data(), sout.data(), sop.data(), sin.data(), sip.data(), pre.data(),
                                    qsl.data(), dec.data(), slot.data()) == PKV_OK);
    CHECK(info.num_prefill_tokens + info.num_decode <= tokens);
    if (info.num_prefill > 0) {
      CHECK(qsl[0] == 0 && qsl[info.num_prefill] == info.num_prefill_tokens);
      for (int32_t i = 0; i < info.num_prefill; ++i) CHECK(qsl[i + 1] > qsl[i]);
    }
    for (int32_t i = 0; i < info.num_prefill_tokens + info.num_decode; ++i)
      CHECK(slot[i] >= 0 && slot[i] < static_cast<int64_t>(nb) * bs);
    for (int32_t i = 0; i < info.num_swap_out_pairs; ++i)
      CHECK(sop[2 * i] >= 0 && sop[2 * i] < nb && sop[2 * i + 1] >= 0 && sop[2 * i + 1] < host_blocks);
    for (int32_t i = 0; i < info.num_swap_in_pairs; ++i)
      CHECK(sip[2 * i] >= 0 && sip[2 * i] < host_blocks && sip[2 * i + 1] >= 0 && sip[2 * i + 1] < nb);
    if (info.num_prefill == 0 && info.num_decode == 0 && info.num_swapped_in == 0) break;
  }
  int64_t steps = 0, busy = 0;
  int32_t waiting = 0, running = 0, swapped = 0;
  CHECK(pkv_scheduler_stats(s, &steps, &busy, &waiting, &running, &swapped) == PKV_OK);
  CHECK(steps >= 0 && busy >= 0 && waiting >= 0 && running >= 0 && swapped >= 0);
  pkv_scheduler_destroy(s);
  pkv_allocator_destroy(a);
  return steps;
}

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? static_cast<unsigned>(std::strtoul(argv[1], nullptr, 10)) : 1u;
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 50;
  std::mt19937 rng(seed);
  int64_t steps = 0;
  for (int i = 0; i < rounds; ++i) {
    allocator_round(rng);
    steps += scheduler_round(rng);
  }
  std::printf("ok %d rounds, %lld scheduler steps\n", rounds, static_cast<long long>(steps));
  return 0;
}

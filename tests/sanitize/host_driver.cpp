// Host-side driver for the sanitizer build of the library's front end
// (built by tests/test_host_sanitizers.py with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code).  It exercises every path that
// runs on the CPU: the FIFO pool, argument validation of the compression
// entry points (which must reject before touching any device pointer), the
// host plan, the periodic schedule and the serving-policy simulator.  Device
// pointers passed here are never valid; a path that dereferenced one would
// crash.  Exits 0 when every check holds.

#include "../../include/kara.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

static int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static void* fake(size_t k) { return (void*)(uintptr_t)(0x1000 * k); }

int main() {
  // ---- pool ----
  std::vector<int32_t> ids = {5, 3, 9, 0, 7};
  kara_pool* pool = nullptr;
  CHECK(kara_pool_create(10, ids.data(), (int32_t)ids.size(), &pool) == KARA_OK);
  int32_t got[8];
  CHECK(kara_pool_alloc(pool, 2, got) == KARA_OK && got[0] == 5 && got[1] == 3);
  CHECK(kara_pool_alloc(pool, 9, got) == KARA_E_NOBLOCKS);
  CHECK(kara_pool_free(pool, got, 2) == KARA_OK);
  const int32_t dup[2] = {4, 4};
  CHECK(kara_pool_free(pool, dup, 2) == KARA_E_INVAL);
  const int32_t out_of_range[1] = {10};
  CHECK(kara_pool_free(pool, out_of_range, 1) == KARA_E_INVAL);
  CHECK(kara_pool_num_free(pool) == 5);
  int32_t snap[8];
  CHECK(kara_pool_snapshot(pool, snap, 8) == 5 && snap[0] == 9 && snap[3] == 5 && snap[4] == 3);
  CHECK(kara_pool_snapshot(pool, snap, 2) == 2);
  kara_pool* bad = nullptr;
  const int32_t rep[2] = {1, 1};
  CHECK(kara_pool_create(4, rep, 2, &bad) == KARA_E_INVAL && bad == nullptr);

  // ---- compression entry points: validation before any side effect ----
  kara_shape sh = {2, 8, 2, 128, 4, KARA_BF16};
  kara_params pr = {8, 2, 2, 3, 0};
  const int32_t lens[2] = {10, 13};
  std::vector<int32_t> table = {0, 1, 2, -1, -1, 3, 4, 5, 6, -1};
  std::vector<int32_t> free_ids;
  for (int i = 7; i < 20; ++i) free_ids.push_back(i);
  kara_pool* p2 = nullptr;
  CHECK(kara_pool_create(20, free_ids.data(), (int32_t)free_ids.size(), &p2) == KARA_OK);
  std::vector<int32_t> new_table(10, 0), new_lens(2, 0);
  const size_t ws = kara_workspace_bytes(&sh, &pr, 2);
  CHECK(ws > 0);
  kara_params bad_pr = pr;
  bad_pr.top_k = 7;
  CHECK(kara_compress(&sh, &bad_pr, 2, fake(1), fake(2), 20, table.data(), (int32_t*)fake(3), 5, lens,
                      (int32_t*)fake(4), p2, new_table.data(), (int32_t*)fake(5), new_lens.data(), fake(6), ws,
                      nullptr, nullptr, nullptr, nullptr, nullptr) == KARA_E_INVAL);
  CHECK(kara_compress(&sh, &pr, 2, fake(1), fake(2), 20, table.data(), (int32_t*)fake(3), 5, lens,
                      (int32_t*)fake(4), p2, new_table.data(), (int32_t*)fake(5), new_lens.data(), fake(6), 0,
                      nullptr, nullptr, nullptr, nullptr, nullptr) == KARA_E_WORKSPACE);
  std::vector<int32_t> dup_table = {0, 1, 2, -1, -1, 3, 4, 2, 6, -1};
  CHECK(kara_compress(&sh, &pr, 2, fake(1), fake(2), 20, dup_table.data(), (int32_t*)fake(3), 5, lens,
                      (int32_t*)fake(4), p2, new_table.data(), (int32_t*)fake(5), new_lens.data(), fake(6), ws,
                      nullptr, nullptr, nullptr, nullptr, nullptr) == KARA_E_INVAL);
  kara_pool* p3 = nullptr;
  const int32_t one_free[1] = {7};
  CHECK(kara_pool_create(20, one_free, 1, &p3) == KARA_OK);
  CHECK(kara_compress(&sh, &pr, 2, fake(1), fake(2), 20, table.data(), (int32_t*)fake(3), 5, lens,
                      (int32_t*)fake(4), p3, new_table.data(), (int32_t*)fake(5), new_lens.data(), fake(6), ws,
                      nullptr, nullptr, nullptr, nullptr, nullptr) == KARA_E_NOBLOCKS);
  CHECK(kara_pool_num_free(p3) == 1 && new_lens[0] == 0 && new_lens[1] == 0);
  CHECK(kara_compress(&sh, &pr, 0, nullptr, nullptr, 20, nullptr, nullptr, 5, nullptr, nullptr, p2, nullptr,
                      nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr) == KARA_OK);
  int n = 1;
  while (kara_workspace_bytes(&sh, &pr, n) <= kara_static_scratch_bytes()) n *= 2;
  CHECK(kara_compress_static(&sh, &pr, n, fake(1), fake(2), 20, (int32_t*)fake(7), (int32_t*)fake(3), 5,
                             (int32_t*)fake(8), (int32_t*)fake(4), p2, (int32_t*)fake(9), (int32_t*)fake(5),
                             (int32_t*)fake(10), nullptr, nullptr, nullptr, nullptr, nullptr) == KARA_E_WORKSPACE);
  CHECK(kara_pool_num_free(p2) == (int32_t)free_ids.size());
  kara_query_ring ring = {fake(11), 2, 16, (int32_t*)fake(12), (int32_t*)fake(13)};
  CHECK(kara_append(&sh, 8, 1, 0, fake(1), fake(2), fake(3), fake(4), 20, (int32_t*)fake(5), 5,
                    (int32_t*)fake(6), &ring, nullptr) == KARA_E_INVAL);
  CHECK(kara_topk(4, 10, 11, (float*)fake(1), (int32_t*)fake(2), nullptr) == KARA_E_INVAL);
  CHECK(kara_token2chunk(4, 10, 3, 11, (float*)fake(1), (int32_t*)fake(2), (int32_t*)fake(3), nullptr) ==
        KARA_E_INVAL);

  // ---- host plan and schedule ----
  int32_t nl[2], fr[2];
  const int32_t plan_lens[2] = {1000, 1031};
  kara_params pp = {1024, 128, 64, 179, 0};
  CHECK(kara_plan_lengths(&pp, 16, 2, plan_lens, nl, fr) == KARA_E_INVAL);
  const int32_t plan_lens2[2] = {1024, 1031};
  CHECK(kara_plan_lengths(&pp, 16, 2, plan_lens2, nl, fr) == KARA_OK);
  CHECK(nl[0] == 1024 - 896 + 179 && fr[0] == (179 + 128 + 15) / 16 && fr[1] == (7 + 179 + 128 + 15) / 16);
  const int32_t sl[4] = {3000, 5000, 900, 2048};
  const int32_t wm[4] = {0, 4500, 0, 0};
  const uint8_t sel[4] = {1, 1, 1, 0};
  int32_t batch[4], nb = -1;
  CHECK(kara_schedule_step(256, 128, 1024, 4, sl, wm, sel, batch, &nb) == KARA_OK && nb == 1 && batch[0] == 0);
  CHECK(kara_schedule_step(200, 128, 1024, 4, sl, wm, sel, batch, &nb) == KARA_OK && nb == 0);

  // ---- serving-policy simulator ----
  for (int policy = 0; policy < 3; ++policy) {
    kara_sim_config cfg = {};
    cfg.policy = policy;
    cfg.n_requests = 24;
    cfg.max_batch = 8;
    cfg.cap_blocks = 1500;
    cfg.block_size = 16;
    cfg.prompt_len = 256;
    cfg.gen_min = 600;
    cfg.gen_max = 2000;
    cfg.seed = 5;
    cfg.window = 256;
    cfg.protect = 32;
    cfg.budget = 44;
    cfg.period = 64;
    cfg.threshold = 1024;
    cfg.keep = 512;
    cfg.decode_ms_fixed = 2.0;
    cfg.decode_ms_per_token = 1e-4;
    cfg.compress_ms_per_seq = 0.5;
    cfg.compress_ms_per_key = 1e-3;
    cfg.max_steps = 200000;
    kara_sim_result res = {};
    std::vector<int32_t> active(cfg.max_steps), comps(cfg.max_steps);
    std::vector<double> ms(cfg.max_steps);
    CHECK(kara_policy_sim(&cfg, &res, active.data(), comps.data(), ms.data()) == KARA_OK);
    CHECK(res.finished == cfg.n_requests && res.tokens > 0 && res.steps > 0);
  }

  kara_pool_destroy(pool);
  kara_pool_destroy(p2);
  kara_pool_destroy(p3);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host sanitizer driver: all checks passed\n");
  return 0;
}

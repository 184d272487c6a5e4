// Host-side checks of libvc under AddressSanitizer and UndefinedBehaviorSanitizer (built and run
// on the CPU by tests/test_host_sanitize.py; the library's sources are compiled host-only).
//
// Everything driven here runs on the host before any HIP call: the page allocator and the Admit
// scheduler (host code by nature, exercised with random operation sequences against simple
// models), and the attention calls' validation and launch planning (request checks, split
// planning, the request table and workspace sizing).  A planned launch with a workspace that is
// too small returns VC_ENOSPACE after planning and before any device call, which is how the
// planner is reached without a GPU.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <set>
#include <vector>

#include "vc.h"

static int g_fail = 0;
#define CHECK(c)                                                                 \
  do {                                                                           \
    if (!(c)) {                                                                  \
      fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #c);  \
      ++g_fail;                                                                  \
      return;                                                                    \
    }                                                                            \
  } while (0)

// ---------------------------------------------------------------- page allocator vs a model
static void test_allocator(uint32_t seed) {
  std::mt19937 rng(seed);
  const int nb = 1 + (int)(rng() % 300), nres = (int)(rng() % (nb + 1));
  void* a = nullptr;
  CHECK(vc_alloc_create(nb, nres, &a) == VC_OK && a);
  std::set<int32_t> held[2];
  for (int step = 0; step < 2000; ++step) {
    const int kind = (int)(rng() % 2);
    const int cap = kind == VC_PAGE_RESIDENT ? nres : nb - nres;
    const int op = (int)(rng() % 4);
    if (op == 0) {  // take n
      const int n = (int)(rng() % 9);
      std::vector<int32_t> ids(std::max(1, n), -7);
      const int rc = vc_alloc_pages(a, kind, n, ids.data());
      if ((int)held[kind].size() + n <= cap) {
        CHECK(rc == VC_OK);
        for (int i = 0; i < n; ++i) {
          CHECK(ids[i] >= (kind ? nres : 0) && ids[i] < (kind ? nb : nres));
          CHECK(held[kind].insert(ids[i]).second);
        }
      } else {
        CHECK(rc == VC_ENOMEM);
      }
    } else if (op == 1 && !held[kind].empty()) {  // give back a random subset
      std::vector<int32_t> v(held[kind].begin(), held[kind].end());
      std::shuffle(v.begin(), v.end(), rng);
      v.resize(1 + rng() % v.size());
      CHECK(vc_alloc_release(a, kind, (int)v.size(), v.data()) == VC_OK);
      for (int32_t id : v) held[kind].erase(id);
    } else if (op == 2) {  // bad releases change nothing
      int32_t bad[3] = {-1, nb, nb + 1000};
      CHECK(vc_alloc_release(a, kind, 1, &bad[rng() % 3]) == VC_EINVAL);
      if (!held[kind].empty()) {
        const int32_t id = *held[kind].begin();
        int32_t twice[2] = {id, id};
        CHECK(vc_alloc_release(a, kind, 2, twice) == VC_EINVAL);
        CHECK(vc_alloc_release(a, 1 - kind, 1, &twice[0]) == VC_EINVAL);
      }
    } else {  // a page-table row grown and shrunk
      const int32_t maxp = 1 + (int)(rng() % 12);
      std::vector<int32_t> row(maxp, -1);
      const int32_t len0 = (int32_t)(rng() % (16 * maxp + 1));
      int rc = vc_page_row_extend(a, kind, row.data(), maxp, 0, len0);
      if (rc == VC_OK) {
        const int pages = (len0 + 15) / 16;
        for (int q = 0; q < pages; ++q) CHECK(held[kind].insert(row[q]).second);
        for (int q = pages; q < maxp; ++q) CHECK(row[q] == -1);
        const int32_t len1 = (int32_t)(rng() % (len0 + 1));
        const std::vector<int32_t> before(row);
        CHECK(vc_page_row_truncate(a, kind, row.data(), maxp, len0, len1) == VC_OK);
        const int keep = (len1 + 15) / 16;
        for (int q = 0; q < keep; ++q) CHECK(row[q] == before[q]);
        for (int q = keep; q < pages; ++q) {  // released: back in the free pool
          CHECK(row[q] == -1);
          held[kind].erase(before[q]);
        }
      } else {
        CHECK(rc == VC_ENOMEM || rc == VC_EINVAL);
      }
    }
    CHECK(vc_alloc_free_count(a, kind) >= 0);
  }
  CHECK(vc_alloc_free_count(a, 5) == -1);
  vc_alloc_destroy(a);
}

// A cleaner row test: every page a row takes is released by its truncation, and the free counts
// come back to where they started.
static void test_rows(uint32_t seed) {
  std::mt19937 rng(seed);
  void* a = nullptr;
  CHECK(vc_alloc_create(64, 32, &a) == VC_OK);
  const int32_t f0 = vc_alloc_free_count(a, VC_PAGE_RESIDENT), f1 = vc_alloc_free_count(a, VC_PAGE_TRANSIENT);
  for (int it = 0; it < 500; ++it) {
    const int kind = (int)(rng() % 2);
    std::vector<int32_t> row(20, -1);
    int32_t len = 0;
    for (int k = 0; k < 6; ++k) {
      const int32_t nl = (int32_t)(rng() % 400);
      int rc;
      if (nl >= len) rc = vc_page_row_extend(a, kind, row.data(), 20, len, nl);
      else rc = vc_page_row_truncate(a, kind, row.data(), 20, len, nl);
      CHECK(rc == VC_OK || rc == VC_ENOMEM || rc == VC_EINVAL);
      if (rc == VC_OK) len = nl;
    }
    CHECK(vc_page_row_truncate(a, kind, row.data(), 20, len, 0) == VC_OK);
    for (int32_t v : row) CHECK(v == -1);
  }
  CHECK(vc_alloc_free_count(a, VC_PAGE_RESIDENT) == f0 && vc_alloc_free_count(a, VC_PAGE_TRANSIENT) == f1);
  vc_alloc_destroy(a);
}

// ---------------------------------------------------------------- Admit scheduler invariants
static void test_scheduler(uint32_t seed) {
  std::mt19937 rng(seed);
  vc_sched_cfg cfg;
  cfg.window = 2 + (int)(rng() % 40);
  cfg.draft_len = 1 + (int)(rng() % 40);
  cfg.t_iter = 0.001 * (1 + rng() % 50);
  cfg.link_bw = 1e9 * (1 + rng() % 60);
  cfg.hbm_budget = 1e9 * (rng() % 40);
  void* s = nullptr;
  CHECK(vc_sched_create(&cfg, &s) == VC_OK && s);
  std::set<int32_t> live;
  for (int step = 0; step < 3000; ++step) {
    const int op = (int)(rng() % 3);
    if (op < 2) {
      const int32_t req = (int32_t)(rng() % 64);
      const double bytes = 1e8 * (1 + rng() % 200);
      int64_t when = -5;
      const int rc = vc_sched_admit(s, req, bytes, &when);
      if (live.count(req)) {
        CHECK(rc == VC_EINVAL);
      } else if (rc == VC_OK) {
        CHECK(when >= vc_sched_now(s) && when < vc_sched_now(s) + cfg.window);
        live.insert(req);
      } else {
        CHECK(rc == VC_EAGAIN && when == -1);
      }
    } else {
      int32_t rl[128], vl[128], nr = -1, nv = -1;
      CHECK(vc_sched_due(s, 128, rl, &nr, vl, &nv) == VC_OK);
      CHECK(nr >= 0 && nv >= 0);
      for (int i = 1; i < nv; ++i) CHECK(vl[i - 1] < vl[i]);
      for (int i = 0; i < nv; ++i) live.erase(vl[i]);
      CHECK(vc_sched_advance(s) == VC_OK);
    }
    for (int i = 0; i < cfg.window; ++i) {
      double link = -1, hbm = -1;
      CHECK(vc_sched_ring(s, i, &link, &hbm) == VC_OK);
      CHECK(link >= -1e-12 && link <= cfg.t_iter * (1 + 1e-9) + 1e-15);
      CHECK(hbm >= -1e-3 && hbm <= cfg.hbm_budget * (1 + 1e-12) + 1e-3);
    }
  }
  double l2, h2;
  CHECK(vc_sched_ring(s, cfg.window, &l2, &h2) == VC_EINVAL);
  vc_sched_destroy(s);
  cfg.window = 1;
  CHECK(vc_sched_create(&cfg, &s) == VC_EINVAL);
}

// ---------------------------------------------------------------- launch planning and validation
static void test_planning(uint32_t seed) {
  std::mt19937 rng(seed);
  static int32_t dummy_table[4];
  char fake_dev[64];
  void* p = fake_dev;
  for (int it = 0; it < 400; ++it) {
    vc_shape s;
    s.num_layers = 1 + (int)(rng() % 8);
    s.num_kv_heads = 1 + (int)(rng() % 8);
    s.num_q_heads = s.num_kv_heads * (1 + (int)(rng() % 16));
    s.head_dim = rng() % 2 ? 128 : 64;
    s.max_rows = 16 * (1 + (int)(rng() % 4));
    const int nreq = (int)(rng() % 1100);
    std::vector<vc_req> reqs(std::max(1, nreq));
    for (int i = 0; i < nreq; ++i) {
      vc_req& r = reqs[i];
      r.slot = (int32_t)(rng() % 64);
      r.kind = rng() % 3 ? VC_VERIFY : VC_DRAFT;
      r.pool = r.kind == VC_VERIFY ? 0 : 1 + (int)(rng() % 2);
      r.ctx_len = (int32_t)(rng() % 3 ? rng() % 20000 : rng() % 17);
      r.page_row = (int32_t)(rng() % 64);
      const int G = s.num_q_heads / s.num_kv_heads;
      if (r.kind == VC_DRAFT) {
        r.rows = 1;
        r.q0 = (int32_t)(rng() % s.max_rows);
      } else {
        r.rows = 1 + (int32_t)(rng() % s.max_rows);
        r.q0 = (int32_t)(rng() % (s.max_rows - r.rows + 1));
      }
      if (r.kind == VC_DRAFT && G > 16) r.kind = VC_VERIFY;
      if (rng() % 50 == 0) r.rows = 0;                   // invalid
      if (rng() % 50 == 0) r.ctx_len = -3;               // invalid
    }
    const int split = rng() % 2 ? 0 : 4 * (int)(rng() % 64);
    const size_t ws = vc_attn_workspace_size(&s, nreq, reqs.data(), split);
    (void)ws;
    vc_pool pools[3];
    for (int k = 0; k < 3; ++k) {
      pools[k].bits = k == 2 ? (rng() % 2 ? 2 : 4) : 16;
      pools[k].max_pages = 1 + 20000 / 16;
      pools[k].num_blocks = 1 + (int64_t)(rng() % 100000);
      pools[k].page_table = dummy_table;
      pools[k].k = p;
      pools[k].v = p;
      pools[k].k_sz = pools[k].bits == 16 ? nullptr : p;
      pools[k].v_sz = pools[k].bits == 16 ? nullptr : p;
    }
    // no workspace: a launch that needs one is planned to the end and then refused; a valid
    // launch that needs none would go on to the device (none here: the HIP call fails), and an
    // invalid one is refused during planning
    if (ws == 0 && nreq <= 64 && split == 0) continue;
    const int rc = vc_attn_mixed(&s, nreq, reqs.data(), p, p, p, 3, pools, (float*)p, nullptr, 0, split, nullptr);
    if (ws > 0) CHECK(rc == VC_ENOSPACE);
    else if (nreq == 0) CHECK(rc == VC_OK);   // nothing to launch
    else {
      if (!(rc == VC_EINVAL || rc == VC_EUNSUPPORTED || rc == VC_EHIP))
        fprintf(stderr, "nreq %d split %d ws %zu: rc %d (%s)\n", nreq, split, ws, rc, vc_last_error());
      CHECK(rc == VC_EINVAL || rc == VC_EUNSUPPORTED || rc == VC_EHIP);
    }
    if (rc == VC_EHIP) CHECK(nreq <= 64);
    CHECK(vc_last_error() != nullptr);
    const int rc2 = vc_attn_mixed_noalloc(&s, nreq, reqs.data(), p, p, p, 3, pools, (float*)p, split, nullptr);
    if (ws > (size_t)VC_SCRATCH_BYTES) CHECK(rc2 == VC_ENOSPACE);
  }
}

static void test_validation() {
  char fake[64];
  void* p = fake;
  vc_shape s = {2, 8, 2, 128, 32};
  vc_req r = {0, 0, 100, 0, 0, 8, VC_VERIFY};
  static int32_t table[4];
  vc_pool pool = {16, 8, 16, table, p, p, nullptr, nullptr};
  CHECK(vc_verify_attn(nullptr, 1, &r, p, p, p, &pool, (float*)p, nullptr, 0, 0, nullptr) == VC_EINVAL);
  CHECK(vc_verify_attn(&s, -1, &r, p, p, p, &pool, (float*)p, nullptr, 0, 0, nullptr) == VC_EINVAL);
  CHECK(vc_verify_attn(&s, 1025, &r, p, p, p, &pool, (float*)p, nullptr, 0, 0, nullptr) == VC_EINVAL);
  CHECK(vc_verify_attn(&s, 1, nullptr, p, p, p, &pool, (float*)p, nullptr, 0, 0, nullptr) == VC_EINVAL);
  CHECK(vc_verify_attn(&s, 1, &r, p, p, p, nullptr, (float*)p, nullptr, 0, 0, nullptr) == VC_EINVAL);
  CHECK(vc_verify_attn(&s, 1, &r, p, p, p, &pool, (float*)p, nullptr, 0, 6, nullptr) == VC_EINVAL);
  CHECK(vc_verify_attn(&s, 1, &r, p, p, p, &pool, (float*)p, nullptr, 0, 4, nullptr) == VC_ENOSPACE);
  vc_shape bad = s;
  bad.head_dim = 96;
  CHECK(vc_verify_attn(&bad, 1, &r, p, p, p, &pool, (float*)p, nullptr, 0, 0, nullptr) == VC_EUNSUPPORTED);
  CHECK(vc_accept(1, 65, 65, 10, (int32_t*)p, (int32_t*)p, (float*)p, (float*)p, (int32_t*)p, (int32_t*)p,
                  (int32_t*)p, (int32_t*)p, nullptr) == VC_EINVAL);
  CHECK(vc_logits(4, 8, 8, (float*)p, 4, p, (float*)p, nullptr) == VC_EINVAL);
  CHECK(vc_stage_kv(nullptr, nullptr, 0, nullptr, nullptr) == VC_OK);
  CHECK(vc_stage_kv(nullptr, p, 16, nullptr, nullptr) == VC_EINVAL);
  int32_t lens[129];
  for (int i = 0; i < 129; ++i) lens[i] = 16;
  CHECK(vc_compress(&s, 129, lens, &pool, nullptr, 0, &pool, nullptr) == VC_EINVAL);
  vc_commit c = {0, 0, 1, 0, 0};
  CHECK(vc_commit_rows(&s, 129, &c, p, p, &pool, nullptr, 0, nullptr) == VC_EINVAL);
  CHECK(strlen(vc_last_error()) > 0);
  CHECK(strncmp(vc_version(), "vc ", 3) == 0);
}

int main() {
  for (uint32_t seed = 1; seed <= 40; ++seed) {
    test_allocator(seed);
    test_rows(seed);
    test_scheduler(seed);
  }
  for (uint32_t seed = 1; seed <= 20; ++seed) test_planning(seed);
  test_validation();
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("host sanitize checks passed\n");
  return 0;
}

// Randomized exercise of the library's host-only logic (page pool, planner, residency
// manager, admission scheduler, argument validation), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitize.py. No GPU is touched: pools are
// created over a placeholder device address and no compute call gets past validation.
// Invariants are checked as it goes; any violation or sanitizer report fails the run.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "slora.h"

static int g_fail = 0;
static int64_t g_plans = 0, g_groups = 0, g_tokens = 0, g_fetches = 0;  // coverage counts
#define CHECK(c)                                                             \
  do {                                                                       \
    if (!(c)) {                                                              \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

static void* const kFakeDev = reinterpret_cast<void*>(0x7F0000000000ull);

// Page pool: random adapter / KV allocations and frees; free + owned pages = all pages.
static void pool_round(std::mt19937_64& rng) {
  const int64_t n_pages = 64 + (int64_t)(rng() % 400);
  const int32_t P = 8 * (1 + (int32_t)(rng() % 64));
  slora_pool* pool = nullptr;
  const bool ordered = rng() & 1;
  int rc = ordered ? slora_pool_create_ordered(kFakeDev, n_pages, P, SLORA_BF16, &pool)
                   : slora_pool_create(kFakeDev, n_pages, P, SLORA_F16, rng(), &pool);
  CHECK(rc == SLORA_OK && pool);
  std::map<int32_t, std::vector<int32_t>> dims;  // adapter -> {n_proj, rank, d_in..., d_out...}
  std::vector<int32_t> kv;
  for (int it = 0; it < 300; ++it) {
    const int op = (int)(rng() % 6);
    if (op == 0) {
      const int32_t id = (int32_t)(rng() % 40), rank = (int32_t)(rng() % 20);
      const int32_t n_proj = 1 + (int32_t)(rng() % 3);
      std::vector<int32_t> din(n_proj), dout(n_proj);
      for (int p = 0; p < n_proj; ++p) {
        din[p] = 8 * (1 + (int32_t)(rng() % 40));
        dout[p] = 8 * (1 + (int32_t)(rng() % 40));
      }
      rc = slora_pool_alloc_adapter(pool, id, rank, n_proj, din.data(), dout.data());
      CHECK(rc == SLORA_OK || rc == SLORA_E_POOL_FULL || rc == SLORA_E_STATE || rc == SLORA_E_INVALID);
      if (rc == SLORA_OK) {
        std::vector<int32_t> d = {n_proj, rank};
        d.insert(d.end(), din.begin(), din.end());
        d.insert(d.end(), dout.begin(), dout.end());
        dims[id] = d;
      }
    } else if (op == 1 && !dims.empty()) {
      auto it2 = dims.begin();
      std::advance(it2, (long)(rng() % dims.size()));
      CHECK(slora_pool_free_adapter(pool, it2->first) == SLORA_OK);
      dims.erase(it2);
    } else if (op == 2) {
      const int32_t n = (int32_t)(rng() % 12);
      std::vector<int32_t> got((size_t)n + 1);
      rc = slora_pool_alloc_kv(pool, n, got.data());
      if (rc == SLORA_OK) kv.insert(kv.end(), got.begin(), got.begin() + n);
    } else if (op == 3 && !kv.empty()) {
      const size_t n = 1 + rng() % kv.size();
      std::shuffle(kv.begin(), kv.end(), rng);
      CHECK((rng() & 1 ? slora_pool_free_kv(pool, kv.data(), (int32_t)n)
                       : slora_pool_free(pool, kv.data(), (int32_t)n)) == SLORA_OK);
      kv.erase(kv.begin(), kv.begin() + (long)n);
      if (!kv.empty()) {  // a repeated id in one call is refused and frees nothing
        int32_t twice[2] = {kv[0], kv[0]};
        CHECK(slora_pool_free_kv(pool, twice, 2) == SLORA_E_INVALID);
      }
    } else if (op == 4) {
      const int32_t proj = (int32_t)(rng() % 3);
      int64_t len = 0;
      std::vector<int32_t> pt(4096);
      std::vector<int64_t> base(41);
      std::vector<int32_t> rank(41);
      rc = slora_pool_page_table(pool, proj, 41, pt.data(), (int64_t)pt.size(), &len, base.data(),
                                 rank.data());
      CHECK(rc == SLORA_OK || rc == SLORA_E_INVALID);
    } else {
      std::vector<int32_t> owner((size_t)n_pages);
      CHECK(slora_pool_owners(pool, owner.data()) == SLORA_OK);
      int64_t free_count = 0, n_free = -1, n_free2 = -1;
      for (int32_t o : owner) free_count += o == -1;
      CHECK(slora_pool_info(pool, nullptr, &n_free, nullptr, nullptr) == SLORA_OK);
      CHECK(slora_pool_n_free(pool, &n_free2) == SLORA_OK);
      CHECK(free_count == n_free && n_free == n_free2);
      int64_t kv_count = 0;
      for (int32_t o : owner) kv_count += o == -2;
      CHECK(kv_count == (int64_t)kv.size());
    }
  }
  CHECK(slora_pool_destroy(pool) == SLORA_OK);
}

// Planner: random calls through slora_plan_inspect and the compute calls' validation;
// every routed token appears exactly once in the plan.
static void plan_round(std::mt19937_64& rng) {
  const int32_t n_ad = 1 + (int32_t)(rng() % 30), P = 8 * (1 + (int32_t)(rng() % 64));
  const int32_t d_in = 8 * (1 + (int32_t)(rng() % 100)), d_out = 8 * (1 + (int32_t)(rng() % 100));
  const int32_t cA = (d_in + P - 1) / P, cB = (d_out + P - 1) / P;
  std::vector<int64_t> base(n_ad);
  std::vector<int32_t> rank(n_ad);
  std::vector<float> scale(n_ad, 0.5f);
  int64_t at = 0;
  int32_t r_max = 1;
  for (int a = 0; a < n_ad; ++a) {
    rank[a] = (int32_t)(rng() % 5 == 0 ? 0 : rng() % 129);
    base[a] = rng() % 7 == 0 ? -1 : at;
    if (base[a] >= 0) at += (int64_t)rank[a] * (cA + cB);
    if (base[a] >= 0) r_max = std::max(r_max, rank[a]);
  }
  slora_lora L;
  std::memset(&L, 0, sizeof L);
  L.pool = kFakeDev;
  L.n_pages = 1 << 20;
  L.page_elems = P;
  L.dtype = rng() & 1 ? SLORA_F16 : SLORA_BF16;
  L.d_in = d_in;
  L.d_out = d_out;
  L.page_table = reinterpret_cast<const int32_t*>(kFakeDev);
  L.page_table_len = std::max<int64_t>(at, 1);
  L.n_adapters = n_ad;
  L.base = base.data();
  L.rank = rank.data();
  L.scale = scale.data();
  L.r_max = r_max;
  const int32_t T = (int32_t)(rng() % 600);
  const int32_t S = T ? (int32_t)(rng() % 9) : 0;
  std::vector<int32_t> off((size_t)S + 1, 0), seg_ad((size_t)S + 1), tok_ad((size_t)T + 1);
  const int32_t seg_tok = S ? (int32_t)(rng() % (T + 1)) : 0;
  for (int s = 1; s < S; ++s) off[(size_t)s] = (int32_t)(rng() % (seg_tok + 1));
  off[(size_t)S] = seg_tok;
  std::sort(off.begin(), off.end());
  for (int s = 0; s < S; ++s) seg_ad[(size_t)s] = (int32_t)(rng() % (n_ad + 1)) - 1;
  for (int t = 0; t < T - seg_tok; ++t) tok_ad[(size_t)t] = (int32_t)(rng() % (n_ad + 1)) - 1;
  slora_routing R;
  std::memset(&R, 0, sizeof R);
  R.n_tokens = T;
  R.n_segments = S;
  R.seg_offsets = S ? off.data() : nullptr;
  R.seg_adapter = seg_ad.data();
  R.token_adapter = tok_ad.data();
  R.policy = (int32_t)(rng() % 3);
  std::vector<int32_t> info(5 * (size_t)(T + 8) + 5), toks((size_t)T + 1);
  int32_t n_groups = 0;
  const int rc = slora_plan_inspect(&L, &R, &n_groups, info.data(), (int32_t)info.size(), toks.data());
  // SLORA_E_STATE: a token routed to an adapter that is not resident (base -1)
  if (rc != SLORA_OK && rc != SLORA_E_INVALID && rc != SLORA_E_STATE)
    std::fprintf(stderr, "plan_inspect rc %d: %s\n", rc, slora_last_error());
  CHECK(rc == SLORA_OK || rc == SLORA_E_INVALID || rc == SLORA_E_STATE);
  if (rc == SLORA_OK) {
    ++g_plans;
    g_groups += n_groups;
    std::vector<int> seen((size_t)T + 1, 0);
    int32_t n_routed = 0;
    for (int g = 0; g < n_groups; ++g) {
      const int32_t first = info[5 * (size_t)g + 1], n = info[5 * (size_t)g + 2];
      CHECK(first >= 0 && n > 0 && first + n <= T);
      for (int q = 0; q < n && first + q <= T; ++q) {
        const int32_t t = toks[(size_t)(first + q)];
        CHECK(t >= 0 && t < T);
        if (t >= 0 && t < T) ++seen[(size_t)t];
      }
      n_routed += n;
    }
    for (int t = 0; t < T; ++t) CHECK(seen[(size_t)t] <= 1);
    int64_t ws = 0;
    CHECK(slora_workspace_size(&L, &R, &ws) == SLORA_OK && ws >= 256);
    int64_t gws = 0;
    const int grc = slora_gathered_workspace_size(&L, &R, &gws);
    CHECK(grc == SLORA_OK || grc == SLORA_E_INVALID);
  }
  // compute calls with a misaligned x are refused before anything reaches a device
  const char* xbad = reinterpret_cast<const char*>(kFakeDev) + 2;
  if (T > 0 && rc == SLORA_OK) {
    CHECK(slora_apply(&L, &R, xbad, kFakeDev, kFakeDev, 1 << 30, nullptr) == SLORA_E_INVALID);
    CHECK(slora_shrink(&L, &R, xbad, reinterpret_cast<float*>(kFakeDev), kFakeDev, 1 << 30,
                       nullptr) == SLORA_E_INVALID);
    // several projections: one region per projection; projections that cannot share the
    // plan, a misaligned x or a projection count outside 1..8 are refused up front
    const int32_t n = 1 + (int32_t)(rng() % 8);
    std::vector<slora_lora> Ls((size_t)n + 1, L);
    std::vector<const void*> xs((size_t)n + 1, kFakeDev);
    std::vector<void*> ys((size_t)n + 1, kFakeDev);
    int64_t one = 0, multi = 0;
    CHECK(slora_workspace_size(&L, &R, &one) == SLORA_OK);
    CHECK(slora_workspace_size_multi(n, Ls.data(), &R, &multi) == SLORA_OK);
    CHECK(multi == n * ((one + 255) / 256 * 256));
    CHECK(slora_workspace_size_multi(9, Ls.data(), &R, &multi) == SLORA_E_INVALID);
    xs[(size_t)(rng() % n)] = xbad;
    CHECK(slora_apply_multi(n, Ls.data(), &R, xs.data(), ys.data(), kFakeDev, 1 << 30, nullptr) ==
          SLORA_E_INVALID);
    std::fill(xs.begin(), xs.end(), kFakeDev);
    if (n > 1) {
      std::vector<int64_t> base2(base);
      std::vector<float> scale2(scale);
      const int32_t q = 1 + (int32_t)(rng() % (n - 1));
      switch (rng() % 3) {
        case 0: Ls[(size_t)q].d_out = d_out + 8; break;
        case 1: base2[(size_t)(rng() % n_ad)] += 1; Ls[(size_t)q].base = base2.data(); break;
        default: scale2[(size_t)(rng() % n_ad)] = 2.f; Ls[(size_t)q].scale = scale2.data(); break;
      }
      CHECK(slora_apply_multi(n, Ls.data(), &R, xs.data(), ys.data(), kFakeDev, 1 << 30, nullptr) ==
            SLORA_E_INVALID);
      CHECK(std::strstr(slora_last_error(), "projection") != nullptr);
    }
  }
}

// Residency manager and admission scheduler on one pool or two; every step keeps the
// pages of both pools conserved.
static void sched_round(std::mt19937_64& rng) {
  const int32_t P = 64;
  const int64_t n_kv = 200 + (int64_t)(rng() % 600);
  const bool split = rng() & 1;
  slora_pool *kvp = nullptr, *adp = nullptr;
  CHECK(slora_pool_create(kFakeDev, n_kv, P, SLORA_F16, rng(), &kvp) == SLORA_OK);
  if (split) CHECK(slora_pool_create_ordered(kFakeDev, 300, P, SLORA_F16, &adp) == SLORA_OK);
  slora_pool* ap = split ? adp : kvp;
  const int32_t d_in[2] = {64, 128}, d_out[2] = {64, 64};
  slora_residency* res = nullptr;
  CHECK(slora_residency_create(ap, 2, d_in, d_out, &res) == SLORA_OK);
  slora_sched_config cfg;
  cfg.kv_pages_per_token = 1 + (int32_t)(rng() % 3);
  cfg.max_batch_tokens = 64 + (int32_t)(rng() % 256);
  cfg.max_running = 1 + (int32_t)(rng() % 24);
  slora_sched* sch = nullptr;
  CHECK(slora_sched_create(kvp, res, &cfg, &sch) == SLORA_OK);
  std::vector<int32_t> ranks(20);
  for (auto& r : ranks) r = 1 + (int32_t)(rng() % 16);
  int64_t next_id = 0;
  std::set<int64_t> live;
  for (int step = 0; step < 200; ++step) {
    for (int k = (int)(rng() % 4); k > 0; --k) {
      const int32_t a = (int32_t)(rng() % 21) - 1;
      const int rc = slora_sched_submit(sch, next_id, a, a >= 0 ? ranks[(size_t)a] : 0,
                                        1 + (int32_t)(rng() % cfg.max_batch_tokens),
                                        1 + (int32_t)(rng() % 20),
                                        rng() % 5 == 0 ? step + (int64_t)(rng() % 10) : -1);
      CHECK(rc == SLORA_OK);
      live.insert(next_id++);
    }
    if (!live.empty() && rng() % 3 == 0) {
      auto it = live.begin();
      std::advance(it, (long)(rng() % live.size()));
      CHECK(slora_sched_finish(sch, *it) == SLORA_OK);
      live.erase(it);
    }
    slora_sched_batch b;
    CHECK(slora_sched_step(sch, &b) == SLORA_OK);
    CHECK(b.n_tokens >= 0 && b.n_tokens <= cfg.max_batch_tokens + cfg.max_running);
    CHECK(b.n_running <= cfg.max_running);
    g_tokens += b.n_tokens;
    g_fetches += b.n_fetch;
    for (int i = 0; i < b.n_finished; ++i) live.erase(b.finished[i]);
    for (int i = 0; i < b.n_aborted; ++i) live.erase(b.aborted[i]);
    if (b.n_segments > 0) CHECK(b.seg_offsets[0] == 0 && b.seg_offsets[b.n_segments] <= b.n_tokens);
    std::vector<int32_t> owner((size_t)n_kv);
    CHECK(slora_pool_owners(kvp, owner.data()) == SLORA_OK);
    int64_t fr = 0;
    for (int32_t o : owner) fr += o == -1;
    CHECK(fr == b.free_pages);
    slora_residency_stats st;
    CHECK(slora_residency_info(res, &st) == SLORA_OK && st.pinned <= st.resident);
  }
  CHECK(slora_sched_destroy(sch) == SLORA_OK);
  slora_residency_stats st;
  CHECK(slora_residency_info(res, &st) == SLORA_OK && st.pinned == 0);
  CHECK(slora_residency_destroy(res) == SLORA_OK);
  std::vector<int32_t> owner((size_t)n_kv);
  CHECK(slora_pool_owners(kvp, owner.data()) == SLORA_OK);
  for (int32_t o : owner) CHECK(o != -2);  // every KV page came back
  CHECK(slora_pool_destroy(kvp) == SLORA_OK);
  if (adp) CHECK(slora_pool_destroy(adp) == SLORA_OK);
}

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 40;
  std::mt19937_64 rng(20261203);
  for (int i = 0; i < rounds; ++i) {
    pool_round(rng);
    plan_round(rng);
    sched_round(rng);
  }
  std::printf("host driver: %d rounds, %lld plans (%lld groups), %lld scheduled tokens, %lld adapter "
              "fetches; %d failed checks\n", rounds, (long long)g_plans, (long long)g_groups,
              (long long)g_tokens, (long long)g_fetches, g_fail);
  return g_fail ? 1 : 0;
}

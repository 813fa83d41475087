// Adapter residency and continuous-batching admission over the unified pool (host,
// integer only).
//
// Residency. All adapters live in host memory and the ones running requests use are
// fetched to GPU memory on demand (review "S-LoRA: Serving Thousands of Concurrent
// LoRA Adapters", abstract and "Proposed method"); when the active adapters outgrow the
// pool, adapters are swapped over PCIe and the copies show in the tail latency
// ("Makale Bulteni - S-LoRA", section "Iddia ve Gerceklik"). slora_residency keeps the
// adapters of one pool with a pin count each (pinned = used by a running request) and
// evicts unpinned ones in least-recently-used order (an adapter's recency is its last
// release, or its prefetch) when an acquire needs room; a
// prefetch makes an adapter resident only from free pages. It never copies: the caller
// fetches what an acquire or prefetch reports (slora_fetch_async) before using it.
//
// Admission. Requests wait in a FIFO queue; every step the scheduler keeps the running
// requests (one decode token each), and admits waiting requests while the pool has
// free pages for their prompt's KV cache and the step has token budget left, without
// waiting for the batch to drain; a request that reaches its output length, or is
// finished by the caller, leaves the batch and its KV pages return to the free list at
// once (the continuous-batching page, sections "Surekli Gruplama ... Nasil Calisir?" and
// "vLLM Zamanlayicisi: Istekleri Dinamik Olarak Yonetme": admission by the count of
// free KV pages, pages freed on completion). S-LoRA integrates early-abort scheduling
// with the unified pool (review, "Proposed method"); here a request carries a
// deadline step, and a waiting or running request past it is aborted at once, its
// pages freed, so no pool space or compute goes to a request that has already missed
// it. When the running requests' next tokens need more KV pages than are free, the
// most recently admitted requests are aborted until the rest fit.
//
// KV pages: one page holds one token's K or V vector for one layer (page = hidden
// size), so a token takes kv_pages_per_token pages. Every batch a step produces is a
// slora_routing: the prompts of newly admitted requests as segments, then one decode
// token per running request.
#include <string.h>

#include <algorithm>
#include <deque>
#include <map>
#include <set>
#include <vector>

#include "guard.h"
#include "internal.h"

using namespace slora;

struct slora_residency {
  slora_pool* pool = nullptr;
  std::vector<int32_t> d_in, d_out;
  struct Rec {
    int32_t rank = 0;
    int32_t pins = 0;
    uint64_t last_use = 0;
  };
  std::map<int32_t, Rec> resident;
  std::set<std::pair<uint64_t, int32_t>> lru;  // unpinned resident adapters, oldest first
  uint64_t clock = 0;
  int64_t hits = 0, misses = 0, evictions = 0, prefetches = 0;
};

namespace {

int64_t need_pages(const slora_residency* r, int32_t rank) {
  return pool_adapter_need(r->pool, rank, (int32_t)r->d_in.size(), r->d_in.data(), r->d_out.data());
}

int64_t pool_free(const slora_pool* pool) {
  int64_t f = 0;
  (void)slora_pool_info(pool, nullptr, &f, nullptr, nullptr);
  return f;
}

// Unpinned adapters other than `keep`, least recently used first, whose eviction
// would bring the free pages to `need`; none with a fetch that may still be in flight.
// *enough is false (and nothing may be evicted) when all of them together fall short.
int plan_evictions(slora_residency* r, int64_t need, std::vector<int32_t>* victims, bool* enough,
                   int32_t keep = -1) {
  victims->clear();
  int64_t have = pool_free(r->pool);
  *enough = have >= need;
  for (auto it = r->lru.begin(); it != r->lru.end() && !*enough; ++it) {
    if (it->second == keep) continue;
    int64_t pages = 0;
    bool busy = false;
    const int rc = pool_adapter_state(r->pool, it->second, &pages, &busy);
    if (rc) return rc;
    if (busy) continue;
    victims->push_back(it->second);
    have += pages;
    *enough = have >= need;
  }
  return SLORA_OK;
}

int evict(slora_residency* r, int32_t id) {
  auto it = r->resident.find(id);
  const int rc = slora_pool_free_adapter(r->pool, id);
  if (rc) return rc;
  r->lru.erase({it->second.last_use, id});
  r->resident.erase(it);
  ++r->evictions;
  return SLORA_OK;
}

// Acquire (pin) or prefetch (no pin, free pages only) adapter `id`.
int acquire(slora_residency* r, int32_t id, int32_t rank, bool pin, int32_t* needs_fetch,
            std::vector<int32_t>* evicted) {
  *needs_fetch = 0;
  auto it = r->resident.find(id);
  if (it != r->resident.end()) {
    if (it->second.rank != rank)
      return fail(SLORA_E_INVALID, "residency: adapter %d is resident with rank %d, not %d", id,
                  it->second.rank, rank);
    if (!pin) return SLORA_OK;  // a prefetch of a resident adapter does nothing
    if (it->second.pins == 0) r->lru.erase({it->second.last_use, id});
    ++it->second.pins;
    it->second.last_use = ++r->clock;
    ++r->hits;
    return SLORA_OK;
  }
  const int64_t need = need_pages(r, rank);
  if (pin) {
    std::vector<int32_t> victims;
    bool enough = false;
    int rc = plan_evictions(r, need, &victims, &enough);
    if (rc) return rc;
    if (!enough)
      return fail(SLORA_E_POOL_FULL, "residency: adapter %d needs %lld pages; free and evictable "
                  "pages do not reach that", id, (long long)need);
    for (int32_t v : victims) {
      rc = evict(r, v);
      if (rc) return rc;
      if (evicted) evicted->push_back(v);
    }
  } else if (pool_free(r->pool) < need) {
    return SLORA_OK;  // no room without evicting: no prefetch
  }
  int rc = slora_pool_alloc_adapter(r->pool, id, rank, (int32_t)r->d_in.size(), r->d_in.data(),
                                    r->d_out.data());
  if (rc) return rc;
  slora_residency::Rec rec;
  rec.rank = rank;
  rec.pins = pin ? 1 : 0;
  rec.last_use = ++r->clock;
  r->resident[id] = rec;
  if (!pin) r->lru.insert({rec.last_use, id});
  ++(pin ? r->misses : r->prefetches);
  *needs_fetch = 1;
  return SLORA_OK;
}

int release(slora_residency* r, int32_t id) {
  auto it = r->resident.find(id);
  if (it == r->resident.end() || it->second.pins <= 0)
    return fail(SLORA_E_STATE, "residency: adapter %d is not pinned", id);
  if (--it->second.pins == 0) {  // in use until now: its recency is this release
    it->second.last_use = ++r->clock;
    r->lru.insert({it->second.last_use, id});
  }
  return SLORA_OK;
}

}  // namespace

// ---------------------------------------------------------------- scheduler
struct slora_sched {
  slora_pool* pool = nullptr;
  slora_residency* res = nullptr;
  slora_sched_config cfg{};
  struct Req {
    int64_t id = 0;
    int32_t adapter = -1, rank = 0, prompt = 0, max_new = 0, generated = 0;
    int64_t deadline = -1;
    std::vector<int32_t> kv;  // KV pages held
  };
  std::deque<Req> queue;
  std::vector<Req> running;  // in admission order
  std::set<int64_t> ids;     // ids waiting or running
  int64_t step = 0;
  // the last step's batch (slora_sched_batch points into these)
  std::vector<int32_t> seg_offsets, seg_adapter, token_adapter, fetch, evicted, abort_reason;
  std::vector<int64_t> seg_request, token_request, finished, aborted;
  int64_t n_admitted = 0, n_finished = 0, n_aborted = 0;
};

namespace {

int free_kv(slora_sched* s, slora_sched::Req& q) {
  if (!q.kv.empty()) {
    const int rc = slora_pool_free_kv(s->pool, q.kv.data(), (int32_t)q.kv.size());
    if (rc) return rc;
    q.kv.clear();
  }
  return SLORA_OK;
}

// A running request leaves the batch: KV pages back to the pool, adapter unpinned.
int retire(slora_sched* s, slora_sched::Req& q) {
  int rc = free_kv(s, q);
  if (rc) return rc;
  if (s->res && q.adapter >= 0 && q.rank > 0) rc = release(s->res, q.adapter);
  s->ids.erase(q.id);
  return rc;
}

void note_abort(slora_sched* s, int64_t id, int32_t reason) {
  s->aborted.push_back(id);
  s->abort_reason.push_back(reason);
  ++s->n_aborted;
}

int do_step(slora_sched* s) {
  s->seg_offsets.assign(1, 0);
  s->seg_adapter.clear();
  s->token_adapter.clear();
  s->seg_request.clear();
  s->token_request.clear();
  s->fetch.clear();
  s->evicted.clear();
  s->finished.clear();
  s->aborted.clear();
  s->abort_reason.clear();
  const int64_t now = ++s->step;
  const int32_t ppt = s->cfg.kv_pages_per_token;
  int rc = SLORA_OK;

  // 1. requests that reached their output length leave; requests past their deadline
  //    are aborted, waiting or running
  std::vector<slora_sched::Req> keep;
  keep.reserve(s->running.size());
  for (auto& q : s->running) {
    const bool done = q.generated >= q.max_new;
    const bool late = q.deadline >= 0 && now > q.deadline;
    if (done || late) {
      rc = retire(s, q);
      if (rc) return rc;
      if (done) {
        s->finished.push_back(q.id);
        ++s->n_finished;
      } else {
        note_abort(s, q.id, SLORA_ABORT_DEADLINE);
      }
    } else {
      keep.push_back(std::move(q));
    }
  }
  s->running.swap(keep);
  for (auto it = s->queue.begin(); it != s->queue.end();) {
    if (it->deadline >= 0 && now > it->deadline) {
      note_abort(s, it->id, SLORA_ABORT_DEADLINE);
      s->ids.erase(it->id);
      it = s->queue.erase(it);
    } else {
      ++it;
    }
  }

  // 2. every running request decodes one token, which needs ppt more KV pages; the most
  //    recently admitted requests are aborted while the pool cannot hold them all
  while (!s->running.empty() && pool_free(s->pool) < (int64_t)s->running.size() * ppt) {
    rc = retire(s, s->running.back());
    if (rc) return rc;
    note_abort(s, s->running.back().id, SLORA_ABORT_POOL_FULL);
    s->running.pop_back();
  }
  int64_t tokens = 0;
  for (auto& q : s->running) {
    const size_t at = q.kv.size();
    q.kv.resize(at + (size_t)ppt);
    rc = slora_pool_alloc_kv(s->pool, ppt, q.kv.data() + at);
    if (rc) return rc;  // cannot happen: the pages were counted above
    s->token_adapter.push_back(q.adapter);
    s->token_request.push_back(q.id);
    ++q.generated;
    ++tokens;
  }

  // 3. FIFO admission while the step has token budget and the pool has pages for the
  //    prompt's KV (and the adapter, evicting unpinned adapters if need be); the head of
  //    the queue that does not fit stops admission
  std::vector<slora_sched::Req> admitted;
  int32_t seg_tokens = 0;
  while (!s->queue.empty() && (int64_t)s->running.size() + (int64_t)admitted.size() < s->cfg.max_running) {
    slora_sched::Req& q = s->queue.front();
    if (tokens + q.prompt > s->cfg.max_batch_tokens) break;
    const int64_t kv_need = (int64_t)q.prompt * ppt;
    const bool lora = s->res && q.adapter >= 0 && q.rank > 0;
    if (lora) {
      // room for the adapter (unless resident) and the prompt's KV together, from free
      // pages and evictions of other unpinned adapters; then pin the adapter. With the
      // adapters in a pool of their own, the two needs are met by their own pools.
      auto it = s->res->resident.find(q.adapter);
      const int64_t a_need = it == s->res->resident.end() ? need_pages(s->res, q.rank) : 0;
      const bool unified = s->res->pool == s->pool;
      if (!unified && pool_free(s->pool) < kv_need) break;
      std::vector<int32_t> victims;
      bool enough = false;
      rc = plan_evictions(s->res, unified ? a_need + kv_need : a_need, &victims, &enough, q.adapter);
      if (rc) return rc;
      if (!enough) break;
      for (int32_t v : victims) {
        rc = evict(s->res, v);
        if (rc) return rc;
        s->evicted.push_back(v);
      }
      int32_t needs_fetch = 0;
      rc = acquire(s->res, q.adapter, q.rank, true, &needs_fetch, &s->evicted);
      if (rc) return rc;  // cannot be short of pages: they were freed above
      if (needs_fetch) s->fetch.push_back(q.adapter);
    } else if (pool_free(s->pool) < kv_need) {
      break;
    }
    q.kv.resize((size_t)kv_need);
    rc = slora_pool_alloc_kv(s->pool, (int32_t)kv_need, q.kv.data());
    if (rc) return rc;
    q.generated = 1;  // the prompt's step yields the first output token
    s->seg_adapter.push_back(q.adapter);
    s->seg_request.push_back(q.id);
    seg_tokens += q.prompt;
    s->seg_offsets.push_back(seg_tokens);
    tokens += q.prompt;
    admitted.push_back(std::move(q));
    s->queue.pop_front();
    ++s->n_admitted;
  }
  // the batch: the new prompts (segments) first, then the decode tokens
  for (auto& q : admitted) s->running.push_back(std::move(q));
  return SLORA_OK;
}

}  // namespace

extern "C" {

int slora_residency_create(slora_pool* pool, int32_t n_proj, const int32_t* d_in,
                           const int32_t* d_out, slora_residency** out) {
  return guarded(__func__, [&] {
    clear_error();
    if (!out) return fail(SLORA_E_INVALID, "residency_create: out is NULL");
    *out = nullptr;
    if (!pool || n_proj < 1 || n_proj > 64 || !d_in || !d_out)
      return fail(SLORA_E_INVALID, "residency_create: bad arguments");
    for (int32_t p = 0; p < n_proj; ++p)
      if (d_in[p] <= 0 || d_out[p] <= 0 || d_in[p] % 8 || d_out[p] % 8)
        return fail(SLORA_E_INVALID, "residency_create: projection %d shape %dx%d", p, d_in[p], d_out[p]);
    auto* r = new slora_residency;
    r->pool = pool;
    r->d_in.assign(d_in, d_in + n_proj);
    r->d_out.assign(d_out, d_out + n_proj);
    *out = r;
    return SLORA_OK;
  });
}

int slora_residency_destroy(slora_residency* r) {
  return guarded(__func__, [&] {
    clear_error();
    delete r;
    return SLORA_OK;
  });
}

int slora_residency_acquire(slora_residency* r, int32_t adapter_id, int32_t rank,
                            int32_t* needs_fetch, int32_t* evicted, int32_t evicted_cap,
                            int32_t* n_evicted) {
  return guarded(__func__, [&] {
    clear_error();
    if (!r || !needs_fetch || !n_evicted || evicted_cap < 0 || (evicted_cap > 0 && !evicted))
      return fail(SLORA_E_INVALID, "residency_acquire: bad arguments");
    if (adapter_id < 0 || rank < 0 || rank > kMaxRank)
      return fail(SLORA_E_INVALID, "residency_acquire: adapter %d rank %d", adapter_id, rank);
    std::vector<int32_t> ev;
    const int rc = acquire(r, adapter_id, rank, true, needs_fetch, &ev);
    *n_evicted = (int32_t)ev.size();
    for (size_t i = 0; i < ev.size() && (int32_t)i < evicted_cap; ++i) evicted[i] = ev[i];
    if (rc == SLORA_OK && (int32_t)ev.size() > evicted_cap)
      return fail(SLORA_E_INVALID, "residency_acquire: %zu evictions, room for %d listed", ev.size(),
                  evicted_cap);
    return rc;
  });
}

int slora_residency_prefetch(slora_residency* r, int32_t adapter_id, int32_t rank, int32_t* needs_fetch) {
  return guarded(__func__, [&] {
    clear_error();
    if (!r || !needs_fetch || adapter_id < 0 || rank < 0 || rank > kMaxRank)
      return fail(SLORA_E_INVALID, "residency_prefetch: bad arguments");
    return acquire(r, adapter_id, rank, false, needs_fetch, nullptr);
  });
}

int slora_residency_release(slora_residency* r, int32_t adapter_id) {
  return guarded(__func__, [&] {
    clear_error();
    if (!r) return fail(SLORA_E_INVALID, "residency_release: NULL");
    return release(r, adapter_id);
  });
}

int slora_residency_info(const slora_residency* r, slora_residency_stats* st) {
  return guarded(__func__, [&] {
    clear_error();
    if (!r || !st) return fail(SLORA_E_INVALID, "residency_info: NULL");
    memset(st, 0, sizeof *st);
    st->resident = (int32_t)r->resident.size();
    for (const auto& kv : r->resident) st->pinned += kv.second.pins > 0 ? 1 : 0;
    st->hits = r->hits;
    st->misses = r->misses;
    st->evictions = r->evictions;
    st->prefetches = r->prefetches;
    return SLORA_OK;
  });
}

int slora_residency_is_resident(const slora_residency* r, int32_t adapter_id, int32_t* pins) {
  return guarded(__func__, [&] {
    clear_error();
    if (!r || !pins) return fail(SLORA_E_INVALID, "residency_is_resident: NULL");
    auto it = r->resident.find(adapter_id);
    *pins = it == r->resident.end() ? -1 : it->second.pins;
    return SLORA_OK;
  });
}

int slora_sched_create(slora_pool* pool, slora_residency* res, const slora_sched_config* cfg,
                       slora_sched** out) {
  return guarded(__func__, [&] {
    clear_error();
    if (!out) return fail(SLORA_E_INVALID, "sched_create: out is NULL");
    *out = nullptr;
    if (!pool || !cfg) return fail(SLORA_E_INVALID, "sched_create: pool / config is NULL");
    if (cfg->kv_pages_per_token < 1 || cfg->max_running < 1 || cfg->max_batch_tokens < cfg->max_running)
      return fail(SLORA_E_INVALID, "sched_create: kv_pages_per_token, max_running >= 1 and "
                  "max_batch_tokens >= max_running required");
    auto* s = new slora_sched;
    s->pool = pool;
    s->res = res;
    s->cfg = *cfg;
    s->seg_offsets.assign(1, 0);
    *out = s;
    return SLORA_OK;
  });
}

int slora_sched_destroy(slora_sched* s) {
  return guarded(__func__, [&] {
    clear_error();
    if (!s) return SLORA_OK;
    int rc = SLORA_OK;
    for (auto& q : s->running) {
      const int r2 = retire(s, q);
      if (rc == SLORA_OK) rc = r2;
    }
    delete s;
    return rc;
  });
}

int slora_sched_submit(slora_sched* s, int64_t request_id, int32_t adapter_id, int32_t rank,
                       int32_t prompt_len, int32_t max_new_tokens, int64_t deadline_step) {
  return guarded(__func__, [&] {
    clear_error();
    if (!s) return fail(SLORA_E_INVALID, "sched_submit: NULL");
    if (prompt_len < 1 || max_new_tokens < 1 || adapter_id < -1 || rank < 0 || rank > kMaxRank)
      return fail(SLORA_E_INVALID, "sched_submit: request %lld: bad shape", (long long)request_id);
    if (prompt_len > s->cfg.max_batch_tokens)
      return fail(SLORA_E_INVALID, "sched_submit: prompt of %d tokens exceeds the step budget %d",
                  prompt_len, s->cfg.max_batch_tokens);
    if (!s->ids.insert(request_id).second)
      return fail(SLORA_E_STATE, "sched_submit: request %lld is already queued or running",
                  (long long)request_id);
    slora_sched::Req q;
    q.id = request_id;
    q.adapter = adapter_id;
    q.rank = rank;
    q.prompt = prompt_len;
    q.max_new = max_new_tokens;
    q.deadline = deadline_step;
    s->queue.push_back(std::move(q));
    return SLORA_OK;
  });
}

int slora_sched_finish(slora_sched* s, int64_t request_id) {
  return guarded(__func__, [&] {
    clear_error();
    if (!s) return fail(SLORA_E_INVALID, "sched_finish: NULL");
    for (size_t i = 0; i < s->running.size(); ++i)
      if (s->running[i].id == request_id) {
        const int rc = retire(s, s->running[i]);
        s->running.erase(s->running.begin() + (ptrdiff_t)i);
        ++s->n_finished;
        return rc;
      }
    for (auto it = s->queue.begin(); it != s->queue.end(); ++it)
      if (it->id == request_id) {
        s->ids.erase(it->id);
        s->queue.erase(it);
        ++s->n_aborted;
        return SLORA_OK;
      }
    return fail(SLORA_E_STATE, "sched_finish: request %lld is neither queued nor running",
                (long long)request_id);
  });
}

int slora_sched_step(slora_sched* s, slora_sched_batch* out) {
  return guarded(__func__, [&] {
    clear_error();
    if (!s || !out) return fail(SLORA_E_INVALID, "sched_step: NULL");
    const int rc = do_step(s);
    memset(out, 0, sizeof *out);
    out->step = s->step;
    out->n_segments = (int32_t)s->seg_adapter.size();
    out->n_tokens = s->seg_offsets.back() + (int32_t)s->token_adapter.size();
    out->seg_offsets = s->seg_offsets.data();
    out->seg_adapter = s->seg_adapter.data();
    out->token_adapter = s->token_adapter.data();
    out->seg_request = s->seg_request.data();
    out->token_request = s->token_request.data();
    out->n_fetch = (int32_t)s->fetch.size();
    out->fetch = s->fetch.data();
    out->n_evicted = (int32_t)s->evicted.size();
    out->evicted = s->evicted.data();
    out->n_finished = (int32_t)s->finished.size();
    out->finished = s->finished.data();
    out->n_aborted = (int32_t)s->aborted.size();
    out->aborted = s->aborted.data();
    out->abort_reason = s->abort_reason.data();
    out->n_waiting = (int32_t)s->queue.size();
    out->n_running = (int32_t)s->running.size();
    out->free_pages = pool_free(s->pool);
    return rc;
  });
}

int slora_sched_request_pages(const slora_sched* s, int64_t request_id, int32_t* pages, int32_t cap,
                              int32_t* n) {
  return guarded(__func__, [&] {
    clear_error();
    if (!s || !n || cap < 0 || (cap > 0 && !pages)) return fail(SLORA_E_INVALID, "sched_request_pages: bad arguments");
    for (const auto& q : s->running)
      if (q.id == request_id) {
        *n = (int32_t)q.kv.size();
        if (*n > cap) return fail(SLORA_E_INVALID, "sched_request_pages: %d pages, room for %d", *n, cap);
        if (*n) memcpy(pages, q.kv.data(), q.kv.size() * sizeof(int32_t));
        return SLORA_OK;
      }
    *n = 0;
    return fail(SLORA_E_STATE, "sched_request_pages: request %lld is not running", (long long)request_id);
  });
}

}  // extern "C"

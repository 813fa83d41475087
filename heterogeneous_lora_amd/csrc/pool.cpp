// Unified page pool: one shuffled free list shared by adapter weights and KV-cache
// pages, per-adapter page lists, page-table export, and the host->HBM fetch.
//
// S-LoRA overview (Chinese), section "1. Unified Paging": one memory pool holds the
// weights of adapters of different ranks and KV tensors of different sequence
// lengths. Paper review "S-LoRA: Serving Thousands of Concurrent LoRA Adapters",
// abstract and "Proposed method": all adapters stay in host memory; those the
// running requests use are fetched to GPU memory on demand. "Makale Bulteni -
// S-LoRA", section "Iddia ve Gerceklik": the transfer is asynchronous and page by
// page from DRAM to the GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <memory>
#include <mutex>

#include "guard.h"
#include "internal.h"

namespace slora {

static thread_local std::string t_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    t_error = buf;
  } catch (...) {  // no message rather than an exception across the C ABI
  }
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SLORA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

void clear_error() { t_error.clear(); }

}  // namespace slora

using namespace slora;

namespace {

// The completion event of one fetch call, shared by the adapters it moved.
struct FetchMark {
  hipEvent_t ev = nullptr;
  ~FetchMark() {
    if (ev) (void)hipEventDestroy(ev);
  }
};

struct AdapterRec {
  int32_t rank = 0;
  std::vector<int32_t> d_in, d_out;
  std::vector<std::vector<int32_t>> pages;  // per projection, page-table order
  std::shared_ptr<FetchMark> fetch;         // the last fetch into this adapter, if any
};

// splitmix64: a small seeded generator for the free-list shuffle
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  uint64_t below(uint64_t n) {  // unbiased in [0, n)
    uint64_t lim = UINT64_MAX - UINT64_MAX % n;
    uint64_t x;
    do x = next(); while (x >= lim);
    return x % n;
  }
};

constexpr int32_t kFree = -1;
constexpr int32_t kKV = -2;

}  // namespace

// Pinned page lists of fetch launches, reused round-robin; one is refilled only after
// the launch that read it has finished (its event).
constexpr int kFetchStages = 4;
struct FetchStage {
  slora::FetchPage* host = nullptr;
  int64_t cap = 0;  // entries
  hipEvent_t ev = nullptr;
  bool pending = false;
};

struct slora_pool {
  void* dev = nullptr;
  int64_t n_pages = 0;
  int32_t P = 0;
  int32_t dtype = 0;
  std::vector<int32_t> free_list;  // stack: pop from the back
  std::vector<int32_t> owner;      // per page: adapter id, kFree or kKV
  std::map<int32_t, AdapterRec> adapters;
  FetchStage stage[kFetchStages];
  int stage_next = 0;
  std::vector<slora::FetchPage> pages_scratch;  // a call's page list before it is staged
};

namespace slora {

int pool_adapter_state(const slora_pool* pool, int32_t id, int64_t* pages, bool* busy) {
  *pages = 0;
  *busy = false;
  auto it = pool->adapters.find(id);
  if (it == pool->adapters.end()) return SLORA_OK;
  for (const auto& pg : it->second.pages) *pages += (int64_t)pg.size();
  if (it->second.fetch) {
    const hipError_t e = hipEventQuery(it->second.fetch->ev);
    if (e == hipErrorNotReady) *busy = true;
    else if (e != hipSuccess) return hip_fail(e, "hipEventQuery");
  }
  return SLORA_OK;
}

int64_t pool_adapter_need(const slora_pool* pool, int32_t rank, int32_t n_proj, const int32_t* d_in,
                          const int32_t* d_out) {
  int64_t need = 0;
  for (int32_t p = 0; p < n_proj; ++p)
    need += (int64_t)rank * ((d_in[p] + pool->P - 1) / pool->P + (d_out[p] + pool->P - 1) / pool->P);
  return need;
}

}  // namespace slora

extern "C" {

const char* slora_last_error(void) { return t_error.c_str(); }

int slora_abi_version(void) { return SLORA_ABI_VERSION; }

static int impl_slora_pool_create(void* dev_pages, int64_t n_pages, int32_t page_elems, int32_t dtype,
                      uint64_t shuffle_seed, bool ordered, slora_pool** out) {
  clear_error();
  if (!out) return fail(SLORA_E_INVALID, "pool_create: out is NULL");
  *out = nullptr;
  if (!dev_pages) return fail(SLORA_E_INVALID, "pool_create: dev_pages is NULL");
  if ((reinterpret_cast<uintptr_t>(dev_pages) & 15) != 0)
    return fail(SLORA_E_INVALID, "pool_create: dev_pages must be 16-byte aligned");
  if (n_pages <= 0 || n_pages > INT32_MAX)
    return fail(SLORA_E_INVALID, "pool_create: n_pages %lld out of range", (long long)n_pages);
  if (page_elems <= 0 || page_elems % 8 != 0)
    return fail(SLORA_E_INVALID, "pool_create: page_elems %d must be a positive multiple of 8",
                page_elems);
  if (dtype != SLORA_F16 && dtype != SLORA_BF16)
    return fail(SLORA_E_INVALID, "pool_create: unknown dtype %d", dtype);
  slora_pool* p = new (std::nothrow) slora_pool;
  if (!p) return fail(SLORA_E_INVALID, "pool_create: out of host memory");
  p->dev = dev_pages;
  p->n_pages = n_pages;
  p->P = page_elems;
  p->dtype = dtype;
  p->owner.assign((size_t)n_pages, kFree);
  p->free_list.resize((size_t)n_pages);
  for (int64_t i = 0; i < n_pages; ++i) p->free_list[(size_t)i] = (int32_t)i;
  if (ordered) {  // a stack popped from the back: pages are handed out in ascending order
    std::reverse(p->free_list.begin(), p->free_list.end());
  } else {
    SplitMix64 rng{shuffle_seed};
    for (int64_t i = n_pages - 1; i > 0; --i) {  // Fisher-Yates
      int64_t j = (int64_t)rng.below((uint64_t)i + 1);
      std::swap(p->free_list[(size_t)i], p->free_list[(size_t)j]);
    }
  }
  *out = p;
  return SLORA_OK;
}

static int impl_slora_pool_destroy(slora_pool* pool) {
  clear_error();
  if (!pool) return SLORA_OK;
  int rc = SLORA_OK;
  for (auto& kv : pool->adapters) {
    AdapterRec& a = kv.second;
    if (a.fetch) {
      hipError_t e = hipEventSynchronize(a.fetch->ev);
      if (e != hipSuccess && rc == SLORA_OK) rc = hip_fail(e, "pool_destroy: hipEventSynchronize");
    }
  }
  for (FetchStage& st : pool->stage) {
    if (st.pending) {
      hipError_t e = hipEventSynchronize(st.ev);
      if (e != hipSuccess && rc == SLORA_OK) rc = hip_fail(e, "pool_destroy: hipEventSynchronize");
    }
    if (st.ev) (void)hipEventDestroy(st.ev);
    if (st.host) (void)hipHostFree(st.host);
  }
  delete pool;
  return rc;
}

static int impl_slora_pool_info(const slora_pool* pool, int64_t* n_pages, int64_t* n_free, int32_t* page_elems,
                    int32_t* dtype) {
  clear_error();
  if (!pool) return fail(SLORA_E_INVALID, "pool_info: pool is NULL");
  if (n_pages) *n_pages = pool->n_pages;
  if (n_free) *n_free = (int64_t)pool->free_list.size();
  if (page_elems) *page_elems = pool->P;
  if (dtype) *dtype = pool->dtype;
  return SLORA_OK;
}

static int impl_slora_pool_alloc_kv(slora_pool* pool, int32_t n, int32_t* out_page_ids) {
  clear_error();
  if (!pool) return fail(SLORA_E_INVALID, "alloc_kv: pool is NULL");
  if (n < 0) return fail(SLORA_E_INVALID, "alloc_kv: n < 0");
  if (n > 0 && !out_page_ids) return fail(SLORA_E_INVALID, "alloc_kv: out_page_ids is NULL");
  if ((size_t)n > pool->free_list.size())
    return fail(SLORA_E_POOL_FULL, "alloc_kv: %d pages requested, %zu free", n,
                pool->free_list.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t pg = pool->free_list.back();
    pool->free_list.pop_back();
    pool->owner[(size_t)pg] = kKV;
    out_page_ids[i] = pg;
  }
  return SLORA_OK;
}

static int impl_slora_pool_free_kv(slora_pool* pool, const int32_t* page_ids, int32_t n) {
  clear_error();
  if (!pool) return fail(SLORA_E_INVALID, "free_kv: pool is NULL");
  if (n < 0 || (n > 0 && !page_ids)) return fail(SLORA_E_INVALID, "free_kv: bad page list");
  std::vector<int32_t> seen;
  for (int32_t i = 0; i < n; ++i) {  // validate everything first: all-or-nothing
    int32_t pg = page_ids[i];
    if (pg < 0 || pg >= pool->n_pages || pool->owner[(size_t)pg] != kKV)
      return fail(SLORA_E_INVALID, "free_kv: page %d is not a KV page of this pool", pg);
    seen.push_back(pg);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(SLORA_E_INVALID, "free_kv: duplicate page id");
  for (int32_t i = 0; i < n; ++i) {
    pool->owner[(size_t)page_ids[i]] = kFree;
    pool->free_list.push_back(page_ids[i]);
  }
  return SLORA_OK;
}

static int impl_slora_pool_alloc_adapter(slora_pool* pool, int32_t adapter_id, int32_t rank, int32_t n_proj,
                             const int32_t* d_in, const int32_t* d_out) {
  clear_error();
  if (!pool) return fail(SLORA_E_INVALID, "alloc_adapter: pool is NULL");
  if (adapter_id < 0) return fail(SLORA_E_INVALID, "alloc_adapter: adapter_id %d < 0", adapter_id);
  if (rank < 0 || rank > kMaxRank)
    return fail(SLORA_E_INVALID, "alloc_adapter: rank %d outside [0, %d]", rank, kMaxRank);
  if (n_proj < 1 || n_proj > 64 || !d_in || !d_out)
    return fail(SLORA_E_INVALID, "alloc_adapter: bad projection list");
  if (pool->adapters.count(adapter_id))
    return fail(SLORA_E_STATE, "alloc_adapter: adapter %d is already resident", adapter_id);
  int64_t need = 0;
  for (int32_t p = 0; p < n_proj; ++p) {
    if (d_in[p] <= 0 || d_out[p] <= 0 || d_in[p] % 8 || d_out[p] % 8)
      return fail(SLORA_E_INVALID, "alloc_adapter: projection %d shape %dx%d (multiples of 8)", p,
                  d_in[p], d_out[p]);
    int64_t cA = (d_in[p] + pool->P - 1) / pool->P, cB = (d_out[p] + pool->P - 1) / pool->P;
    need += (int64_t)rank * (cA + cB);
  }
  if (need > (int64_t)pool->free_list.size())
    return fail(SLORA_E_POOL_FULL, "alloc_adapter: adapter %d needs %lld pages, %zu free",
                adapter_id, (long long)need, pool->free_list.size());
  AdapterRec rec;
  rec.rank = rank;
  rec.d_in.assign(d_in, d_in + n_proj);
  rec.d_out.assign(d_out, d_out + n_proj);
  rec.pages.resize((size_t)n_proj);
  for (int32_t p = 0; p < n_proj; ++p) {
    int64_t cA = (d_in[p] + pool->P - 1) / pool->P, cB = (d_out[p] + pool->P - 1) / pool->P;
    int64_t n = (int64_t)rank * (cA + cB);
    std::vector<int32_t>& pg = rec.pages[(size_t)p];
    pg.resize((size_t)n);
    for (int64_t e = 0; e < n; ++e) {
      int32_t id = pool->free_list.back();
      pool->free_list.pop_back();
      pool->owner[(size_t)id] = adapter_id;
      pg[(size_t)e] = id;
    }
  }
  pool->adapters.emplace(adapter_id, std::move(rec));
  return SLORA_OK;
}

static int impl_slora_pool_free_adapter(slora_pool* pool, int32_t adapter_id) {
  clear_error();
  if (!pool) return fail(SLORA_E_INVALID, "free_adapter: pool is NULL");
  auto it = pool->adapters.find(adapter_id);
  if (it == pool->adapters.end())
    return fail(SLORA_E_STATE, "free_adapter: adapter %d is not resident", adapter_id);
  AdapterRec& a = it->second;
  if (a.fetch) {
    hipError_t e = hipEventQuery(a.fetch->ev);
    if (e == hipErrorNotReady)
      return fail(SLORA_E_STATE, "free_adapter: a fetch into adapter %d is still in flight",
                  adapter_id);
    if (e != hipSuccess) return hip_fail(e, "free_adapter: hipEventQuery");
  }
  for (auto& pg : a.pages)
    for (int32_t id : pg) {
      pool->owner[(size_t)id] = kFree;
      pool->free_list.push_back(id);
    }
  pool->adapters.erase(it);
  return SLORA_OK;
}

static int impl_slora_pool_page_table(const slora_pool* pool, int32_t proj, int32_t n_adapters, int32_t* pt,
                          int64_t pt_cap, int64_t* pt_len, int64_t* base, int32_t* rank) {
  clear_error();
  if (!pool) return fail(SLORA_E_INVALID, "page_table: pool is NULL");
  if (proj < 0 || n_adapters < 0 || !pt_len || pt_cap < 0 || (pt_cap > 0 && !pt))
    return fail(SLORA_E_INVALID, "page_table: bad arguments");
  if (n_adapters > 0 && (!base || !rank))
    return fail(SLORA_E_INVALID, "page_table: base / rank is NULL");
  int64_t len = 0;
  for (int32_t i = 0; i < n_adapters; ++i) {
    auto it = pool->adapters.find(i);
    if (it != pool->adapters.end() && proj < (int32_t)it->second.pages.size())
      len += (int64_t)it->second.pages[(size_t)proj].size();
  }
  *pt_len = len;
  if (!pt) {  // length query only
    for (int32_t i = 0; i < n_adapters; ++i) { base[i] = -1; rank[i] = 0; }
    return SLORA_OK;
  }
  if (len > pt_cap)
    return fail(SLORA_E_INVALID, "page_table: %lld entries do not fit in %lld", (long long)len,
                (long long)pt_cap);
  int64_t at = 0;
  for (int32_t i = 0; i < n_adapters; ++i) {
    auto it = pool->adapters.find(i);
    if (it == pool->adapters.end() || proj >= (int32_t)it->second.pages.size()) {
      base[i] = -1;
      rank[i] = 0;
      continue;
    }
    const std::vector<int32_t>& pg = it->second.pages[(size_t)proj];
    base[i] = at;
    rank[i] = it->second.rank;
    if (!pg.empty()) memcpy(pt + at, pg.data(), pg.size() * sizeof(int32_t));
    at += (int64_t)pg.size();
  }
  return SLORA_OK;
}

static int impl_slora_pool_owners(const slora_pool* pool, int32_t* owner) {
  clear_error();
  if (!pool || !owner) return fail(SLORA_E_INVALID, "pool_owners: NULL argument");
  memcpy(owner, pool->owner.data(), pool->owner.size() * sizeof(int32_t));
  return SLORA_OK;
}

// Host rows are read by the fetch kernel straight from pinned memory over PCIe
// (zero-copy), one workgroup per destination page; the page list is staged in pinned
// memory too, so one launch covers every page of a call with no device staging buffer
// and no per-page DMA call.
static int device_view(const void* host, const void** dev, const char* what) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof attr);
  hipError_t e = hipPointerGetAttributes(&attr, host);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(SLORA_E_INVALID, "fetch: %s is not pinned host memory (%s)", what,
                hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeHost)
    return fail(SLORA_E_INVALID, "fetch: %s is not pinned host memory (type %d)", what,
                (int)attr.type);
  if (!attr.devicePointer)
    return fail(SLORA_E_INVALID, "fetch: %s is pinned but not mapped for device access", what);
  *dev = attr.devicePointer;
  return SLORA_OK;
}

// Appends the pages of one matrix (rows x L, row-major at the device-visible src) whose
// page-table entries start at pg[first]: row k, chunk c -> pg[first + k * chunks + c].
static void add_pages(std::vector<FetchPage>* out, const uint16_t* src, int32_t rows, int32_t L,
                      int32_t P, const std::vector<int32_t>& pg, int32_t first) {
  const int32_t chunks = (L + P - 1) / P;
  for (int32_t k = 0; k < rows; ++k)
    for (int32_t c = 0; c < chunks; ++c)
      out->push_back(FetchPage{src + (int64_t)k * L + (int64_t)c * P,
                               pg[(size_t)(first + k * chunks + c)], std::min(P, L - c * P)});
}

static int impl_fetch_many(slora_pool* pool, int32_t n, const int32_t* ids,
                           const void* const* const* host_AT, const void* const* const* host_B,
                           void* side_stream, void* done_event) {
  clear_error();
  if (!pool) return fail(SLORA_E_INVALID, "fetch: pool is NULL");
  if (n < 0 || (n > 0 && !ids)) return fail(SLORA_E_INVALID, "fetch: %d adapters, ids %p", n, (const void*)ids);
  hipStream_t s = (hipStream_t)side_stream;
  // every adapter and source checked, and the whole page list built, before anything launches
  for (int32_t i = 0; i < n; ++i)
    if (pool->adapters.find(ids[i]) == pool->adapters.end())
      return fail(SLORA_E_STATE, "fetch: adapter %d is not resident", ids[i]);
  // Device views of this call's sources: the first row pointer in an allocation is looked
  // up, the others in the same allocation follow from its range (one query per buffer
  // instead of one per matrix); a matrix that would run past its allocation is refused.
  struct View {
    uintptr_t h0, h1, d0;
  };
  std::vector<View> views;
  auto view = [&](const void* host, int64_t bytes, const void** dev, const char* what) -> int {
    const uintptr_t h = reinterpret_cast<uintptr_t>(host);
    for (const View& v : views)
      if (h >= v.h0 && h < v.h1) {
        if (h + (uintptr_t)bytes > v.h1)
          return fail(SLORA_E_INVALID, "fetch: %s rows run past the end of their allocation", what);
        *dev = reinterpret_cast<const void*>(v.d0 + (h - v.h0));
        return SLORA_OK;
      }
    const int rc = device_view(host, dev, what);
    if (rc) return rc;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)host) == hipSuccess && size > 0 &&
        reinterpret_cast<uintptr_t>(base) <= h && h < reinterpret_cast<uintptr_t>(base) + size) {
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(base);
      if (h + (uintptr_t)bytes > b0 + size)
        return fail(SLORA_E_INVALID, "fetch: %s rows run past the end of their allocation", what);
      views.push_back(View{b0, b0 + size, reinterpret_cast<uintptr_t>(*dev) - (h - b0)});
    } else {
      (void)hipGetLastError();
    }
    return SLORA_OK;
  };
  std::vector<FetchPage>& d = pool->pages_scratch;
  d.clear();
  for (int32_t i = 0; i < n; ++i) {
    const AdapterRec& a = pool->adapters.find(ids[i])->second;
    if (a.rank <= 0) continue;
    if (!host_AT || !host_B || !host_AT[i] || !host_B[i])
      return fail(SLORA_E_INVALID, "fetch: host arrays of adapter %d are NULL", ids[i]);
    for (size_t p = 0; p < a.pages.size(); ++p) {
      const void* at = host_AT[i][p];
      const void* b = host_B[i][p];
      if (!at || !b) return fail(SLORA_E_INVALID, "fetch: projection %zu source NULL", p);
      if ((reinterpret_cast<uintptr_t>(at) | reinterpret_cast<uintptr_t>(b)) & 15)
        return fail(SLORA_E_INVALID, "fetch: host rows must be 16-byte aligned");
      const void *dat = nullptr, *db = nullptr;
      int rc = view(at, (int64_t)a.rank * a.d_in[p] * 2, &dat, "host_AT");
      if (rc) return rc;
      rc = view(b, (int64_t)a.rank * a.d_out[p] * 2, &db, "host_B");
      if (rc) return rc;
      const int32_t cA = (a.d_in[p] + pool->P - 1) / pool->P;
      add_pages(&d, (const uint16_t*)dat, a.rank, a.d_in[p], pool->P, a.pages[p], 0);
      add_pages(&d, (const uint16_t*)db, a.rank, a.d_out[p], pool->P, a.pages[p], a.rank * cA);
    }
  }
  if (!d.empty()) {
    FetchStage& st = pool->stage[pool->stage_next];
    if (st.pending) {  // the launch that last read this list must be done
      const hipError_t e = hipEventSynchronize(st.ev);
      if (e != hipSuccess) return hip_fail(e, "fetch: hipEventSynchronize");
      st.pending = false;
    }
    if (st.cap < (int64_t)d.size()) {
      if (st.host) (void)hipHostFree(st.host);
      st.host = nullptr;
      st.cap = 0;
      const int64_t cap = std::max<int64_t>((int64_t)d.size(), 4096);
      void* h = nullptr;
      const hipError_t e = hipHostMalloc(&h, (size_t)cap * sizeof(FetchPage), hipHostMallocDefault);
      if (e != hipSuccess) return hip_fail(e, "fetch: hipHostMalloc");
      st.host = (FetchPage*)h;
      st.cap = cap;
    }
    if (!st.ev) {
      const hipError_t e = hipEventCreateWithFlags(&st.ev, hipEventDisableTiming);
      if (e != hipSuccess) {
        st.ev = nullptr;
        return hip_fail(e, "fetch: hipEventCreate");
      }
    }
    memcpy(st.host, d.data(), d.size() * sizeof(FetchPage));
    hipError_t e = timed_fetch(st.host, (int64_t)d.size(), (uint16_t*)pool->dev, pool->P, s);
    if (e != hipSuccess) return hip_fail(e, "fetch: kernel launch");
    e = hipEventRecord(st.ev, s);
    if (e != hipSuccess) return hip_fail(e, "fetch: hipEventRecord");
    st.pending = true;
    pool->stage_next = (pool->stage_next + 1) % kFetchStages;
  }
  if (n > 0) {  // one fetch-in-flight marker for every adapter of the call
    auto mark = std::make_shared<FetchMark>();
    hipError_t e = hipEventCreateWithFlags(&mark->ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      mark->ev = nullptr;
      return hip_fail(e, "fetch: hipEventCreate");
    }
    e = hipEventRecord(mark->ev, s);
    if (e != hipSuccess) return hip_fail(e, "fetch: hipEventRecord");
    for (int32_t i = 0; i < n; ++i) pool->adapters.find(ids[i])->second.fetch = mark;
  }
  if (done_event) {
    hipError_t e = hipEventRecord((hipEvent_t)done_event, s);
    if (e != hipSuccess) return hip_fail(e, "fetch: hipEventRecord(done)");
  }
  return SLORA_OK;
}

static int impl_slora_fetch_async(slora_pool* pool, int32_t adapter_id, const void* const* host_AT,
                                  const void* const* host_B, void* side_stream, void* done_event) {
  return impl_fetch_many(pool, 1, &adapter_id, &host_AT, &host_B, side_stream, done_event);
}

}  // extern "C"

// Entry points: every C++ exception (host memory exhausted included) becomes an
// error code here, so none crosses the C ABI.
extern "C" {

int slora_pool_create(void* dev_pages, int64_t n_pages, int32_t page_elems, int32_t dtype,
                      uint64_t shuffle_seed, slora_pool** out) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_create(dev_pages, n_pages, page_elems, dtype, shuffle_seed, false, out); });
}

int slora_pool_create_ordered(void* dev_pages, int64_t n_pages, int32_t page_elems, int32_t dtype,
                              slora_pool** out) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_create(dev_pages, n_pages, page_elems, dtype, 0, true, out); });
}

int slora_pool_destroy(slora_pool* pool) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_destroy(pool); });
}

int slora_pool_info(const slora_pool* pool, int64_t* n_pages, int64_t* n_free, int32_t* page_elems,
                    int32_t* dtype) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_info(pool, n_pages, n_free, page_elems, dtype); });
}

int slora_pool_alloc_kv(slora_pool* pool, int32_t n, int32_t* out_page_ids) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_alloc_kv(pool, n, out_page_ids); });
}

int slora_pool_free_kv(slora_pool* pool, const int32_t* page_ids, int32_t n) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_free_kv(pool, page_ids, n); });
}

int slora_pool_free(slora_pool* pool, const int32_t* page_ids, int32_t n) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_free_kv(pool, page_ids, n); });
}

int slora_pool_n_free(const slora_pool* pool, int64_t* n_free) {
  return slora::guarded(__func__, [&] {
    if (!n_free) return fail(SLORA_E_INVALID, "pool_n_free: n_free is NULL");
    return impl_slora_pool_info(pool, nullptr, n_free, nullptr, nullptr);
  });
}

int slora_pool_alloc_adapter(slora_pool* pool, int32_t adapter_id, int32_t rank, int32_t n_proj,
                             const int32_t* d_in, const int32_t* d_out) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_alloc_adapter(pool, adapter_id, rank, n_proj, d_in, d_out); });
}

int slora_pool_free_adapter(slora_pool* pool, int32_t adapter_id) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_free_adapter(pool, adapter_id); });
}

int slora_pool_page_table(const slora_pool* pool, int32_t proj, int32_t n_adapters, int32_t* pt,
                          int64_t pt_cap, int64_t* pt_len, int64_t* base, int32_t* rank) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_page_table(pool, proj, n_adapters, pt, pt_cap, pt_len, base, rank); });
}

int slora_pool_owners(const slora_pool* pool, int32_t* owner) {
  return slora::guarded(__func__, [&] { return impl_slora_pool_owners(pool, owner); });
}

int slora_fetch_async(slora_pool* pool, int32_t adapter_id, const void* const* host_AT,
                      const void* const* host_B, void* side_stream, void* done_event) {
  return slora::guarded(__func__, [&] { return impl_slora_fetch_async(pool, adapter_id, host_AT, host_B, side_stream, done_event); });
}

int slora_fetch_many_async(slora_pool* pool, int32_t n, const int32_t* adapter_ids,
                           const void* const* const* host_AT, const void* const* const* host_B,
                           void* side_stream, void* done_event) {
  return slora::guarded(__func__, [&] { return impl_fetch_many(pool, n, adapter_ids, host_AT, host_B, side_stream, done_event); });
}

}  // extern "C"

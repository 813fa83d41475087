/*
 * slora.h - C ABI of the heterogeneous batched LoRA library (libslora.so, gfx950).
 *
 * What the library computes. For every token t of a mixed batch, with i = a(t)
 * the adapter that token uses, r_i its rank and s_i its scale:
 *
 *     v[t, k] = sum_j x[t, j] * A_i[j, k]                       (shrink, k < r_i)
 *     y[t, n] = y0[t, n] + s_i * sum_k v[t, k] * B_i[k, n]       (expand)
 *
 * y[t, :] = y0[t, :] bit for bit when t has no adapter (id -1) or r_i = 0.
 * Sources: "Makale Bulteni - S-LoRA", section "Iddia ve Gerceklik: S-LoRA" (one
 * batched GEMM needs one weight; the S-LoRA kernel multiplies every token of a
 * batch by its own adapter; ranks such as 8, 16, 64 coexist); the paper review
 * "S-LoRA: Serving Thousands of Concurrent LoRA Adapters", abstract and section
 * "Proposed method" (all adapters live in host memory, the active ones are
 * fetched to GPU memory on demand; base-model compute is separate, so y0 is an
 * input); the S-LoRA overview (Chinese), sections "1. Unified Paging" and
 * "2. Heterogeneous Batching" (one memory pool for adapter weights of any rank
 * and for KV-cache tensors; kernels that read non-contiguous memory directly).
 *
 * Memory model. Every device buffer (pool, page table, x, y, v, workspace) is
 * allocated and owned by the caller. The library owns host bookkeeping (the pool
 * handle) and a small pinned staging ring for work lists (16 slots, reused in
 * groups of 8 calls). All compute calls are asynchronous on the stream they are
 * given; argument validation is synchronous. A call blocks the host only when it
 * reaches a group of slots whose previous calls (8 to 16 calls back) have not
 * finished on the GPU; if that group's calls used more than one stream, the wait is
 * a device synchronization.
 *
 * Paged layout. The pool is n_pages pages of page_elems elements of one dtype.
 * A page holds one chunk of one row: adapter i's projection p occupies, for each
 * of its r rows of A^T (row k = column k of A, length d_in) ceil(d_in/P) pages,
 * then for each of its r rows of B (length d_out) ceil(d_out/P) pages. The last
 * chunk of a row whose length is not a multiple of P leaves the page tail unused.
 * KV-cache pages come from the same free list and are never read by this library.
 * Page tables are int32 arrays; adapter i's entries start at base[i] in that
 * order (A^T rows, chunks ascending; then B rows, chunks ascending).
 *
 * Errors. Every call returns SLORA_OK (0) or a negative code; slora_last_error()
 * returns a thread-local message for the last failure on the calling thread.
 * A failing call changes nothing (allocation is all-or-nothing). No C++ exception
 * leaves the library: host memory running out inside a call is SLORA_E_INVALID
 * with a message saying so.
 *
 * Threads. A pool handle is not thread-safe: one owner at a time. Compute calls
 * may run from several threads on different streams.
 */
#ifndef SLORA_H_
#define SLORA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLORA_ABI_VERSION 1

#define SLORA_OK 0
#define SLORA_E_INVALID (-1)   /* bad argument, shape, alignment or routing; host memory exhausted */
#define SLORA_E_POOL_FULL (-2) /* not enough free pages; nothing was allocated */
#define SLORA_E_STATE (-3)     /* adapter absent / already resident / fetch in flight */
#define SLORA_E_HIP (-4)       /* a HIP runtime call failed */

#define SLORA_F16 0  /* IEEE binary16 */
#define SLORA_BF16 1 /* bfloat16 */

/* Which kernel family serves which tokens (slora_routing.policy). */
/* AUTO: segment tokens -> SGMV (MFMA); per-token ids -> MBGMV, except that the ids of an
 * adapter with 4 or more of them in the call go to SGMV when SGMV runs anyway (segments)
 * or there are at least 256 such ids making at least a fifth of all per-token ids, and
 * that all ids go to SGMV when it runs and fewer than 128 would be left for MBGMV. The
 * routing changes which kernels run, not results beyond rounding. */
#define SLORA_POLICY_AUTO 0
#define SLORA_POLICY_MBGMV 1 /* every routed token -> MBGMV (segments grouped like ids) */
#define SLORA_POLICY_SGMV 2  /* every routed token -> SGMV (ids bucketed by adapter) */

typedef struct slora_pool slora_pool; /* opaque host-side handle */

/* Message for the last failing call on this thread ("" if none). Never NULL. */
const char* slora_last_error(void);

/* SLORA_ABI_VERSION of the loaded library. */
int slora_abi_version(void);

/* ------------------------------------------------------------------ unified pool
 * Unified Paging (S-LoRA overview, section "1. Unified Paging"; review, section
 * "Proposed method"): one pool of fixed-size pages shared by adapter weights of
 * any rank and by KV-cache pages, allocated from one free list. The free list is
 * shuffled with shuffle_seed, so allocations land on scattered pages, the way
 * pages of a long-running server end up.
 */

/* Create a pool over caller-owned device memory dev_pages (n_pages * page_elems
 * elements of dtype, 16-byte aligned). page_elems must be a positive multiple of
 * 8. The pool never frees dev_pages. Returns the handle in *out. */
int slora_pool_create(void* dev_pages, int64_t n_pages, int32_t page_elems, int32_t dtype,
                      uint64_t shuffle_seed, slora_pool** out);

/* A pool whose free list is not shuffled: pages are handed out in ascending id order
 * (so pages allocated together, such as one adapter's, are consecutive) and freed pages
 * are reused last-freed first. For the ablation of the unified pool (the S-LoRA
 * overview, section "S-LoRA的性能评估": S-LoRA without unified memory keeps adapters
 * and the KV cache in separate memory): an adapter-only pool of this kind stores each
 * adapter contiguously, and KV pages come from a second pool. */
int slora_pool_create_ordered(void* dev_pages, int64_t n_pages, int32_t page_elems, int32_t dtype,
                              slora_pool** out);

/* Destroy the handle (waits for this pool's fetches to finish). NULL is a no-op. */
int slora_pool_destroy(slora_pool* pool);

/* Pool geometry and the number of free pages. Any output pointer may be NULL. */
int slora_pool_info(const slora_pool* pool, int64_t* n_pages, int64_t* n_free,
                    int32_t* page_elems, int32_t* dtype);

/* Take n pages for KV cache from the shared free list; their ids go to
 * out_page_ids[n]. SLORA_E_POOL_FULL (nothing taken) if fewer than n are free. */
int slora_pool_alloc_kv(slora_pool* pool, int32_t n, int32_t* out_page_ids);

/* Return KV pages to the free list. Every id must be a KV page of this pool;
 * all-or-nothing (SLORA_E_INVALID and nothing freed on a bad or repeated id). */
int slora_pool_free_kv(slora_pool* pool, const int32_t* page_ids, int32_t n);

/* The same as slora_pool_free_kv (the name the scope of this library gives the call
 * that returns pages to the shared free list). */
int slora_pool_free(slora_pool* pool, const int32_t* page_ids, int32_t n);

/* Free pages of the pool in *n_free (slora_pool_info's n_free alone). */
int slora_pool_n_free(const slora_pool* pool, int64_t* n_free);

/* Reserve pages for adapter `adapter_id` (>= 0): rank r >= 0 (shared by its
 * projections) and n_proj projections with shapes d_in[p] x d_out[p] (multiples
 * of 8). All-or-nothing: SLORA_E_POOL_FULL when the free list is too short,
 * SLORA_E_STATE when the adapter is already resident. */
int slora_pool_alloc_adapter(slora_pool* pool, int32_t adapter_id, int32_t rank, int32_t n_proj,
                             const int32_t* d_in, const int32_t* d_out);

/* Return the adapter's pages. SLORA_E_STATE if it is not resident or if a fetch
 * into it has not finished yet (checked with hipEventQuery, never waits). */
int slora_pool_free_adapter(slora_pool* pool, int32_t adapter_id);

/* Export projection `proj`'s page table for adapters 0..n_adapters-1 into the host
 * array pt[pt_cap]: resident adapters' entries in ascending id order, in the
 * layout described above. base[i] gets the first entry (-1 when adapter i is not
 * resident or has no projection `proj`), rank[i] its rank (0 when absent).
 * *pt_len gets the number of entries written (pt may be NULL with pt_cap 0 to
 * query the length). The caller copies pt to device memory for the compute calls. */
int slora_pool_page_table(const slora_pool* pool, int32_t proj, int32_t n_adapters, int32_t* pt,
                          int64_t pt_cap, int64_t* pt_len, int64_t* base, int32_t* rank);

/* Owner of every page, for inspection: owner[p] = adapter id, -1 free, -2 KV. */
int slora_pool_owners(const slora_pool* pool, int32_t* owner);

/* Copy a resident adapter's weights from host memory into its pages, page by
 * page, asynchronously on side_stream (a hipStream_t), then record done_event (a
 * hipEvent_t, may be NULL) on it. Review, abstract and "Proposed method"; "Makale
 * Bulteni - S-LoRA", section "Iddia ve Gerceklik" (DRAM -> GPU, page by page,
 * asynchronously).
 *   host_AT[p]: pinned host memory (hipHostMalloc / torch pin_memory), r x d_in[p]
 *               row-major, row k = column k of A.
 *   host_B[p] : pinned host memory, r x d_out[p] row-major.
 * The host buffers must stay alive and unchanged until done_event completes. The
 * compute stream must wait for done_event (hipStreamWaitEvent) before a compute
 * call reads the adapter. Pages of other adapters and KV pages are never written. */
int slora_fetch_async(slora_pool* pool, int32_t adapter_id, const void* const* host_AT,
                      const void* const* host_B, void* side_stream, void* done_event);

/* slora_fetch_async for n adapters at once (one kernel launch moves every page): adapter
 * adapter_ids[i] takes its rows from host_AT[i][p] / host_B[i][p], laid out as for
 * slora_fetch_async. The S-LoRA serving loop fetches the adapters a batch needs together
 * (review, "Proposed method"). All-or-nothing: every id and source is checked before
 * anything is launched (SLORA_E_STATE for an id that is not resident). An id may appear
 * twice (its pages are written twice with the same bytes). The page list is staged in
 * library-owned pinned memory; a fifth call in a row may wait on the host for the
 * first one's launch to finish before it reuses that list. */
int slora_fetch_many_async(slora_pool* pool, int32_t n, const int32_t* adapter_ids,
                           const void* const* const* host_AT, const void* const* const* host_B,
                           void* side_stream, void* done_event);

/* ------------------------------------------------------------------ adapter residency
 * All adapters stay in host memory; those running requests use are fetched to the pool
 * on demand (review, abstract and "Proposed method"), and when the active set outgrows
 * the pool adapters are swapped over PCIe ("Makale Bulteni - S-LoRA", section "Iddia
 * ve Gerceklik": thrashing shows in the tail latency). A residency manager owns the
 * adapters of one pool (the caller must not allocate or free adapters of that pool
 * itself): each resident adapter has a pin count (pinned = in use); acquiring an
 * adapter that is not resident allocates its pages, evicting unpinned adapters in
 * least-recently-used order when the free list is short (never one whose fetch may
 * still be in flight; recency = the adapter's last release or its prefetch), and
 * reports that the caller must fetch it (slora_fetch_async)
 * before any compute call reads it. Page tables change with every allocation or
 * eviction: export them again (slora_pool_page_table) before the next compute call.
 * Host only; a manager is not thread-safe. */
typedef struct slora_residency slora_residency;
typedef struct {
  int32_t resident, pinned;  /* adapters resident now, and pinned among them */
  int64_t hits, misses;      /* acquires that found the adapter resident / had to allocate it */
  int64_t evictions, prefetches;
} slora_residency_stats;

/* A manager for `pool`; every adapter has n_proj projections d_in[p] x d_out[p]. */
int slora_residency_create(slora_pool* pool, int32_t n_proj, const int32_t* d_in,
                           const int32_t* d_out, slora_residency** out);
/* Frees the manager (not the adapters: they stay resident in the pool). */
int slora_residency_destroy(slora_residency* res);

/* Pin adapter `adapter_id` of rank `rank` for use. *needs_fetch = 1 when it was not
 * resident and its pages were just allocated (fetch before use), else 0. Adapters
 * evicted to make room are written to evicted[evicted_cap] (*n_evicted of them).
 * SLORA_E_POOL_FULL, with nothing evicted or allocated, when free pages plus the pages
 * of evictable adapters are not enough. SLORA_E_INVALID when it is resident with
 * another rank. */
int slora_residency_acquire(slora_residency* res, int32_t adapter_id, int32_t rank,
                            int32_t* needs_fetch, int32_t* evicted, int32_t evicted_cap,
                            int32_t* n_evicted);
/* Make an adapter resident ahead of use without pinning it, only if the free list holds
 * its pages (evicts nothing); *needs_fetch = 1 when it was allocated now. */
int slora_residency_prefetch(slora_residency* res, int32_t adapter_id, int32_t rank,
                             int32_t* needs_fetch);
/* Unpin (SLORA_E_STATE if not pinned); at zero pins the adapter becomes evictable. */
int slora_residency_release(slora_residency* res, int32_t adapter_id);
int slora_residency_info(const slora_residency* res, slora_residency_stats* stats);
/* *pins = the adapter's pin count, or -1 when it is not resident. */
int slora_residency_is_resident(const slora_residency* res, int32_t adapter_id, int32_t* pins);

/* ------------------------------------------------------------------ admission
 * Continuous batching over the unified pool (the continuous-batching page, sections
 * "Surekli Gruplama (Continuous Batching) Nedir ve Nasil Calisir?" and "vLLM
 * Zamanlayicisi: Istekleri Dinamik Olarak Yonetme"; review, "Proposed method": early-
 * abort scheduling on the unified pool). Requests wait in a FIFO queue. Each step:
 *   1. running requests that produced max_new_tokens leave (their KV pages are freed,
 *      their adapter unpinned); waiting or running requests past their deadline step
 *      are aborted the same way (SLORA_ABORT_DEADLINE);
 *   2. every running request decodes one token and takes kv_pages_per_token more KV
 *      pages; while the pool cannot give them all, the most recently admitted running
 *      request is aborted (SLORA_ABORT_POOL_FULL);
 *   3. waiting requests are admitted in order while the step's token budget
 *      (max_batch_tokens), max_running and the pool (the prompt's KV pages, and the
 *      adapter's pages through the residency manager, evicting unpinned adapters) allow;
 *      the first that does not fit stops admission. Its prompt is the step's prefill.
 * The step's batch is a ready slora_routing: admitted prompts as segments, then one
 * decode token per running request. One token's KV takes kv_pages_per_token pages of
 * the pool (a page holds one token's K or V vector for one layer). */
typedef struct slora_sched slora_sched;
typedef struct {
  int32_t kv_pages_per_token; /* >= 1 */
  int32_t max_batch_tokens;   /* tokens per step (prefill + decode), >= max_running */
  int32_t max_running;        /* running requests at most, >= 1 */
} slora_sched_config;
#define SLORA_ABORT_DEADLINE 1  /* the request's deadline step passed */
#define SLORA_ABORT_POOL_FULL 2 /* its next token's KV pages did not fit the pool */
/* One step's batch. Every pointer points into the scheduler and stays valid until its
 * next step or destroy. */
typedef struct {
  int64_t step;
  int32_t n_tokens, n_segments;
  const int32_t* seg_offsets;     /* [n_segments + 1] */
  const int32_t* seg_adapter;     /* [n_segments] */
  const int32_t* token_adapter;   /* [n_tokens - seg_offsets[n_segments]] */
  const int64_t* seg_request;     /* request of each segment */
  const int64_t* token_request;   /* request of each decode token */
  int32_t n_fetch;                /* adapters allocated this step: fetch before the compute call */
  const int32_t* fetch;
  int32_t n_evicted;              /* adapters evicted this step */
  const int32_t* evicted;
  int32_t n_finished;             /* requests that left this step, done */
  const int64_t* finished;
  int32_t n_aborted;              /* requests aborted this step, with the reason of each */
  const int64_t* aborted;
  const int32_t* abort_reason;
  int32_t n_waiting, n_running;   /* after the step */
  int64_t free_pages;             /* of the pool, after the step */
} slora_sched_batch;

/* A scheduler over `pool`, which holds the KV pages; `res` (may be NULL: adapters are
 * then the caller's business) manages the adapters requests use, in its own pool: the
 * same pool (unified paging: adapters and KV compete for one free list) or another one
 * (adapters and KV in separate memory). */
int slora_sched_create(slora_pool* pool, slora_residency* res, const slora_sched_config* cfg,
                       slora_sched** out);
/* Frees the running requests' KV pages and unpins their adapters, then the scheduler. */
int slora_sched_destroy(slora_sched* sched);
/* Queue a request: adapter_id (-1 = none) of rank `rank`, a prompt of prompt_len tokens
 * (<= max_batch_tokens), at most max_new_tokens output tokens, aborted once a step past
 * deadline_step begins (-1 = no deadline). SLORA_E_STATE if the id is queued or running. */
int slora_sched_submit(slora_sched* sched, int64_t request_id, int32_t adapter_id, int32_t rank,
                       int32_t prompt_len, int32_t max_new_tokens, int64_t deadline_step);
/* The request is done now (an end-of-sequence token, or the client went away): if
 * running, its KV pages are freed and its adapter unpinned; if waiting, it is dropped. */
int slora_sched_finish(slora_sched* sched, int64_t request_id);
/* Plan the next step (see above) into *batch. */
int slora_sched_step(slora_sched* sched, slora_sched_batch* batch);
/* KV pages a running request holds, in allocation order (pages[cap], *n of them). */
int slora_sched_request_pages(const slora_sched* sched, int64_t request_id, int32_t* pages,
                              int32_t cap, int32_t* n);

/* ------------------------------------------------------------------ compute */

/* One projection of the batch. All pointers are read only. */
typedef struct {
  const void* pool;          /* DEVICE: the pool's pages (as given to slora_pool_create) */
  int64_t n_pages;           /* pool size in pages; page ids >= n_pages read as NaN */
  int32_t page_elems;        /* P */
  int32_t dtype;             /* SLORA_F16 | SLORA_BF16 (x, y and pool) */
  int32_t d_in, d_out;       /* multiples of 8 */
  const int32_t* page_table; /* DEVICE int32 [page_table_len] */
  int64_t page_table_len;
  int32_t n_adapters;
  const int64_t* base;       /* HOST [n_adapters]: first page-table entry, -1 = not resident */
  const int32_t* rank;       /* HOST [n_adapters]: 0 allowed (delta is zero) */
  const float* scale;        /* HOST [n_adapters]: s_i (alpha / r_i in the standard form) */
  int32_t r_max;             /* row stride of v; >= every rank a routed token uses, <= 128 */
} slora_lora;

/* Which adapter each token uses (all HOST arrays). Tokens [0, seg_offsets[S])
 * are routed by segments (a request's contiguous tokens share one adapter);
 * tokens [seg_offsets[S], n_tokens) by one id each. Ids are in [-1, n_adapters). */
typedef struct {
  int32_t n_tokens;
  int32_t n_segments;           /* S >= 0 */
  const int32_t* seg_offsets;   /* [S + 1], seg_offsets[0] = 0, nondecreasing; NULL if S = 0 */
  const int32_t* seg_adapter;   /* [S] */
  const int32_t* token_adapter; /* [n_tokens - seg_offsets[S]], -1 = no adapter */
  int32_t policy;               /* SLORA_POLICY_* */
} slora_routing;

/* Device workspace bytes a compute call with these arguments needs (>= 256). The
 * workspace must be zero-filled once when it is allocated and then left to the
 * library: it holds per-group completion counters tagged with a call epoch, which
 * need no reset between calls. Calls that share a workspace must be ordered (one
 * stream, or synchronized streams); calls on different workspaces may overlap. */
int slora_workspace_size(const slora_lora* lora, const slora_routing* routing, int64_t* bytes);

/* Shrink only: v[t, k] (fp32, DEVICE [n_tokens x r_max]) for routed tokens and
 * k < rank; other entries of v are left unchanged. x: DEVICE [n_tokens x d_in]. */
int slora_shrink(const slora_lora* lora, const slora_routing* routing, const void* x, float* v,
                 void* ws, int64_t ws_bytes, void* stream);

/* Expand only, in place: y (DEVICE [n_tokens x d_out], holds y0 on entry) gets
 * y0 + s * v B for routed tokens, rounded once (round to nearest even) from
 * fp32. Rows of unrouted tokens are not touched. */
int slora_expand(const slora_lora* lora, const slora_routing* routing, const float* v, void* y,
                 void* ws, int64_t ws_bytes, void* stream);

/* Shrink + expand in one call (v lives in the workspace). y holds y0 on entry.
 * Each family runs in one launch, and a call with both usually runs both in one:
 * decode tokens' shrink workgroups publish v per group and the group's expand
 * workgroups wait for it; prefill segments' shrink workgroups write their partial sums
 * of a tile and a flag, and the tile's expand workgroups wait for every flag of the
 * tile (bounded waits; see slora_workspace_status). Every shrink workgroup of a launch
 * comes before its expand workgroups in dispatch order and never waits, so the waits
 * end. The work
 * list is read by the kernels from a pinned host staging ring owned by the library.
 * Two such launches resident on one device at once could each hold the compute
 * slots the other's shrink workgroups need, so the library orders them: a call
 * whose launches go to another stream than the previous such call on the device
 * first makes its stream wait for the work queued on that previous stream (an
 * event recorded there; if that stream no longer exists, a device
 * synchronization). Launches from other processes sharing the device are not
 * ordered. */
int slora_apply(const slora_lora* lora, const slora_routing* routing, const void* x, void* y,
                void* ws, int64_t ws_bytes, void* stream);

/* slora_apply over several projections of one batch at once (for instance a layer's q,
 * k, v and o): loras[p] describes projection p, which reads xs[p] (DEVICE [n_tokens x
 * d_in]) and updates ys[p] (DEVICE [n_tokens x d_out], y0 on entry) as slora_apply
 * would. The results are slora_apply's bit for bit for decode groups and for one
 * projection; with segment tiles and several projections the launch may split the
 * segment shrink into fewer k-ranges (its other projections' work fills the device), so
 * the same fp32 terms are added in another grouping and outputs agree with
 * slora_apply's to rounding (the intermediate v, which the segment expand reads in the
 * storage type, can round the other way, and y's own rounding can then land one unit
 * away). Repeated calls give the same bits.
 * Every loras[p] has the same pool, n_pages,
 * page_elems, dtype, d_in, d_out, n_adapters, r_max and page_table_len as loras[0], and
 * equal base, rank and scale arrays: the projections share the routing, the adapters and
 * the layout of their page tables (each its own page_table). A request's adapter applies
 * to every projection it adapts, and all adapter weights live in the one pool (the
 * S-LoRA overview, section "1. Unified Paging"); running several projections in one
 * launch is this library's own step, not one the pages give. A projection that differs
 * is refused with SLORA_E_INVALID before anything runs. The call plans once and runs the
 * work of all n_proj (1..8) projections in one launch (or two, when its segments get a
 * launch per rank class, as in slora_apply), which saves every launch's fixed ramp and
 * tail but one. ws: n_proj regions of slora_workspace_size_multi / n_proj bytes each,
 * zero-filled once; give-ups are read with slora_workspace_status(ws, ...). */
int slora_workspace_size_multi(int32_t n_proj, const slora_lora* loras, const slora_routing* routing,
                               int64_t* bytes);
int slora_apply_multi(int32_t n_proj, const slora_lora* loras, const slora_routing* routing,
                      const void* const* xs, void* const* ys, void* ws, int64_t ws_bytes,
                      void* stream);

/* Ablation baseline "S-LoRA with conventional batched matmul" (the S-LoRA overview,
 * section "S-LoRA的性能评估", comparison of S-LoRA variants): the same function as
 * slora_apply, computed the conventional way. Every request (a segment, or a decode
 * token on its own) gets a contiguous copy of its adapter, gathered out of the pool and
 * padded with zero rows to the largest rank of the batch, and one padded batched GEMM
 * (the MFMA segment kernels over the copies, every adapter at the padded rank) produces
 * y. Results agree with slora_apply within rounding. The workspace (caller-owned, size
 * from slora_gathered_workspace_size, zero-filled once) holds the segment kernels' own
 * workspace first, then the copies: n_requests x r_pad x (ceil(d_in/P) + ceil(d_out/P))
 * pages. The routing's policy is ignored. The segment kernels run as in slora_apply (one
 * launch whose expand workgroups wait for their tile's shrink workgroups), so a give-up
 * is read with slora_workspace_status on this workspace. */
int slora_gathered_workspace_size(const slora_lora* lora, const slora_routing* routing,
                                  int64_t* bytes);
int slora_apply_gathered(const slora_lora* lora, const slora_routing* routing, const void* x,
                         void* y, void* ws, int64_t ws_bytes, void* stream);

/* slora_apply for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments minus
 * the workspace, same kernels, same results bit for bit. The workspace is a static
 * device array of the library, 64 MiB on every GPU it runs on, held until the process
 * ends; a call that needs more (256 + n_tokens * r_max * 8 bytes + the prefill
 * partial sums + n_tokens * 64 bytes of prefill flags, each part rounded up to 256
 * bytes) is refused with SLORA_E_INVALID before anything runs, and so is one whose
 * work list would outgrow its 1 MiB staging slot. The call allocates no
 * device or pinned memory, except on its first call on a device, which also creates the
 * library's staging ring if no compute call has yet, resolves the array's address and
 * clears the array on `stream`. Every call on a GPU shares that GPU's array, which keeps
 * the last call's contents; the library orders the calls it is given (a call on another
 * stream than the previous one first waits for that stream's queued work), so calls
 * that overlap on one GPU (another process, or work outside the library writing the
 * array) race. Give-ups are read with slora_workspace_status(NULL, ...). */
int slora_apply_noalloc(const slora_lora* lora, const slora_routing* routing, const void* x,
                        void* y, void* stream);

/* Status of the slora_apply calls that used workspace ws since the previous status
 * read, once the work on `stream` has finished (this call synchronizes the stream):
 * 0 = clean; 1 = in at least one of them a workgroup gave up waiting for v (or a
 * prefill tile's partial sums) that another workgroup of the same launch should have
 * published (that call's results are not valid). The give-up is sticky in the workspace header until this
 * call reads it, and reading clears it. ws = NULL reads the current device's static
 * scratch of slora_apply_noalloc (0 if no such call has run on it). */
int slora_workspace_status(void* ws, void* stream, int32_t* status);

/* Bound of the waits in slora_apply's launches: an expand wave polls for its v (decode
 * tokens) or for its tile's flags (prefill segments) at most `polls` times before it
 * gives up (see slora_workspace_status). polls = 0 restores the default
 * (2^20 polls, far beyond any wait a valid launch has). Applies to launches made after
 * the call, on every device. Tests of the give-up path set a small bound (1 poll: waves
 * that find v not yet published give up at once, so the launch ends with invalid
 * results and a set status instead of waiting). */
int slora_set_wait_limit(int32_t polls);

/* Kernel timing for benchmarks. While enabled (on != 0), every kernel a compute
 * call launches carries two HIP events that the launch itself records on the call's
 * stream when the kernel starts and when it ends (hipExtLaunchKernel), so a timed
 * interval spans the kernel alone.
 * Recorded launches accumulate across enable / disable until slora_timing_read
 * returns and clears them, so a caller can time a sample of its calls. Kernel ids: SLORA_K_MBGMV_SHRINK,
 * SLORA_K_MBGMV_EXPAND, SLORA_K_SGMV_SHRINK, SLORA_K_SGMV_EXPAND (the separate launches of
 * slora_shrink and slora_expand), SLORA_K_MBGMV_FUSED and SLORA_K_SGMV_FUSED (shrink and expand
 * in one launch, as slora_apply runs each family), SLORA_K_MIXED_FUSED (a call with both
 * families whose segments fit one launch: everything in that launch). */
#define SLORA_K_MBGMV_SHRINK 0
#define SLORA_K_MBGMV_EXPAND 1
#define SLORA_K_SGMV_SHRINK 2
#define SLORA_K_SGMV_EXPAND 3
#define SLORA_K_MBGMV_FUSED 4
#define SLORA_K_GATHER 5 /* slora_apply_gathered's copy of the adapters out of the pool */
#define SLORA_K_FETCH 6  /* slora_fetch_async / slora_fetch_many_async's copy into the pool */
#define SLORA_K_SGMV_FUSED 7
#define SLORA_K_MIXED_FUSED 8 /* both families of one slora_apply in one launch */
#define SLORA_K_MULTI_FUSED 9 /* the launch(es) of one slora_apply_multi, timed as one interval */
#define SLORA_K_COUNT 10
int slora_timing_enable(int32_t on);

/* Waits for the recorded events, then writes per kernel id the number of timed
 * launches and their summed duration in milliseconds (arrays of n_kernels entries,
 * n_kernels <= SLORA_K_COUNT), and clears the counters. */
int slora_timing_read(int32_t n_kernels, int64_t* launches, double* total_ms);

/* Every timed launch since the last read, in launch order: kernel[i] its kernel id,
 * ms[i] its duration (arrays of cap entries); *n gets the count (SLORA_E_INVALID,
 * nothing cleared, if it exceeds cap). Waits for the events, then clears them. The
 * event pairs are created by slora_timing_enable (512 of them), so timed compute
 * calls create none unless more launches are timed before a read. */
int slora_timing_read_all(int64_t cap, int32_t* kernel, double* ms, int64_t* n);

/* Work lists a call with these arguments would run, for inspection and tests
 * (host only; validates exactly like slora_apply, launches nothing). Groups come
 * in dispatch order; for group g, info[5g .. 5g+4] = {family (0 MBGMV, 1 SGMV),
 * first slot in tokens[], token count, first page-table entry, rank}. tokens gets
 * the routed token ids grouped (n_tokens entries suffice). *n_groups gets the
 * group count; SLORA_E_INVALID if it exceeds info_cap. */
int slora_plan_inspect(const slora_lora* lora, const slora_routing* routing, int32_t* n_groups,
                       int32_t* info, int32_t info_cap, int32_t* tokens);

#ifdef __cplusplus
}
#endif

#endif /* SLORA_H_ */

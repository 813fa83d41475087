// Internal declarations shared by the host code and the HIP kernels of libslora.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "slora.h"

namespace slora {

// ---------------------------------------------------------------- errors
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char* what);
void clear_error();

// ---------------------------------------------------------------- work lists
constexpr int kMaxRank = 128;       // largest rank the kernels accept (r_max <= kMaxRank)
constexpr int kMbGroup = 4;         // MBGMV: tokens per group (one read of the adapter per group)
constexpr int kMbShrinkRows = 8;    // MBGMV shrink: A^T rows per workgroup (4 waves x 2 rows)
constexpr int kMbExpandTok = 2;     // MBGMV expand: tokens per workgroup
constexpr int kMbWaveCols = 512;    // MBGMV expand: output columns per wave (64 lanes x 8)
constexpr int kMbRowsPerWave = 16;  // MBGMV expand: B rows a wave keeps in flight
constexpr int kSgTile = 64;         // SGMV: tokens per tile
constexpr int kSgSplitTiles = 64;    // SGMV: tiles of ranks <= 64 and > 64, each, for separate launches
constexpr int kAutoSgmvTok = 4;     // AUTO: an adapter's per-token ids go to SGMV from this many
constexpr int kAutoSgmvBatch = 256; // AUTO: ... when at least this many such tokens (or segments run)
constexpr int kAutoSgmvShare = 4;   // ... and they are at least 1 / (1 + this) of the per-token ids
constexpr int kAutoMbgmvMin = 128;  // AUTO: fewer per-token ids left for MBGMV join SGMV when it runs
constexpr int kSgMaxSplit = 8;      // SGMV shrink: most k-ranges d_in is cut into

// k-ranges the SGMV shrink may cut d_in into (each at least 256 long).
inline int sg_max_split(int d_in) {
  const int s = d_in / 256;
  return s < 1 ? 1 : s > kSgMaxSplit ? kSgMaxSplit : s;
}
// Row stride of the SGMV partial v in the workspace (16-byte rows).
inline int sg_v_stride(int r_max) { return (r_max + 3) / 4 * 4; }

// Expand waves that split one column slice's rows: 1, 2 or 4 (4 waves per workgroup).
inline int mb_split(int rank) { return rank <= 16 ? 1 : rank <= 32 ? 2 : 4; }

// One MBGMV work item (one workgroup), 32 bytes, read by the kernel straight from
// the pinned staging buffer. Token ids are inline so a workgroup needs one load to
// know all it has to read.
struct MbItem {
  int32_t tok[kMbGroup];  // token ids (n_tok() of them)
  int32_t pt_base;        // page-table entry of the adapter's A^T row 0, chunk 0
  float scale;
  int16_t part;           // shrink: row block; expand: column tile
  uint8_t rank;           // 1 .. kMaxRank
  uint8_t info;           // bits 0-2: n_tok; bit 3: role (0 shrink, 1 expand); bits 4-6: split
  int32_t pad;
  __host__ __device__ int n_tok() const { return info & 7; }
  __host__ __device__ int role() const { return (info >> 3) & 1; }
  __host__ __device__ int split() const { return (info >> 4) & 7; }  // expand: mb_split(rank)
  __host__ __device__ static uint8_t pack_info(int n_tok, int role, int split) {
    return (uint8_t)(n_tok | (role << 3) | (split << 4));
  }
};
static_assert(sizeof(MbItem) == 32, "MbItem layout");
static_assert(kMaxRank <= 255, "rank is stored in 8 bits");

// One SGMV tile: up to kSgTile tokens of one adapter. 32 bytes.
struct SgTile {
  int32_t tok_begin;  // first index into the token list
  int32_t n_tok;
  int32_t pt_base;
  int32_t rank;
  float scale;
  int32_t first_tok;  // >= 0: the tokens are first_tok + [0, n_tok) (a segment); -1: the list
  int32_t pad[2];
};
static_assert(sizeof(SgTile) == 32, "SgTile layout");

// Geometry of one projection, as the kernels see it.
struct Geom {
  const uint16_t* pool;
  int64_t n_pages;
  int32_t P;        // page elements
  int32_t dtype;    // SLORA_F16 | SLORA_BF16
  int32_t d_in, d_out;
  int32_t cA, cB;   // pages per A^T row, per B row
  const int32_t* pt;
  int32_t r_max;
};

// Host plan of one call, built straight into a pinned staging buffer:
// [MbItem x n_mb][SgTile x n_sg][int32 tokens x n_tok]
struct PlanView {
  MbItem* mb = nullptr;
  int32_t n_mb = 0, n_mb_shrink = 0, n_groups = 0;
  SgTile* sg = nullptr;
  int32_t n_sg = 0;
  int32_t* tok = nullptr;
  int32_t n_tok = 0;
  int32_t n_routed = 0;
  int32_t mb_max_tok = 0;
  int32_t sg_max_rank = 0;
};

// Scratch the planner reuses between calls (thread-local, grows only).
struct PlanScratch {
  std::vector<int32_t> mb_ad, mb_in, sg_ad, sg_in;  // kept (adapter, token) pairs in token order
  std::vector<int32_t> mb_tok, sg_tok;  // the same tokens bucketed by adapter (ascending id)
  std::vector<int32_t> grp;    // MBGMV groups: (index into mb_tok, count, adapter) triples
  std::vector<int32_t> tiles;  // SGMV tiles: (first token or index into sg_tok, count, adapter, listed)
  std::vector<int32_t> order, tile_order, tiles_sorted, used, hist, seen;
  std::vector<int32_t> cnt;    // per adapter; all zero between calls
  std::vector<uint64_t> bits;
};

// Validate, group and count; returns the bytes the plan needs, or a negative
// SLORA_E_* code. counts gets the sizes.
int64_t plan_bytes(const slora_lora* L, const slora_routing* R, PlanScratch* sc, PlanView* counts);
// Write the plan into buf (plan_bytes bytes, 64-byte aligned) from the state plan_bytes left.
void plan_write(const slora_lora* L, const slora_routing* R, PlanScratch* sc, void* buf,
                PlanView* out);

// Workspace (device, caller-owned, zero-filled once at allocation):
//   [0, 256): header: uint64, nonzero once a fused call's wait gave up (sticky until
//             slora_workspace_status reads and clears it)
//   v_off: MBGMV v as uint64 words [n_tokens x r_max]: (tag << 32) | fp32 bits
//   sg_off: SGMV partial v, fp32 [sg_max_split(d_in)][n_tokens x sg_v_stride(r_max)]
//   flg_off: SGMV shrink flags, uint32 [n_tokens x 2 x kSgMaxSplit] (at most one tile per
//            token, at most two row blocks per tile)
constexpr int64_t kHeaderBytes = 256;
struct WsLayout {
  int64_t v_off, sg_off, flg_off, total;
};
WsLayout ws_layout(const slora_lora* L, const slora_routing* R);

// slora_apply on the current device's static scratch (api.cpp): ordered after the previous
// such call on the device, and a plan that would need a larger staging slot is an error.
int apply_shared(const slora_lora* L, const slora_routing* R, const void* x, void* y, void* ws,
                 int64_t ws_bytes, void* stream);
// The current device's static scratch (noalloc.hip): *ptr its device address, or nullptr
// when no allocation-free call has resolved it on this device yet; *bytes its size.
// Resolves nothing itself.
int shared_scratch(void** ptr, int64_t* bytes);

// ---------------------------------------------------------------- pool queries (pool.cpp)
// Pages adapter `id` holds (0 if not resident) and whether a fetch into it may still be
// in flight (its event not yet complete). Host only; returns SLORA_OK or an error code.
int pool_adapter_state(const slora_pool* pool, int32_t id, int64_t* pages, bool* busy);
// Pages an adapter of this rank would take for projections d_in[p] x d_out[p].
int64_t pool_adapter_need(const slora_pool* pool, int32_t rank, int32_t n_proj, const int32_t* d_in,
                          const int32_t* d_out);

// ---------------------------------------------------------------- launchers
// Optional HIP events that the launch itself records at the kernel's start and end
// (hipExtLaunchKernel), so a timed interval holds the kernel and nothing else.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
// One launch over items (role per item; `shrinks` / `expands` say which roles
// occur). tag != 0 makes it a fused apply: v is the workspace's tagged words,
// shrink items write them and expand items poll them. tag == 0: v is plain fp32.
// spin_limit: polls an expand wave makes for its v before it gives up (fused only).
constexpr int32_t kDefaultSpinLimit = 1 << 20;
hipError_t launch_mbgmv(const Geom& g, const MbItem* items, int32_t n_items, bool shrinks,
                        bool expands, int32_t max_tok, const void* x, void* v, void* y,
                        uint32_t tag, unsigned long long* err, int32_t spin_limit, hipStream_t s,
                        const LaunchEvents& ev = LaunchEvents());
// Zero `bytes` (a multiple of 16) of device memory with a kernel.
hipError_t launch_zero(void* p, int64_t bytes, hipStream_t s);
// SGMV shrink over ksplit (<= kSgMaxSplit) k-ranges of kc (a multiple of 128)
// elements: range ks writes its partial sums to vpart + ks * split_stride, rows of
// v_stride floats per token. The expand adds the ksplit partials in range order.
// slots: shrink workgroups the device holds at once (sgmv_shrink_resident); n_proj:
// projections whose tiles the launch runs.
struct SgSplit {
  int32_t ksplit, kc;
};
SgSplit sg_split(int32_t d_in, int32_t n_tiles, int32_t slots, int32_t n_proj = 1);
// Workgroups of the shrink template for ranks up to max_rank that fit on the current
// device at once (0 if the runtime cannot say).
int sgmv_shrink_resident(int32_t max_rank, int32_t dtype);
hipError_t launch_sgmv_shrink(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit, int32_t kc,
                              const void* x, float* vpart, int32_t v_stride, int64_t split_stride,
                              hipStream_t s, const LaunchEvents& ev = LaunchEvents());
hipError_t launch_sgmv_expand(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit,
                              const float* vpart, int32_t v_stride, int64_t split_stride, void* y,
                              hipStream_t s, const LaunchEvents& ev = LaunchEvents());

// Shrink and expand of an apply call in one launch: shrink items write their partial sums
// and then their flag words (one per shrink item, at most 2 * ksplit per tile); expand
// items wait for their tile's flags (spin_limit polls, a give-up recorded in *err).
// v_stride % 4 == 0; tiles in descending rank (host-readable: the pinned work list).
// With n_mb > 0 the call's MBGMV items (shrink items first, as launch_mbgmv takes them,
// v_mb their tagged v) run in the same launch: every shrink item of both families
// before every expand item.
hipError_t launch_sgmv_fused(const Geom& g, const int32_t* tok, const SgTile* tiles,
                             int32_t n_tiles, int32_t max_rank, int32_t ksplit, int32_t kc,
                             const void* x, float* vpart, int32_t v_stride, int64_t split_stride,
                             uint32_t* flags, uint32_t tag, int32_t spin_limit,
                             unsigned long long* err, void* y, hipStream_t s,
                             const LaunchEvents& ev = LaunchEvents(),
                             const MbItem* mb_items = nullptr, int32_t n_mb = 0,
                             int32_t n_mb_shrink = 0, int32_t mb_max_tok = 0, void* v_mb = nullptr);

// One projection of a launch over several projections of one batch: its page table, x,
// y (holding y0) and its workspace region's MBGMV v, segment partial sums and flags.
constexpr int kMaxProj = 8;
struct ProjIO {
  const int32_t* pt;
  const void* x;
  void* y;
  void* v_mb;
  float* vpart;
  uint32_t* flags;
};

// The apply of n_proj projections (shared plan: the same routing, ranks and page-table
// layout, one ProjIO each) in one launch: MBGMV items and segment tiles of every
// projection, every shrink item before every expand item. err: the give-up word of the
// first projection's workspace region. Tiles in descending rank, as launch_sgmv_fused.
hipError_t launch_multi_fused(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit, int32_t kc,
                              int32_t v_stride, int64_t split_stride, const ProjIO* io,
                              int32_t n_proj, uint32_t tag, int32_t spin_limit,
                              unsigned long long* err, hipStream_t s, const LaunchEvents& ev,
                              const MbItem* mb_items, int32_t n_mb, int32_t n_mb_shrink,
                              int32_t mb_max_tok);

// Ablation baseline: copy each request's adapter out of the pool into contiguous,
// rank-padded memory (gather.hip). One entry per request.
struct GatherReq {
  int32_t pt_base;  // the adapter's first page-table entry
  int32_t rank;     // its rank (rows at or past it are zero in the copy)
};
hipError_t launch_gather(const Geom& g, const GatherReq* reqs, int32_t n_req, int32_t r_pad,
                         void* dst, int32_t* dst_pt, hipStream_t s, const LaunchEvents& ev);

// Adapter fetch (fetch.hip): one workgroup per destination page, the page list read by
// the kernel from pinned host memory. 16 bytes per page.
struct FetchPage {
  const uint16_t* src;  // device-visible address of the page's first element in pinned host rows
  int32_t page;         // destination pool page
  int32_t len;          // elements to copy (<= page_elems; the rest of the page is left as is)
};
static_assert(sizeof(FetchPage) == 16, "FetchPage layout");
hipError_t launch_fetch(const FetchPage* pages, int64_t n, uint16_t* pool, int32_t page_elems,
                        hipStream_t s, const LaunchEvents& ev = LaunchEvents());
// launch_fetch, timed as SLORA_K_FETCH while kernel timing is on (api.cpp).
hipError_t timed_fetch(const FetchPage* pages, int64_t n, uint16_t* pool, int32_t page_elems,
                       hipStream_t s);

}  // namespace slora

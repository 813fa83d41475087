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
// Granularity of the work lists (the planner and the kernels agree on these).
constexpr int kMaxRank = 128;     // largest rank the kernels accept (r_max <= kMaxRank)
constexpr int kMbGroup = 8;       // MBGMV: tokens per group (one read of the adapter per group)
constexpr int kMbShrinkRows = 8;  // MBGMV shrink: A^T rows per workgroup (4 waves x 2 rows)
constexpr int kMbExpandCols = 1024;  // MBGMV expand: output columns per workgroup (2 waves x 512)
constexpr int kSgTile = 64;       // SGMV: tokens per tile (M of the MFMA tiles)
constexpr int kSgExpandCols = 256;   // SGMV expand: output columns per workgroup

// One group of tokens that share an adapter (MBGMV group or SGMV tile). 32 bytes.
struct GroupDesc {
  int32_t tok_begin;  // first index into the token list
  int32_t n_tok;      // tokens in the group (1..kMbGroup or 1..kSgTile)
  int32_t pt_base;    // page-table entry of the adapter's A^T row 0, chunk 0
  int32_t rank;       // r (>= 1)
  float scale;        // s
  int32_t pad0, pad1, pad2;
};
static_assert(sizeof(GroupDesc) == 32, "GroupDesc layout");

// (group, block) work item: row block for shrink kernels.
struct Item {
  int32_t group;
  int32_t block;
};

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

// Host-side plan; copied as one blob into the workspace.
struct Plan {
  std::vector<int32_t> tok;           // token ids, grouped
  std::vector<GroupDesc> mb_groups;   // MBGMV groups (rank-descending order)
  std::vector<Item> mb_shrink;        // (group, row block)
  std::vector<GroupDesc> sg_tiles;    // SGMV tiles (rank-descending order)
  int32_t n_routed = 0;
};

// Byte offsets of the plan sections inside the workspace (after v).
struct PlanLayout {
  int64_t v_off, v_bytes;
  int64_t tok_off, mbg_off, mbs_off, sgt_off;
  int64_t blob_off, blob_bytes;  // [blob_off, blob_off + blob_bytes) is copied from the host
  int64_t total;
};

int validate_and_plan(const slora_lora* L, const slora_routing* R, Plan* plan);
int64_t workspace_bound(const slora_lora* L, const slora_routing* R);
PlanLayout layout_plan(const slora_lora* L, const slora_routing* R, const Plan& p);

// ---------------------------------------------------------------- launchers
hipError_t launch_mbgmv_shrink(const Geom& g, const int32_t* tok, const GroupDesc* groups,
                               const Item* items, int32_t n_items, const void* x, float* v,
                               hipStream_t s);
hipError_t launch_mbgmv_expand(const Geom& g, const int32_t* tok, const GroupDesc* groups,
                               int32_t n_groups, const float* v, void* y, hipStream_t s);
hipError_t launch_sgmv_shrink(const Geom& g, const int32_t* tok, const GroupDesc* tiles,
                              int32_t n_tiles, const void* x, float* v, hipStream_t s);
hipError_t launch_sgmv_expand(const Geom& g, const int32_t* tok, const GroupDesc* tiles,
                              int32_t n_tiles, const float* v, void* y, hipStream_t s);

constexpr int kFetchMaxPages = 240;
struct FetchArgs {
  const uint16_t* src;  // device-visible pointer to pinned host rows (rows x L)
  uint16_t* pool;
  int32_t P;
  int32_t L;            // row length
  int32_t chunks;       // pages per row
  int32_t e0;           // first (row * chunks + chunk) entry of this launch
  int32_t n;            // pages in this launch
  int32_t pad;
  int32_t pages[kFetchMaxPages];
};
hipError_t launch_fetch(const FetchArgs& a, hipStream_t s);

}  // namespace slora

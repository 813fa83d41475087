// MBGMV: the decode path. Per-token adapter routing, mixed ranks, adapter rows
// gathered through the page table straight from the unified pool ("Makale
// Bulteni - S-LoRA", section "Iddia ve Gerceklik": every token of a batch can use
// its own adapter; the S-LoRA overview, section "2. Heterogeneous Batching":
// kernels that work on non-contiguous memory and on mixed ranks at once).
//
// One kernel runs both halves of the LoRA product so that a decode batch is a
// single launch (a decode batch moves tens of MB; two launches would each pay the
// fixed launch and ramp cost, which is of the order of the whole transfer). The
// work list (32-byte items, token ids inline) is read from pinned host memory.
//
//   shrink items (first in the grid): (group of <= 4 tokens, 8 rows of A^T),
//     4 waves x 2 rows. The group's x goes straight from global memory into LDS
//     (global_load_lds_dwordx4); each wave loads its 2 rows (4096 elements per
//     batch) with one 16-byte load per lane and slice, dots them with every
//     token's x (v_dot2 fp16/bf16 -> fp32) and reduces all 2 x G lane partial
//     sums at once (permlane swaps + DPP).
//   expand items: (<= 2 tokens of a group, 2048 / split output columns). The 4
//     waves cover 4 / split slices of 512 columns; the `split` waves of a slice
//     share its rows (split = 1, 2, 4 for rank <= 16, <= 32, more), so no wave
//     holds more than 16 B rows in flight and none walks a long chain of loads.
//     Each wave loads its page ids, prefetches y0 and issues its B rows before it
//     needs v; lane k then holds v[t][k] and the rows read it with v_readlane;
//     acc[t][8] accumulates in fp32; the waves of a slice add their partial sums
//     through LDS in a fixed order, and y = RNE(y0 + s * acc).
//
// Hand-off of v inside one launch: every v entry is one 64-bit word holding the
// fp32 value and the 32-bit tag of the call that wrote it, stored by the shrink
// item with a single relaxed agent-scope store (sc1: performed at the agent's
// coherence point). An expand wave polls its own entries with agent-scope loads
// until every one carries the call's tag. Value and tag travel in one word, so
// no counters, fences or cache maintenance are needed and a shrink workgroup
// exits as soon as its stores are issued. The host gives each call on a workspace
// a fresh tag and clears the workspace before a tag could repeat.
//
// Forward progress: workgroups are dispatched in index order on each XCD and a
// shrink workgroup never waits, so every shrink an expand wave depends on has
// been dispatched before it and finishes. Every wait is bounded anyway: past
// `spin_limit` polls (set by the host, 2^20 by default) the wave records the tag in
// the error word and goes on, so no wave can spin forever.
//
// Every page load issues unconditionally: rows past the rank, invalid page ids and
// lanes past the end of a row are pointed at 16-byte fill vectors (zero or NaN)
// instead of being predicated, so no load waits on another load's result.
#include "mbgmv_dev.h"

namespace slora {
namespace {

using namespace mb;

// One work item per workgroup (mb::run_item).
template <int DT, bool kUniformChunk, bool kTag>
__global__ __launch_bounds__(64 * kWaves) void mbgmv_kernel(
    Geom g, const MbItem* __restrict__ items, const uint16_t* __restrict__ x, void* v,
    uint16_t* __restrict__ y, uint32_t tag, unsigned long long* err, int32_t spin_limit) {
  extern __shared__ uint4 lds[];  // shrink: [G][kBatchVecs] of x; expand: partial sums
  const MbItem it = load_item(items, blockIdx.x);
  run_item<DT, kUniformChunk, kTag, true>(g, it, x, v, y, tag, err, spin_limit, lds);
}

template <int DT, bool kTag>
hipError_t launch_dt(const Geom& g, const MbItem* items, int32_t n_items, bool shrinks,
                     bool expands, int32_t g_max, const void* x, void* v, void* y, uint32_t tag,
                     unsigned long long* err, int32_t spin_limit, hipStream_t s,
                     const LaunchEvents& ev) {
  const dim3 grid((unsigned)n_items), block(64 * kWaves);
  size_t lds = shrinks ? (size_t)g_max * kBatchVecs * sizeof(uint4) : 0;
  if (expands) lds = lds > (size_t)kRedBytes ? lds : (size_t)kRedBytes;
  if (g.P % 512 == 0)
    hipExtLaunchKernelGGL((mbgmv_kernel<DT, true, kTag>), grid, block, lds, s, ev.start, ev.stop, 0,
                          g, items, (const uint16_t*)x, v, (uint16_t*)y, tag, err, spin_limit);
  else
    hipExtLaunchKernelGGL((mbgmv_kernel<DT, false, kTag>), grid, block, lds, s, ev.start, ev.stop, 0,
                          g, items, (const uint16_t*)x, v, (uint16_t*)y, tag, err, spin_limit);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint4* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t launch_mbgmv(const Geom& g, const MbItem* items, int32_t n_items, bool shrinks,
                        bool expands, int32_t max_tok, const void* x, void* v, void* y,
                        uint32_t tag, unsigned long long* err, int32_t spin_limit, hipStream_t s,
                        const LaunchEvents& ev) {
  if (n_items <= 0) return hipSuccess;
  if (max_tok < 1 || max_tok > kMbGroup) return hipErrorInvalidValue;
  const int g_max = max_tok <= 1 ? 1 : max_tok <= 2 ? 2 : 4;
  if (tag)
    return g.dtype == SLORA_F16
               ? launch_dt<SLORA_F16, true>(g, items, n_items, shrinks, expands, g_max, x, v, y, tag, err, spin_limit, s, ev)
               : launch_dt<SLORA_BF16, true>(g, items, n_items, shrinks, expands, g_max, x, v, y, tag, err, spin_limit, s, ev);
  return g.dtype == SLORA_F16
             ? launch_dt<SLORA_F16, false>(g, items, n_items, shrinks, expands, g_max, x, v, y, 0, err, spin_limit, s, ev)
             : launch_dt<SLORA_BF16, false>(g, items, n_items, shrinks, expands, g_max, x, v, y, 0, err, spin_limit, s, ev);
}

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  const int64_t n = bytes / 16;  // callers pass multiples of 256 bytes
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n);
  return hipGetLastError();
}

}  // namespace slora

// Adapter fetch: copy adapter rows (row-major, in pinned host memory) into their pool
// pages. The kernel reads the host rows directly over PCIe (zero-copy) and takes its
// page list from pinned host memory too, so one launch moves every page of a call (one
// adapter or many) on the caller's side stream with no device staging buffer; a fixed
// number of workgroups walks the list. The S-LoRA pages describe this transfer as
// asynchronous, page by page, from host DRAM to GPU memory ("Makale Bulteni - S-LoRA",
// section "Iddia ve Gerceklik"; the paper review "S-LoRA: Serving Thousands of
// Concurrent LoRA Adapters", section "Proposed method": adapters stay in host memory
// and are fetched on demand).
#include "device_common.h"

namespace slora {
namespace {

constexpr int kFetchThreads = 256;
constexpr int kFetchUnroll = 4;  // 16-byte loads a thread has in flight before it stores
// Workgroups of one launch, each walking every kFetchWgs-th page of the list: enough
// reads in flight to keep the link busy. Measured on the decode_7b adapters (57.5 MB):
// 56 GB/s against 53 GB/s with one workgroup per page and 40 GB/s with launches of 256
// pages each (the copy engines move the same bytes at 56.5 GB/s).
constexpr int kFetchWgs = 256;

__global__ __launch_bounds__(kFetchThreads) void fetch_kernel(const FetchPage* __restrict__ pages,
                                                              int32_t n, uint16_t* __restrict__ pool,
                                                              int32_t P) {
  constexpr int kStride = kFetchThreads * 8;  // elements per sweep of the workgroup
  for (int q = (int)blockIdx.x; q < n; q += (int)gridDim.x) {
    const FetchPage f = pages[q];
    uint16_t* dst = pool + (int64_t)f.page * P;
    for (int i0 = (int)threadIdx.x * 8; i0 < f.len; i0 += kFetchUnroll * kStride) {
      uint4 v[kFetchUnroll];
#pragma unroll
      for (int u = 0; u < kFetchUnroll; ++u) {
        const int i = i0 + u * kStride;
        v[u] = i < f.len ? dev::ld16(f.src + i) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kFetchUnroll; ++u) {
        const int i = i0 + u * kStride;
        if (i < f.len) dev::st16(dst + i, v[u]);
      }
    }
  }
}

}  // namespace

hipError_t launch_fetch(const FetchPage* pages, int64_t n, uint16_t* pool, int32_t page_elems,
                        hipStream_t s, const LaunchEvents& ev) {
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX) return hipErrorInvalidValue;
  const int64_t wgs = n < kFetchWgs ? n : kFetchWgs;
  hipExtLaunchKernelGGL(fetch_kernel, dim3((unsigned)wgs), dim3(kFetchThreads), 0, s, ev.start,
                        ev.stop, 0, pages, (int32_t)n, pool, page_elems);
  return hipGetLastError();
}

}  // namespace slora

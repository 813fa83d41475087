// Adapter fetch: copy one matrix of an adapter (rows x L, row-major, in pinned host
// memory) into its pool pages, one workgroup per destination page. The kernel reads
// the host rows directly over PCIe (zero-copy), so a whole batch of pages moves in
// one launch on the caller's side stream with no device staging buffer. The S-LoRA
// pages describe this transfer as asynchronous, page by page, from host DRAM to GPU
// memory ("Makale Bulteni - S-LoRA", section "Iddia ve Gerceklik"; the paper review
// "S-LoRA: Serving Thousands of Concurrent LoRA Adapters", section "Proposed
// method": adapters stay in host memory and are fetched on demand).
#include "device_common.h"

namespace slora {
namespace {

__global__ __launch_bounds__(256) void fetch_kernel(FetchArgs a) {
  const int e = a.e0 + (int)blockIdx.x;
  const int row = e / a.chunks, chunk = e - row * a.chunks;
  const int len = min(a.P, a.L - chunk * a.P);  // elements of this row on this page
  const uint16_t* src = a.src + (int64_t)row * a.L + (int64_t)chunk * a.P;
  uint16_t* dst = a.pool + (int64_t)a.pages[blockIdx.x] * a.P;
  for (int i = (int)threadIdx.x * 8; i < len; i += 256 * 8) dev::st16(dst + i, dev::ld16(src + i));
}

}  // namespace

hipError_t launch_fetch(const FetchArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fetch_kernel, dim3((unsigned)a.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace slora

// Ablation baseline "S-LoRA with conventional batched matmul" (the S-LoRA overview,
// section "S-LoRA的性能评估", its comparison of S-LoRA variants): before the LoRA
// product, every request's adapter is copied out of the paged pool into contiguous
// memory of its own, every adapter padded with zero rows to the batch's largest rank,
// so that one padded batched GEMM can run over the copies. This kernel is the copy:
// one workgroup per destination page. Destination page e of request q holds, in the
// pool's own chunking, A^T row k chunk c (e < r_pad * cA) or B row k chunk c; rows at
// or past the adapter's rank are zero. The workgroup also writes e into the identity
// page table of the copy.
#include "device_common.h"

namespace slora {
namespace {

__global__ __launch_bounds__(256) void gather_kernel(Geom g, const GatherReq* __restrict__ reqs,
                                                     int32_t r_pad, uint16_t* __restrict__ dst,
                                                     int32_t* __restrict__ dst_pt) {
  const int64_t e = blockIdx.x;
  const int32_t per_req = r_pad * (g.cA + g.cB);
  const int32_t q = (int32_t)(e / per_req), w = (int32_t)(e - (int64_t)q * per_req);
  const GatherReq rq = reqs[q];
  const bool a_half = w < r_pad * g.cA;
  const int32_t k = a_half ? w / g.cA : (w - r_pad * g.cA) / g.cB;
  const int32_t c = a_half ? w % g.cA : (w - r_pad * g.cA) % g.cB;
  const int32_t len = a_half ? g.d_in : g.d_out;
  int32_t page = -1;
  if (k < rq.rank)
    page = g.pt[(int64_t)rq.pt_base + (a_half ? (int64_t)k * g.cA + c
                                              : (int64_t)rq.rank * g.cA + (int64_t)k * g.cB + c)];
  const int32_t n = min(g.P, len - c * g.P);  // elements of the row on this page
  uint16_t* out = dst + e * g.P;
  const bool ok = (uint32_t)page < (uint64_t)g.n_pages;
  for (int i = threadIdx.x * 8; i < g.P; i += 256 * 8) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (k < rq.rank && i < n)
      v = dev::ld16(ok ? g.pool + (int64_t)page * g.P + i
                       : g.dtype == SLORA_F16 ? dev::fill_nan<SLORA_F16>() : dev::fill_nan<SLORA_BF16>());
    dev::st16(out + i, v);
  }
  if (threadIdx.x == 0) dst_pt[e] = (int32_t)e;
}

}  // namespace

hipError_t launch_gather(const Geom& g, const GatherReq* reqs, int32_t n_req, int32_t r_pad,
                         void* dst, int32_t* dst_pt, hipStream_t s, const LaunchEvents& ev) {
  const int64_t pages = (int64_t)n_req * r_pad * (g.cA + g.cB);
  if (pages <= 0) return hipSuccess;
  if (pages > INT32_MAX) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL(gather_kernel, dim3((unsigned)pages), dim3(256), 0, s, ev.start, ev.stop, 0, g,
                        reqs, r_pad, (uint16_t*)dst, dst_pt);
  return hipGetLastError();
}

}  // namespace slora

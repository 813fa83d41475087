// MBGMV: the decode path. Per-token adapter routing, mixed ranks, adapter rows
// gathered through the page table straight from the unified pool ("Makale
// Bulteni - S-LoRA", section "Iddia ve Gerceklik": every token of a batch can use
// its own adapter; the S-LoRA overview, section "2. Heterogeneous Batching":
// kernels that work on non-contiguous memory and on mixed ranks at once).
//
// Decode is memory bound: each adapter row is read once per group of up to
// kMbGroup tokens sharing the adapter, so the kernels stream adapter pages from
// HBM with 16-byte loads per lane (a wave reads 1 KiB of one page per load
// instruction) and keep the arithmetic in registers.
//
// shrink: one workgroup = (group, block of 8 rows of A^T); each wave owns 2 rows.
//         Lanes hold 8-element slices of a row, dot them with the group's x rows
//         (v_dot2 fp16/bf16 -> fp32), and one halving butterfly reduces all
//         2 x kMbGroup partial sums of the wave at once. v is written in fp32.
// expand: one workgroup = (group, 1024 output columns); v of the group is staged
//         in LDS, each lane streams 16 bytes of each B row, accumulates
//         kMbGroup x 8 fp32 sums over k, then y = RNE(y0 + s * acc) in place.
#include "device_common.h"

namespace slora {
namespace {

using namespace dev;

constexpr int kShrinkWaves = kMbShrinkRows / 2;  // 2 rows per wave
constexpr int kRowsPerWave = 2;
constexpr int kShrinkU = 8;                      // 16-byte vectors per lane per row in flight
constexpr int kExpandWaves = kMbExpandCols / 512;
constexpr int kExpandKU = 8;                     // B rows in flight per lane

template <int DT, bool kUniformChunk>
__global__ __launch_bounds__(64 * kShrinkWaves) void mbgmv_shrink_kernel(
    Geom g, const int32_t* __restrict__ tok, const GroupDesc* __restrict__ groups,
    const Item* __restrict__ items, const uint16_t* __restrict__ x, float* __restrict__ v) {
  constexpr int G = kMbGroup, R = kRowsPerWave, U = kShrinkU;
  const Item it = items[blockIdx.x];
  const GroupDesc gd = groups[it.group];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k0 = it.block * kMbShrinkRows + wave * R;
  if (k0 >= gd.rank) return;  // wave-uniform; no barrier in this kernel
  const int nrow = min(R, gd.rank - k0);
  const int n = gd.n_tok;
  const int nvec = g.d_in >> 3;  // 16-byte vectors per row

  const uint16_t* xr[G];
#pragma unroll
  for (int t = 0; t < G; ++t)
    xr[t] = x + (int64_t)tok[gd.tok_begin + min(t, n - 1)] * g.d_in;

  float acc[R][G];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < G; ++t) acc[r][t] = 0.f;

  const int32_t* ptA = g.pt + gd.pt_base + (int64_t)k0 * g.cA;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  const uint32_t nw = nan2<DT>();
  const uint4 nanv = make_uint4(nw, nw, nw, nw);

  for (int vb = 0; vb < nvec; vb += 64 * U) {
    uint4 a[R][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = vb + u * 64 + lane;
      const int j = q * 8;
      int c;
      if constexpr (kUniformChunk) c = ((vb + u * 64) * 8) / g.P;  // the 512 elements share a page
      else c = j / g.P;
      const int off = j - c * g.P;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        a[r][u] = zero;
        if (r < nrow && q < nvec) {
          const int32_t page = ptA[r * g.cA + c];
          a[r][u] = ((uint32_t)page < (uint64_t)g.n_pages)
                        ? ld16(g.pool + (int64_t)page * g.P + off)
                        : nanv;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < G; ++t) {
      if (t < n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = vb + u * 64 + lane;
          if (q < nvec) {
            const uint4 xv = ld16(xr[t] + q * 8);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][t] = dot8<DT>(a[r][u], xv, acc[r][t]);
          }
        }
      }
    }
  }

  float flat[R * G];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < G; ++t) flat[r * G + t] = acc[r][t];
  const float tot = xreduce<R * G>(flat, lane);
  if (reduce_writer<R * G>(lane)) {
    const int idx = reduce_index<R * G>(lane);
    const int r = idx / G, t = idx % G;
    if (r < nrow && t < n)
      v[(int64_t)tok[gd.tok_begin + t] * g.r_max + k0 + r] = tot;
  }
}

template <int DT, bool kUniformChunk>
__global__ __launch_bounds__(64 * kExpandWaves) void mbgmv_expand_kernel(
    Geom g, const int32_t* __restrict__ tok, const GroupDesc* __restrict__ groups,
    const float* __restrict__ v, uint16_t* __restrict__ y) {
  constexpr int G = kMbGroup, KU = kExpandKU;
  const GroupDesc gd = groups[blockIdx.x];
  const int r = gd.rank, n = gd.n_tok;
  __shared__ float vs[G][kMaxRank];
  for (int i = threadIdx.x; i < n * r; i += 64 * kExpandWaves) {
    const int t = i / r, k = i - t * r;
    vs[t][k] = v[(int64_t)tok[gd.tok_begin + t] * g.r_max + k];
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int colw = (blockIdx.y * kExpandWaves + wave) * 512;
  if (colw >= g.d_out) return;  // wave-uniform, after the only barrier
  const int col = colw + lane * 8;
  const bool valid = col < g.d_out;
  int c;
  if constexpr (kUniformChunk) c = colw / g.P;
  else c = col / g.P;
  const int off = col - c * g.P;
  const int32_t* ptB = g.pt + gd.pt_base + (int64_t)r * g.cA + c;

  float acc[G][8];
#pragma unroll
  for (int t = 0; t < G; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;

  const uint4 zero = make_uint4(0, 0, 0, 0);
  const uint32_t nw = nan2<DT>();
  const uint4 nanv = make_uint4(nw, nw, nw, nw);
  for (int k = 0; k < r; k += KU) {
    uint4 b[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      b[u] = zero;
      if (k + u < r && valid) {
        const int32_t page = ptB[(int64_t)(k + u) * g.cB];
        b[u] = ((uint32_t)page < (uint64_t)g.n_pages) ? ld16(g.pool + (int64_t)page * g.P + off)
                                                       : nanv;
      }
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      if (k + u < r) {
        float bf[8];
        bf[0] = lo_f32<DT>(b[u].x); bf[1] = hi_f32<DT>(b[u].x);
        bf[2] = lo_f32<DT>(b[u].y); bf[3] = hi_f32<DT>(b[u].y);
        bf[4] = lo_f32<DT>(b[u].z); bf[5] = hi_f32<DT>(b[u].z);
        bf[6] = lo_f32<DT>(b[u].w); bf[7] = hi_f32<DT>(b[u].w);
#pragma unroll
        for (int t = 0; t < G; ++t) {
          if (t < n) {
            const float vt = vs[t][k + u];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(vt, bf[e], acc[t][e]);
          }
        }
      }
    }
  }
  if (!valid) return;
  const float s = gd.scale;
#pragma unroll
  for (int t = 0; t < G; ++t) {
    if (t < n) {
      uint16_t* yr = y + (int64_t)tok[gd.tok_begin + t] * g.d_out + col;
      const uint4 y0 = ld16(yr);
      uint4 o;
      o.x = pack2<DT>(fmaf(s, acc[t][0], lo_f32<DT>(y0.x)), fmaf(s, acc[t][1], hi_f32<DT>(y0.x)));
      o.y = pack2<DT>(fmaf(s, acc[t][2], lo_f32<DT>(y0.y)), fmaf(s, acc[t][3], hi_f32<DT>(y0.y)));
      o.z = pack2<DT>(fmaf(s, acc[t][4], lo_f32<DT>(y0.z)), fmaf(s, acc[t][5], hi_f32<DT>(y0.z)));
      o.w = pack2<DT>(fmaf(s, acc[t][6], lo_f32<DT>(y0.w)), fmaf(s, acc[t][7], hi_f32<DT>(y0.w)));
      st16(yr, o);
    }
  }
}

template <int DT>
hipError_t shrink_dt(const Geom& g, const int32_t* tok, const GroupDesc* groups, const Item* items,
                     int32_t n_items, const void* x, float* v, hipStream_t s) {
  const dim3 grid((unsigned)n_items), block(64 * kShrinkWaves);
  if (g.P % 512 == 0)
    hipLaunchKernelGGL((mbgmv_shrink_kernel<DT, true>), grid, block, 0, s, g, tok, groups, items,
                       (const uint16_t*)x, v);
  else
    hipLaunchKernelGGL((mbgmv_shrink_kernel<DT, false>), grid, block, 0, s, g, tok, groups, items,
                       (const uint16_t*)x, v);
  return hipGetLastError();
}

template <int DT>
hipError_t expand_dt(const Geom& g, const int32_t* tok, const GroupDesc* groups, int32_t n_groups,
                     const float* v, void* y, hipStream_t s) {
  const dim3 grid((unsigned)n_groups, (unsigned)((g.d_out + kMbExpandCols - 1) / kMbExpandCols));
  const dim3 block(64 * kExpandWaves);
  if (g.P % 512 == 0)
    hipLaunchKernelGGL((mbgmv_expand_kernel<DT, true>), grid, block, 0, s, g, tok, groups, v,
                       (uint16_t*)y);
  else
    hipLaunchKernelGGL((mbgmv_expand_kernel<DT, false>), grid, block, 0, s, g, tok, groups, v,
                       (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mbgmv_shrink(const Geom& g, const int32_t* tok, const GroupDesc* groups,
                               const Item* items, int32_t n_items, const void* x, float* v,
                               hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  return g.dtype == SLORA_F16 ? shrink_dt<SLORA_F16>(g, tok, groups, items, n_items, x, v, s)
                              : shrink_dt<SLORA_BF16>(g, tok, groups, items, n_items, x, v, s);
}

hipError_t launch_mbgmv_expand(const Geom& g, const int32_t* tok, const GroupDesc* groups,
                               int32_t n_groups, const float* v, void* y, hipStream_t s) {
  if (n_groups <= 0) return hipSuccess;
  return g.dtype == SLORA_F16 ? expand_dt<SLORA_F16>(g, tok, groups, n_groups, v, y, s)
                              : expand_dt<SLORA_BF16>(g, tok, groups, n_groups, v, y, s);
}

}  // namespace slora

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
#include "device_common.h"

namespace slora {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 2;
static_assert(kWaves * kRowsPerWave == kMbShrinkRows, "shrink row block");
constexpr int kBatchVecs = 512;  // 16-byte vectors of a row per shrink batch (4096 elements)
constexpr int kSlices = kBatchVecs / 64;
constexpr int kKU = kMbRowsPerWave;
constexpr int kRedBytes = (kWaves - 1) * kMbExpandTok * 8 * 64 * 4;  // expand partial sums

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ int pick4(const int (&t)[kMbGroup], int i) {
  return i == 0 ? t[0] : i == 1 ? t[1] : i == 2 ? t[2] : t[3];
}

// ------------------------------------------------------------------ shrink role
template <int DT, bool kUniformChunk, int G, bool kTag>
__device__ __forceinline__ void shrink_body(const Geom& g, const MbItem& it,
                                            const uint16_t* __restrict__ x, void* __restrict__ v,
                                            uint32_t tag, uint4* xs) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int k0 = it.part * kMbShrinkRows + wave * kRowsPerWave;
  const int nrow = max(0, min(kRowsPerWave, it.rank - k0));  // 0: this wave only stages x
  const int n = it.n_tok();
  const int nvec = g.d_in >> 3;
  const int npid = nrow * g.cA;  // <= 2 * 32 (the planner limits cA)
  const int my_pid = lane < npid ? g.pt[(int64_t)it.pt_base + (int64_t)k0 * g.cA + lane] : -1;
  const int tok[kMbGroup] = {it.tok[0], it.tok[1], it.tok[2], it.tok[3]};

  float acc[kRowsPerWave][G];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < G; ++t) acc[r][t] = 0.f;

  for (int vb = 0; vb < nvec; vb += kBatchVecs) {
    uint4 a[kRowsPerWave][kSlices];
#pragma unroll
    for (int u = 0; u < kSlices; ++u) {
      const int qb = vb + u * 64;  // first vector of this slice (uniform)
      const int q = min(qb + lane, nvec - 1);
      int c;
      if constexpr (kUniformChunk) c = (qb * 8) / g.P;  // a 512-element slice never crosses a page
      else c = (q * 8) / g.P;
      const int off = q * 8 - c * g.P;
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const bool live = qb < nvec && r < nrow;  // uniform
        const int idx = live ? r * g.cA + c : 0;
        int page;
        if constexpr (kUniformChunk) page = readlane(my_pid, idx);
        else page = __shfl(my_pid, idx);
        const bool ok = (uint32_t)page < (uint64_t)g.n_pages;
        a[r][u] = ld16(!live ? fill_zero() : ok ? g.pool + (int64_t)page * g.P + off : fill_nan<DT>());
      }
    }
    // this batch of every token's x, global -> LDS directly; zero past the row end
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const uint16_t* xr = x + (int64_t)tok[t < n ? t : 0] * g.d_in;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = vb + h * 256 + tid;
        __builtin_amdgcn_global_load_lds((t < n && q < nvec) ? xr + q * 8 : fill_zero(),
                                         xs + t * kBatchVecs + h * 256 + wave * 64, 16, 0, 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
      for (int u = 0; u < kSlices; ++u) {
        const uint4 xq = xs[t * kBatchVecs + u * 64 + lane];  // zero past the end of the row
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) acc[r][t] = dot8<DT>(a[r][u], xq, acc[r][t]);
      }
    __syncthreads();  // xs is overwritten by the next batch
  }

  constexpr int V = kRowsPerWave * G;
  float flat[V];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < G; ++t) flat[r * G + t] = acc[r][t];
  float tot[WaveSum<V>::kOut];
  wave_sum<V>(flat, tot);
#pragma unroll
  for (int i = 0; i < WaveSum<V>::kOut; ++i) {
    const int idx = wave_sum_index<V>(lane, i);
    const int r = idx / G, t = idx % G;
    if (wave_sum_writer<V>(lane, i) && r < nrow && t < n) {
      const int64_t at = (int64_t)pick4(tok, t) * g.r_max + k0 + r;
      if constexpr (kTag)
        __hip_atomic_store(static_cast<unsigned long long*>(v) + at,
                           ((unsigned long long)tag << 32) | __float_as_uint(tot[i]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        static_cast<float*>(v)[at] = tot[i];
    }
  }
}

// ------------------------------------------------------------------ expand role
template <int DT, bool kUniformChunk, int NT, bool kTag>
__device__ __forceinline__ void expand_body(const Geom& g, const MbItem& it,
                                            const void* __restrict__ v, uint16_t* __restrict__ y,
                                            uint32_t tag, unsigned long long* err, int32_t spin_limit,
                                            float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = it.rank, n = it.n_tok(), split = it.split();
  const int slices = kWaves / split, slice = wave / split, rp = wave % split;
  const int rpw = (r + split - 1) / split;  // rows per wave (<= 32)
  const int k_lo = min(r, rp * rpw), nk = min(r, k_lo + rpw) - k_lo;
  const int colw = (it.part * slices + slice) * kMbWaveCols;  // first column of this wave
  const bool wave_live = colw < g.d_out;
  const int col = min(colw + lane * 8, g.d_out - 8);  // tail lanes duplicate a valid column
  const bool lane_live = colw + lane * 8 < g.d_out;
  int c;
  if constexpr (kUniformChunk) c = min(colw, g.d_out - 8) / g.P;
  else c = col / g.P;
  const int off = col - c * g.P;
  const int64_t pbase = (int64_t)it.pt_base + (int64_t)r * g.cA + c + (int64_t)k_lo * g.cB;
  int pid = -1;  // lane k: page of this wave's row k_lo + k in its chunk (nk <= 32)
  if constexpr (kUniformChunk) pid = lane < nk ? g.pt[pbase + (int64_t)lane * g.cB] : -1;
  const int t0 = it.tok[0], t1 = it.tok[1];

  uint4 y0v[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    y0v[t] = ld16((rp == 0 && t < n && wave_live) ? y + (int64_t)(t ? t1 : t0) * g.d_out + col
                                                   : fill_zero());

  auto load_rows = [&](uint4 (&b)[kKU], int k) {
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int kk = k + u;
      const bool live = kk < nk && wave_live;  // uniform
      int page;
      if constexpr (kUniformChunk) page = readlane(pid, kk & 63);
      else page = g.pt[live ? pbase + (int64_t)kk * g.cB : 0];
      const bool ok = (uint32_t)page < (uint64_t)g.n_pages;
      b[u] = ld16(!live ? fill_zero() : ok ? g.pool + (int64_t)page * g.P + off : fill_nan<DT>());
    }
  };

  uint4 b[kKU];
  load_rows(b, 0);

  float vr[NT];  // lane k: v[t][k_lo + k] (k < 32); rows 32..63 of a wave do not occur
  if constexpr (kTag) {
    // poll until every entry this wave needs carries the call's tag
    const unsigned long long* vt = static_cast<const unsigned long long*>(v);
    const unsigned long long* src[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      src[t] = (t < n && lane < nk) ? vt + (int64_t)(t ? t1 : t0) * g.r_max + k_lo + lane
                                    : reinterpret_cast<const unsigned long long*>(fill_zero());
    unsigned long long w[NT];
    for (int spins = 0;; ++spins) {
      bool ready = true;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        w[t] = __hip_atomic_load(src[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ready = ready && (!(t < n && lane < nk) || (uint32_t)(w[t] >> 32) == tag);
      }
      if (__all(ready)) break;
      if (spins >= spin_limit) {
        if (lane == 0) __hip_atomic_store(err, (unsigned long long)tag, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) vr[t] = __uint_as_float((uint32_t)w[t]);
  } else {
    const float* vf = static_cast<const float*>(v);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      vr[t] = *((t < n && lane < nk) ? vf + (int64_t)(t ? t1 : t0) * g.r_max + k_lo + lane
                                     : reinterpret_cast<const float*>(fill_zero()));
  }

  float acc[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;

  auto mul_rows = [&](int k) {
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      if (k + u < nk) {  // uniform
        float bf[8];
        bf[0] = lo_f32<DT>(b[u].x); bf[1] = hi_f32<DT>(b[u].x);
        bf[2] = lo_f32<DT>(b[u].y); bf[3] = hi_f32<DT>(b[u].y);
        bf[4] = lo_f32<DT>(b[u].z); bf[5] = hi_f32<DT>(b[u].z);
        bf[6] = lo_f32<DT>(b[u].w); bf[7] = hi_f32<DT>(b[u].w);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float vt = readlane_f(vr[t], k + u);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(vt, bf[e], acc[t][e]);
        }
      }
    }
  };
  mul_rows(0);
  if (nk > kKU) {  // rank > 64: a second batch of 16 rows (straight-line: no loop-carried copy)
    load_rows(b, kKU);
    mul_rows(kKU);
  }

  if (split > 1) {  // the waves of a slice add their partial sums, in rank-part order
    if (rp > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[(((wave - 1) * kMbExpandTok + t) * 8 + e) * 64 + lane] = acc[t][e];
    }
    __syncthreads();
    if (rp == 0) {
      for (int q = 1; q < split; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[t][e] += red[(((wave + q - 1) * kMbExpandTok + t) * 8 + e) * 64 + lane];
    }
  }
  if (rp != 0 || !wave_live || !lane_live) return;
  const float s = it.scale;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < n) {
      const uint4 y0 = y0v[t];
      uint4 o;
      o.x = pack2<DT>(fmaf(s, acc[t][0], lo_f32<DT>(y0.x)), fmaf(s, acc[t][1], hi_f32<DT>(y0.x)));
      o.y = pack2<DT>(fmaf(s, acc[t][2], lo_f32<DT>(y0.y)), fmaf(s, acc[t][3], hi_f32<DT>(y0.y)));
      o.z = pack2<DT>(fmaf(s, acc[t][4], lo_f32<DT>(y0.z)), fmaf(s, acc[t][5], hi_f32<DT>(y0.z)));
      o.w = pack2<DT>(fmaf(s, acc[t][6], lo_f32<DT>(y0.w)), fmaf(s, acc[t][7], hi_f32<DT>(y0.w)));
      st16(y + (int64_t)(t ? t1 : t0) * g.d_out + col, o);
    }
  }
}

// Role per item. kTag: one fused call (v tagged, expand waves poll for it);
// otherwise a shrink-only or expand-only launch with plain fp32 v.
template <int DT, bool kUniformChunk, bool kTag>
__global__ __launch_bounds__(64 * kWaves) void mbgmv_kernel(
    Geom g, const MbItem* __restrict__ items, const uint16_t* __restrict__ x, void* v,
    uint16_t* __restrict__ y, uint32_t tag, unsigned long long* err, int32_t spin_limit) {
  extern __shared__ uint4 lds[];  // shrink: [G][kBatchVecs] of x; expand: partial sums
  const MbItem it = items[blockIdx.x];
  if (it.role() == 0) {
    const int n = it.n_tok();
    static_assert(kMbGroup == 4, "shrink bodies cover 1, 2 and 4 tokens");
    if (n <= 1) shrink_body<DT, kUniformChunk, 1, kTag>(g, it, x, v, tag, lds);
    else if (n <= 2) shrink_body<DT, kUniformChunk, 2, kTag>(g, it, x, v, tag, lds);
    else shrink_body<DT, kUniformChunk, 4, kTag>(g, it, x, v, tag, lds);
  } else {
    float* red = reinterpret_cast<float*>(lds);
    if (it.n_tok() <= 1) expand_body<DT, kUniformChunk, 1, kTag>(g, it, v, y, tag, err, spin_limit, red);
    else expand_body<DT, kUniformChunk, 2, kTag>(g, it, v, y, tag, err, spin_limit, red);
  }
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

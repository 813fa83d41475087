// MBGMV device bodies: the decode path's shrink and expand roles and the dispatch of
// one work item to its role. Shared by the MBGMV kernel (mbgmv.hip, whose header
// describes what they compute) and the launch that runs both families at once.
#pragma once

#include "device_common.h"

namespace slora {
namespace mb {

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
template <int DT, bool kUniformChunk, int G, bool kTag, bool kSgprIds>
__device__ __forceinline__ void shrink_body(const Geom& g, const MbItem& it,
                                            const uint16_t* __restrict__ x, void* __restrict__ v,
                                            uint32_t tag, uint4* xs) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int k0 = it.part * kMbShrinkRows + wave * kRowsPerWave;
  const int nrow = max(0, min(kRowsPerWave, it.rank - k0));  // 0: this wave only stages x
  const int n = it.n_tok();
  const int nvec = g.d_in >> 3;
  const int64_t pbase = (int64_t)it.pt_base + (int64_t)k0 * g.cA;
  const int npid = nrow * g.cA;  // <= 2 * 32 (the planner limits cA)
  int my_pid = -1;  // lane i: entry i of this wave's rows
  if constexpr (kUniformChunk && kSgprIds) {
    // read per batch into scalar registers instead (below)
  } else if (kUniformChunk && npid <= 16) {  // scalar cache; no rows: the adapter's first entry
    my_pid = sload16_to_lanes(g.pt + (npid > 0 ? pbase : (int64_t)it.pt_base), 0, max(npid - 1, 0), 1, -1, 0);
  } else {
    my_pid = lane < npid ? g.pt[pbase + lane] : -1;
  }
  const int tok[kMbGroup] = {it.tok[0], it.tok[1], it.tok[2], it.tok[3]};

  float acc[kRowsPerWave][G];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < G; ++t) acc[r][t] = 0.f;

  for (int vb = 0; vb < nvec; vb += kBatchVecs) {
    uint4 a[kRowsPerWave][kSlices];
    int pg[kRowsPerWave * kSlices];  // kSgprIds: this batch's entries, all read before any is used
    if constexpr (kUniformChunk && kSgprIds) {
#pragma unroll
      for (int u = 0; u < kSlices; ++u)
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
          const int qb = vb + u * 64;
          const bool live = qb < nvec && r < nrow;  // a dead row reads the adapter's first entry
          pg[u * kRowsPerWave + r] =
              sload(g.pt + (live ? pbase + r * g.cA + (qb * 8) / g.P : (int64_t)it.pt_base));
        }
      static_assert(kRowsPerWave * kSlices == 16, "settle16");
      settle16(pg);
    }
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
        if constexpr (kUniformChunk) page = kSgprIds ? pg[u * kRowsPerWave + r] : readlane(my_pid, idx);
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
template <int DT, bool kUniformChunk, int NT, bool kTag, bool kSgprIds>
__device__ __forceinline__ void expand_body(const Geom& g, const MbItem& it,
                                            const void* __restrict__ v, uint16_t* __restrict__ y,
                                            uint32_t tag, unsigned long long* err, int32_t spin_limit,
                                            float* red) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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
  const int t0 = it.tok[0], t1 = it.tok[1];

  uint4 y0v[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    y0v[t] = ld16((rp == 0 && t < n && wave_live) ? y + (int64_t)(t ? t1 : t0) * g.d_out + col
                                                   : fill_zero());
  int pid = -1;  // lane k: page of this wave's row k_lo + k in its chunk (nk <= 32)
  if constexpr (kUniformChunk && !kSgprIds) {  // scalar cache; rows past nk repeat row nk - 1
    const int32_t* pb = g.pt + (nk > 0 ? pbase : (int64_t)it.pt_base);  // no rows: first entry
    pid = sload16_to_lanes(pb, 0, max(nk - 1, 0), g.cB, pid, 0);
    if (nk > 16) pid = sload16_to_lanes(pb, 16, nk - 1, g.cB, pid, 16);
  }

  auto load_rows = [&](uint4 (&b)[kKU], int k) {
    int pg[kKU];  // kSgprIds: the batch's entries, all read before any is used
    if constexpr (kUniformChunk && kSgprIds) {
#pragma unroll
      for (int u = 0; u < kKU; ++u)  // a dead row reads the adapter's first entry
        pg[u] = sload(g.pt + (k + u < nk ? pbase + (int64_t)(k + u) * g.cB : (int64_t)it.pt_base));
      static_assert(kKU == 16, "settle16");
      settle16(pg);
    }
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int kk = k + u;
      const bool live = kk < nk && wave_live;  // uniform
      int page;
      if constexpr (kUniformChunk) page = kSgprIds ? pg[u] : readlane(pid, kk & 63);
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

// A work item, read whole through the scalar cache (the list is not written while a
// launch runs).
__device__ __forceinline__ MbItem load_item(const MbItem* items, int64_t i) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(items + i);
  uint32_t w[sizeof(MbItem) / 4];
#pragma unroll
  for (int k = 0; k < (int)(sizeof(MbItem) / 4); ++k) w[k] = sload(p + k);
  MbItem it;
  __builtin_memcpy(&it, w, sizeof(MbItem));
  return it;
}

// Role per item. kTag: one fused call (v tagged, expand waves poll for it); otherwise a
// shrink-only or expand-only launch with plain fp32 v. lds: the group's x (shrink,
// [G][kBatchVecs] vectors) or the split waves' partial sums (expand, kRedBytes).
// Page-table entries of uniform-chunk geometries come through the scalar cache, 16 per
// wave and batch with one wait. kSgprIds: they stay in scalar registers and address the
// rows directly (the MBGMV kernel; a wave issues its rows soonest); otherwise they move
// to lanes of one vector register and are read back per row (the launch that also runs
// segment tiles, whose register budget the extra scalar registers would spill into).
template <int DT, bool kUniformChunk, bool kTag, bool kSgprIds>
__device__ __forceinline__ void run_item(const Geom& g, const MbItem& it, const uint16_t* x,
                                         void* v, uint16_t* y, uint32_t tag,
                                         unsigned long long* err, int32_t spin_limit, uint4* lds) {
  if (it.role() == 0) {
    const int n = it.n_tok();
    static_assert(kMbGroup == 4, "shrink bodies cover 1, 2 and 4 tokens");
    if (n <= 1) shrink_body<DT, kUniformChunk, 1, kTag, kSgprIds>(g, it, x, v, tag, lds);
    else if (n <= 2) shrink_body<DT, kUniformChunk, 2, kTag, kSgprIds>(g, it, x, v, tag, lds);
    else shrink_body<DT, kUniformChunk, 4, kTag, kSgprIds>(g, it, x, v, tag, lds);
  } else {
    float* red = reinterpret_cast<float*>(lds);
    if (it.n_tok() <= 1) expand_body<DT, kUniformChunk, 1, kTag, kSgprIds>(g, it, v, y, tag, err, spin_limit, red);
    else expand_body<DT, kUniformChunk, 2, kTag, kSgprIds>(g, it, v, y, tag, err, spin_limit, red);
  }
}

}  // namespace mb
}  // namespace slora

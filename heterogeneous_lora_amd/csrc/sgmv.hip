// SGMV: the prefill path. A request's prompt tokens share one adapter, so they are
// cut into tiles of up to 64 tokens of one adapter and each tile is a small dense
// product on the matrix cores ("Makale Bulteni - S-LoRA", section "Iddia ve
// Gerceklik": batched LoRA computation with custom kernels over non-contiguous
// memory; the S-LoRA overview, section "2. Heterogeneous Batching": a prefill
// segment is a dense block against one adapter, of whatever rank it has).
//
// Both halves use v_mfma_f32_16x16x32_{bf16,f16}. Lane l of a 16x16x32 product
// holds row l % 16 and the 8 consecutive k at (l / 16) * 8 of each operand, and
// gets rows 4 * (l / 16) + q, q < 4, of column l % 16 of the fp32 result.
//
//   shrink (tile, k-range): v_part[ks][t][k] = sum over the k-range of x[t, j] A^T[k, j].
//     Operands come straight from global memory with 16-byte loads: x rows (the
//     tile's tokens) and A^T rows (rank rows, gathered through the page table)
//     are both contiguous in j. The 4 waves take interleaved 32-wide steps of the
//     k-range and add their partial products through LDS in a fixed order at the
//     end. The k-ranges give the launch enough workgroups to fill the chip; the
//     expand adds the ranges' partial sums in range order, so the result does not
//     depend on scheduling.
//   expand (tile, 256 output columns): y[t, n] = RNE(y0 + s * sum_k v[t, k] B[k, n]).
//     The product is computed transposed, D = B^T v^T, so that each lane ends up
//     with 8 consecutive output columns of one token (16-byte y0 loads and y
//     stores). v (summed over k-ranges, rounded once to the storage type to feed
//     the matrix cores) and 32-row chunks of B are staged in LDS; the B^T operand
//     is read out of LDS column-wise.
#include <algorithm>

#include "device_common.h"

namespace slora {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStep = 32;          // k per MFMA
constexpr int kRound = kWaves * kStep;
constexpr int kTileRows = 64;      // tokens per tile (4 blocks of 16)
static_assert(kTileRows == kSgTile, "tile rows");

template <int DT>
__device__ __forceinline__ f32x4 mfma(const uint4& a, const uint4& b, f32x4 c) {
  if constexpr (DT == SLORA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Token of row m of a tile, or -1 past its end.
__device__ __forceinline__ int tile_token(const SgTile& tl, const int32_t* tok, int m) {
  if (m >= tl.n_tok) return -1;
  return tl.first_tok >= 0 ? tl.first_tok + m : tok[tl.tok_begin + m];
}

// ------------------------------------------------------------------ shrink
// NB: 16-row blocks of rank rows (rank <= 16 * NB).
template <int DT, int NB>
__global__ __launch_bounds__(64 * kWaves) void sgmv_shrink_kernel(
    Geom g, const SgTile* __restrict__ tiles, const int32_t* __restrict__ tok, int32_t kc,
    const uint16_t* __restrict__ x, float* __restrict__ vpart, int64_t split_stride) {
  extern __shared__ float red[];  // [3][4 * 4 * kRedCb][64] partial sums of waves 1..3
  constexpr int kRedCb = NB < 4 ? NB : 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kg = lane >> 4;
  const SgTile tl = tiles[blockIdx.x];
  const int ks = blockIdx.y;
  const int kb = ks * kc, ke = min(g.d_in, kb + kc);
  const int r = tl.rank;

  int tk[4];  // this lane's operand rows: token of row tb * 16 + li
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) tk[tb] = tile_token(tl, tok, tb * 16 + li);

  // A^T row of each rank block for this lane, and the page it reads in chunk c
  int k = kb + wave * kStep + kg * 8;  // this lane's first element
  int c = k / g.P, off = k - c * g.P;
  const uint16_t* arow[NB];  // page start, or a fill vector (then `areal` is false)
  bool areal[NB];
  auto load_pages = [&]() {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int n = cb * 16 + li;
      const uint16_t* p = fill_zero();
      bool real = false;
      if (n < r && c < g.cA) {
        const int page = g.pt[(int64_t)tl.pt_base + (int64_t)n * g.cA + c];
        real = (uint32_t)page < (uint64_t)g.n_pages;
        p = real ? g.pool + (int64_t)page * g.P : fill_nan<DT>();
      }
      arow[cb] = p;
      areal[cb] = real;
    }
  };
  load_pages();

  f32x4 acc[4][NB];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[tb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kb + wave * kStep; k0 < ke; k0 += kRound) {
    const bool live = k < ke;
    uint4 xa[4], aa[NB];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      xa[tb] = ld16(live && tk[tb] >= 0 ? x + (int64_t)tk[tb] * g.d_in + k : fill_zero());
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
      aa[cb] = ld16(!live ? fill_zero() : areal[cb] ? arow[cb] + off : arow[cb]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[tb][cb] = mfma<DT>(xa[tb], aa[cb], acc[tb][cb]);
    k += kRound;
    off += kRound;
    if (off >= g.P) {  // crossed into the next chunk of every A^T row
      while (off >= g.P) { off -= g.P; ++c; }
      load_pages();
    }
  }

  // waves 1..3 hand their partial sums to wave 0, which adds them in wave order
#pragma unroll
  for (int cb0 = 0; cb0 < NB; cb0 += kRedCb) {
    if (wave > 0) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int cc = 0; cc < kRedCb; ++cc)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            red[(((wave - 1) * 4 + tb) * kRedCb * 4 + cc * 4 + q) * 64 + lane] = acc[tb][cb0 + cc][q];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int cc = 0; cc < kRedCb; ++cc) {
          const int n = (cb0 + cc) * 16 + li;  // rank row of this lane's results
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float s = acc[tb][cb0 + cc][q];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
              s += red[(((w - 1) * 4 + tb) * kRedCb * 4 + cc * 4 + q) * 64 + lane];
            const int t = __shfl(tk[tb], 4 * kg + q);  // token of result row 4 * kg + q
            if (t >= 0 && n < r) vpart[ks * split_stride + (int64_t)t * g.r_max + n] = s;
          }
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ expand
constexpr int kCols = kSgCols;             // output columns per workgroup (64 per wave)
constexpr int kBPitch = kCols + 4;         // B chunk row pitch in elements (bank spread)
constexpr int kChunkRows = kStep;          // B rows staged per chunk

// KB: 32-row chunks of the rank (rank <= 32 * KB).
template <int DT, int KB>
__global__ __launch_bounds__(64 * kWaves) void sgmv_expand_kernel(
    Geom g, const SgTile* __restrict__ tiles, const int32_t* __restrict__ tok, int32_t ksplit,
    const float* __restrict__ vpart, int64_t split_stride, uint16_t* __restrict__ y) {
  constexpr int kRp = KB * kStep;     // padded rank
  constexpr int kVPitch = kRp + 8;    // v row pitch in elements
  __shared__ uint16_t vs[kTileRows * kVPitch];
  __shared__ uint16_t bs[kChunkRows * kBPitch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kg = lane >> 4;
  const SgTile tl = tiles[blockIdx.x];
  const int c0 = blockIdx.y * kCols;
  const int r = tl.rank;

  int tk[4];  // token of operand row tb * 16 + li (the v^T operand's column)
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) tk[tb] = tile_token(tl, tok, tb * 16 + li);

  // y0 of this lane's outputs: token tk[tb], columns c0 + wave * 64 + p * 32 + kg * 8 + [0, 8)
  uint4 y0v[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int col = c0 + wave * 64 + p * 32 + kg * 8;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      y0v[p][tb] = ld16(tk[tb] >= 0 && col < g.d_out ? y + (int64_t)tk[tb] * g.d_out + col : fill_zero());
  }

  // v: sum of the k-range partials (in range order), rounded once, into LDS
  {
    constexpr int kThreadsPerRow = (64 * kWaves) / kTileRows;  // 4
    constexpr int kPerThread = kRp / kThreadsPerRow;           // multiple of 4
    static_assert(kPerThread % 4 == 0, "v staging split");
    const int row = tid / kThreadsPerRow, part = tid % kThreadsPerRow;
    const int t = tile_token(tl, tok, row);
#pragma unroll
    for (int q = 0; q < kPerThread; q += 4) {
      const int kk = part * kPerThread + q;
      float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t >= 0) {
        for (int sp = 0; sp < ksplit; ++sp) {
          const float* src = vpart + sp * split_stride + (int64_t)t * g.r_max + kk;
          // rows at or past the rank were never written: read as zero
          float4 a;
          a.x = kk + 0 < r ? src[0] : 0.f;
          a.y = kk + 1 < r ? src[1] : 0.f;
          a.z = kk + 2 < r ? src[2] : 0.f;
          a.w = kk + 3 < r ? src[3] : 0.f;
          s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
        }
      }
      uint2 packed;
      packed.x = pack2<DT>(s.x, s.y);
      packed.y = pack2<DT>(s.z, s.w);
      *reinterpret_cast<uint2*>(&vs[row * kVPitch + kk]) = packed;
    }
  }

  // B staging: thread -> column slot (8 columns) and rows; its page chunk is fixed
  const int slot = tid & 31, row0 = tid >> 5;  // 8 rows per pass, 4 passes per chunk
  const int bcol = c0 + slot * 8;
  const bool bcol_live = bcol < g.d_out;
  const int bc = bcol_live ? bcol / g.P : 0;
  const int boff = bcol - bc * g.P;
  const int64_t bbase = (int64_t)tl.pt_base + (int64_t)r * g.cA + bc;
  auto load_b = [&](uint4 (&b)[4], int chunk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = chunk * kChunkRows + row0 + i * 8;
      const uint16_t* p = fill_zero();
      if (bcol_live && kr < r) {
        const int page = g.pt[bbase + (int64_t)kr * g.cB];
        p = (uint32_t)page < (uint64_t)g.n_pages ? g.pool + (int64_t)page * g.P + boff : fill_nan<DT>();
      }
      b[i] = ld16(p);
    }
  };
  auto store_b = [&](const uint4 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2* d = reinterpret_cast<uint2*>(&bs[(row0 + i * 8) * kBPitch + slot * 8]);
      d[0] = make_uint2(b[i].x, b[i].y);
      d[1] = make_uint2(b[i].z, b[i].w);
    }
  };

  f32x4 acc[2][2][4];  // [pair][half][token block]
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[p][h][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 bn[4];
  load_b(bn, 0);
#pragma unroll
  for (int ch = 0; ch < KB; ++ch) {
    if (ch > 0) __syncthreads();  // the previous chunk has been read
    store_b(bn);
    if (ch + 1 < KB) load_b(bn, ch + 1);
    __syncthreads();
    // v^T operand: token tb * 16 + li, k = ch * 32 + kg * 8 + [0, 8)
    uint4 vo[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      vo[tb] = *reinterpret_cast<const uint4*>(&vs[(tb * 16 + li) * kVPitch + ch * kStep + kg * 8]);
    // B^T operand: output column (p, h, li) = p * 32 + (li / 4) * 8 + h * 4 + li % 4 of this
    // wave's 64, k = kg * 8 + [0, 8) of the chunk
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int colw = wave * 64 + p * 32 + (li >> 2) * 8 + h * 4 + (li & 3);
        const uint16_t* src = &bs[(kg * 8) * kBPitch + colw];
        uint4 bo;
        bo.x = (uint32_t)src[0 * kBPitch] | ((uint32_t)src[1 * kBPitch] << 16);
        bo.y = (uint32_t)src[2 * kBPitch] | ((uint32_t)src[3 * kBPitch] << 16);
        bo.z = (uint32_t)src[4 * kBPitch] | ((uint32_t)src[5 * kBPitch] << 16);
        bo.w = (uint32_t)src[6 * kBPitch] | ((uint32_t)src[7 * kBPitch] << 16);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[p][h][tb] = mfma<DT>(bo, vo[tb], acc[p][h][tb]);
      }
  }

  // lane: token tk[tb], columns c0 + wave * 64 + p * 32 + kg * 8 + h * 4 + q
  const float s = tl.scale;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int col = c0 + wave * 64 + p * 32 + kg * 8;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if (tk[tb] < 0 || col >= g.d_out) continue;
      const uint4 y0 = y0v[p][tb];
      const f32x4 a = acc[p][0][tb], b = acc[p][1][tb];
      uint4 o;
      o.x = pack2<DT>(fmaf(s, a[0], lo_f32<DT>(y0.x)), fmaf(s, a[1], hi_f32<DT>(y0.x)));
      o.y = pack2<DT>(fmaf(s, a[2], lo_f32<DT>(y0.y)), fmaf(s, a[3], hi_f32<DT>(y0.y)));
      o.z = pack2<DT>(fmaf(s, b[0], lo_f32<DT>(y0.z)), fmaf(s, b[1], hi_f32<DT>(y0.z)));
      o.w = pack2<DT>(fmaf(s, b[2], lo_f32<DT>(y0.w)), fmaf(s, b[3], hi_f32<DT>(y0.w)));
      st16(y + (int64_t)tk[tb] * g.d_out + col, o);
    }
  }
}

template <int DT>
hipError_t shrink_dt(const Geom& g, const int32_t* tok, const SgTile* tiles, int32_t n_tiles,
                     int32_t ksplit, int32_t kc, int32_t nb, const void* x, float* vpart,
                     int64_t split_stride, hipStream_t s) {
  const dim3 grid((unsigned)n_tiles, (unsigned)ksplit), block(64 * kWaves);
  const size_t lds = (size_t)3 * 4 * (nb < 4 ? nb : 4) * 4 * 64 * sizeof(float);
  const uint16_t* xp = (const uint16_t*)x;
  switch (nb) {
    case 1: hipLaunchKernelGGL((sgmv_shrink_kernel<DT, 1>), grid, block, lds, s, g, tiles, tok, kc, xp, vpart, split_stride); break;
    case 2: hipLaunchKernelGGL((sgmv_shrink_kernel<DT, 2>), grid, block, lds, s, g, tiles, tok, kc, xp, vpart, split_stride); break;
    case 4: hipLaunchKernelGGL((sgmv_shrink_kernel<DT, 4>), grid, block, lds, s, g, tiles, tok, kc, xp, vpart, split_stride); break;
    default: hipLaunchKernelGGL((sgmv_shrink_kernel<DT, 8>), grid, block, lds, s, g, tiles, tok, kc, xp, vpart, split_stride); break;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t expand_dt(const Geom& g, const int32_t* tok, const SgTile* tiles, int32_t n_tiles,
                     int32_t ksplit, int32_t kb, const float* vpart, int64_t split_stride, void* y,
                     hipStream_t s) {
  const dim3 grid((unsigned)n_tiles, (unsigned)((g.d_out + kCols - 1) / kCols)), block(64 * kWaves);
  uint16_t* yp = (uint16_t*)y;
  switch (kb) {
    case 1: hipLaunchKernelGGL((sgmv_expand_kernel<DT, 1>), grid, block, 0, s, g, tiles, tok, ksplit, vpart, split_stride, yp); break;
    case 2: hipLaunchKernelGGL((sgmv_expand_kernel<DT, 2>), grid, block, 0, s, g, tiles, tok, ksplit, vpart, split_stride, yp); break;
    default: hipLaunchKernelGGL((sgmv_expand_kernel<DT, 4>), grid, block, 0, s, g, tiles, tok, ksplit, vpart, split_stride, yp); break;
  }
  return hipGetLastError();
}

}  // namespace

SgSplit sg_split(int32_t d_in, int32_t n_tiles) {
  SgSplit o;
  int32_t ks = n_tiles > 0 ? (1024 + n_tiles - 1) / n_tiles : 1;
  ks = std::max(1, std::min(ks, sg_max_split(d_in)));
  const int32_t per = (d_in + ks - 1) / ks;
  o.kc = (per + kRound - 1) / kRound * kRound;
  o.ksplit = (d_in + o.kc - 1) / o.kc;
  return o;
}

hipError_t launch_sgmv_shrink(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit, int32_t kc,
                              const void* x, float* vpart, int64_t split_stride, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (max_rank < 1 || max_rank > kMaxRank || ksplit < 1 || kc % kRound) return hipErrorInvalidValue;
  const int nb = max_rank <= 16 ? 1 : max_rank <= 32 ? 2 : max_rank <= 64 ? 4 : 8;
  return g.dtype == SLORA_F16
             ? shrink_dt<SLORA_F16>(g, tok, tiles, n_tiles, ksplit, kc, nb, x, vpart, split_stride, s)
             : shrink_dt<SLORA_BF16>(g, tok, tiles, n_tiles, ksplit, kc, nb, x, vpart, split_stride, s);
}

hipError_t launch_sgmv_expand(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit,
                              const float* vpart, int64_t split_stride, void* y, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (max_rank < 1 || max_rank > kMaxRank || ksplit < 1) return hipErrorInvalidValue;
  const int kb = max_rank <= 32 ? 1 : max_rank <= 64 ? 2 : 4;
  return g.dtype == SLORA_F16
             ? expand_dt<SLORA_F16>(g, tok, tiles, n_tiles, ksplit, kb, vpart, split_stride, y, s)
             : expand_dt<SLORA_BF16>(g, tok, tiles, n_tiles, ksplit, kb, vpart, split_stride, y, s);
}

}  // namespace slora

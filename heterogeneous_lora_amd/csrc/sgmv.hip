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
//     x rows (the tile's tokens) and A^T rows (rank rows, gathered through the
//     page table) are both contiguous in j, so both operands are plain 16-byte
//     loads. Each wave owns 16 tokens and reads its x rows straight from global
//     memory; the A^T rows, which all 4 waves need, pass through LDS once per
//     workgroup. The k-ranges give a launch of one projection enough workgroups to
//     fill the chip without spilling into a second round (a launch of several
//     projections has enough without them: sg_split); the expand adds the ranges'
//     partial sums in range order, so the result does not depend on scheduling.
//   expand (tile, 1024 output columns): y[t, n] = RNE(y0 + s * sum_k v[t, k] B[k, n]).
//     The product is computed transposed, D = B^T v^T, so that each lane ends up
//     with 8 consecutive output columns of one token (16-byte y0 loads and y
//     stores). v (summed over k-ranges, rounded once to the storage type to feed
//     the matrix cores) is staged in LDS once; the columns are walked in passes of
//     128 (32 per wave) whose B rows pass through LDS in 32-row chunks, the B^T
//     operand read out column-wise, while the next pass's y0 is already loading.
//
// slora_apply runs both halves in one launch (sgmv_fused_kernel): the first
// n_tiles * ksplit workgroups are the shrink items, the rest the expand items. A
// shrink item stores its partial sums at device (agent) scope, waits for its stores,
// and then stores its flag word (the call's tag); an expand item polls its tile's
// ksplit flags before it reads the partial sums, also at agent scope, so neither side
// needs a cache flush. Shrink items precede every expand item in dispatch order and
// never wait, so every wait ends; the poll is bounded all the same, and a give-up is
// recorded in the workspace header. One launch instead of two removes the drain of
// the shrink grid before the expand grid can start. slora_shrink / slora_expand keep
// the two separate kernels. A call that also has decode groups runs them in the same
// launch (mixed_fused_kernel, with the MBGMV bodies of mbgmv_dev.h): every shrink item
// of both families first, then every expand item.
#include <algorithm>

#include <map>
#include <mutex>
#include <tuple>

#include "device_common.h"
#include "mbgmv_dev.h"

namespace slora {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

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

// v_mfma_f32_16x16x16_{f16,bf16}: the same layout with 4 consecutive k per lane (at
// (l / 16) * 4), for operands of 16 rows of k (ranks up to 16).
template <int DT>
__device__ __forceinline__ f32x4 mfma16(const uint2& a, const uint2& b, f32x4 c) {
  if constexpr (DT == SLORA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Token of row m of a tile, or -1 past its end.
__device__ __forceinline__ int tile_token(const SgTile& tl, const int32_t* tok, int m) {
  if (m >= tl.n_tok) return -1;
  return tl.first_tok >= 0 ? tl.first_tok + m : tok[tl.tok_begin + m];
}

// ------------------------------------------------------------------ shrink
// NB: 16-row blocks of rank rows (rank <= 16 * NB). Wave w owns the tile's token
// rows 16 w .. 16 w + 15 and every rank row, so no partial sums cross waves.
// The k-range is walked in batches of 128: the batch's A^T slab (16 NB rows x 256 B)
// sits in one of two LDS buffers while the next batch's slab and x rows load into
// registers. In the slab, the 16-byte segment s of row n is stored at position
// s ^ (n % 16), so the 16 rows an MFMA operand read touches land in 16 different
// bank groups.
constexpr int kBatch = 4 * kStep;  // k per batch
constexpr int kSegs = kBatch / 8;  // 16-byte segments per slab row

// Waves per SIMD the register allocation must leave room for. Left to itself the
// compiler spreads these kernels over the unified register file (accumulation
// registers included) and lands at 3 (shrink, NB = 4) or 2 (expand, KB = 2) waves per
// SIMD; the same code fits 4 and 3 without spilling, and the extra resident waves
// keep more loads in flight. The widest expand (KB = 4, ranks above 64) spills ~16
// registers per lane at 3 waves per SIMD and is still faster than at 2 (a launch over
// all of a mixed batch's tiles: 73 -> 63 us). The widest shrink is held to 2 by its
// 64 KB LDS slab whatever its registers.
constexpr int shrink_waves(int nb) { return nb <= 4 ? 4 : 1; }
constexpr int expand_waves(int kb) { return kb <= 1 ? 4 : 3; }
constexpr int32_t kSgMinSplit = 3;       // k-ranges at least, one projection per launch
constexpr int32_t kSgMinSplitMulti = 1;  // the same, several projections in one launch
// 16-row blocks of rank rows the shrink template for ranks up to max_rank holds.
constexpr int shrink_nb(int max_rank) { return max_rank <= 16 ? 1 : max_rank <= 32 ? 2 : max_rank <= 64 ? 4 : 8; }

// One (tile, k-range) with NB 16-row blocks of rank rows from row0 on; slab holds
// 2 x 16 NB x kSegs vectors. kCoherent: the partial sums are stored at agent scope
// (performed at the device's coherence point), for a reader in the same launch.
template <int DT, int NB, bool kCoherent = false>
__device__ __forceinline__ void shrink_tile(const Geom& g, const SgTile& tl,
                                            const int32_t* __restrict__ tok, int32_t kc,
                                            const uint16_t* __restrict__ x,
                                            float* __restrict__ vpart, int32_t v_stride,
                                            int64_t split_stride, int ks, uint4* slab_mem,
                                            int row0 = 0) {
  constexpr int kRows = 16 * NB;
  constexpr int kLoads = kRows * kSegs / (64 * kWaves);  // slab vectors per thread
  static_assert(kLoads >= 1 && kRows * kSegs == kLoads * 64 * kWaves, "slab split");
  uint4 (*slab)[kRows * kSegs] = reinterpret_cast<uint4 (*)[kRows * kSegs]>(slab_mem);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kg = lane >> 4;
  const int kb = ks * kc, ke = min(g.d_in, kb + kc);
  const int r = tl.rank;
  const int n_batch = (ke - kb + kBatch - 1) / kBatch;

  const int tk = tile_token(tl, tok, wave * 16 + li);  // this lane's x row
  const uint16_t* xrow = tk >= 0 ? x + (int64_t)tk * g.d_in : nullptr;

  // slab staging: thread -> slab position i * 256 + tid, i.e. row i * 16 + tid / 16 and
  // stored segment tid % 16, which holds logical segment ls of that row
  const int srow = tid >> 4, ls = (tid & 15) ^ srow;
  const uint16_t* prow[kLoads];  // page of row i * 16 + srow in chunk cur_c, or a fill vector
  bool preal[kLoads];
  int cur_c = -1;
  auto load_slab = [&](uint4 (&v)[kLoads], int bt) {
    const int k = kb + bt * kBatch + ls * 8;
    const bool live = k < ke;
    const int c = live ? k / g.P : cur_c;
    if (live && c != cur_c) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int n = row0 + i * 16 + srow;
        const uint16_t* p = fill_zero();
        bool real = false;
        if (n < r && c < g.cA) {
          const int page = g.pt[(int64_t)tl.pt_base + (int64_t)n * g.cA + c];
          real = (uint32_t)page < (uint64_t)g.n_pages;
          p = real ? g.pool + (int64_t)page * g.P : fill_nan<DT>();
        }
        prow[i] = p;
        preal[i] = real;
      }
      cur_c = c;
    }
    const int off = k - c * g.P;
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      v[i] = ld16(!live ? fill_zero() : preal[i] ? prow[i] + off : prow[i]);
  };
  auto store_slab = [&](const uint4 (&v)[kLoads], int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) slab[buf][i * 256 + tid] = v[i];
  };
  auto load_x = [&](uint4 (&xv)[4], int bt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kb + bt * kBatch + s * kStep + kg * 8;
      xv[s] = ld16(xrow && k < ke ? xrow + k : fill_zero());
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const uint4 (&xv)[4], int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int n = cb * 16 + li;
        const uint4 av = slab[buf][n * kSegs + ((s * 4 + kg) ^ li)];
        acc[cb] = mfma<DT>(xv[s], av, acc[cb]);
      }
  };

  // batch bt multiplies out of slab[bt % 2] and x buffer bt % 2 while batch bt + 1 loads
  uint4 sv[kLoads], x0[4], x1[4];
  if (n_batch > 0) {
    load_slab(sv, 0);
    load_x(x0, 0);
    store_slab(sv, 0);
    if (n_batch > 1) { load_slab(sv, 1); load_x(x1, 1); }
  }
  __syncthreads();
  for (int bt = 0; bt < n_batch; bt += 2) {
    mma(x0, 0);
    if (bt + 1 >= n_batch) break;
    store_slab(sv, 1);
    if (bt + 2 < n_batch) { load_slab(sv, bt + 2); load_x(x0, bt + 2); }
    __syncthreads();
    mma(x1, 1);
    if (bt + 2 >= n_batch) break;
    store_slab(sv, 0);
    if (bt + 3 < n_batch) { load_slab(sv, bt + 3); load_x(x1, bt + 3); }
    __syncthreads();
  }

  // lane: token row 4 kg + q of this wave's block, rank row cb * 16 + li
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = __shfl(tk, 4 * kg + q);
    if (t < 0) continue;
    float* dst = vpart + ks * split_stride + (int64_t)t * v_stride;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int n = row0 + cb * 16 + li;
      if (n >= r) continue;
      if constexpr (kCoherent)
        __hip_atomic_store(dst + n, acc[cb][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        dst[n] = acc[cb][q];
    }
  }
}

// The narrowest shrink body that holds the tile's rank, within a launch whose widest is NBM.
template <int DT, int NBM, bool kCoherent>
__device__ __forceinline__ void shrink_any(const Geom& g, const SgTile& tl,
                                           const int32_t* __restrict__ tok, int32_t kc,
                                           const uint16_t* __restrict__ x, float* vpart,
                                           int32_t v_stride, int64_t split_stride, int ks,
                                           uint4* slab) {
  const int nb = shrink_nb(tl.rank);
  if (NBM >= 8 && nb == 8) shrink_tile<DT, NBM >= 8 ? 8 : NBM, kCoherent>(g, tl, tok, kc, x, vpart, v_stride, split_stride, ks, slab);
  else if (NBM >= 4 && nb == 4) shrink_tile<DT, NBM >= 4 ? 4 : NBM, kCoherent>(g, tl, tok, kc, x, vpart, v_stride, split_stride, ks, slab);
  else if (NBM >= 2 && nb == 2) shrink_tile<DT, NBM >= 2 ? 2 : NBM, kCoherent>(g, tl, tok, kc, x, vpart, v_stride, split_stride, ks, slab);
  else shrink_tile<DT, 1, kCoherent>(g, tl, tok, kc, x, vpart, v_stride, split_stride, ks, slab);
}

// NBM: the widest template of the launch (its registers, LDS and occupancy); each tile
// runs the narrowest one that holds its rank, so a low-rank tile loads, stages and
// multiplies only its own rows (the branch is uniform per workgroup and taken once).
template <int DT, int NBM>
__global__ __launch_bounds__(64 * kWaves, shrink_waves(NBM)) void sgmv_shrink_kernel(
    Geom g, const SgTile* __restrict__ tiles, const int32_t* __restrict__ tok, int32_t kc,
    const uint16_t* __restrict__ x, float* __restrict__ vpart, int32_t v_stride,
    int64_t split_stride) {
  __shared__ uint4 slab[2 * 16 * NBM * kSegs];
  const SgTile tl = tiles[blockIdx.x];
  shrink_any<DT, NBM, false>(g, tl, tok, kc, x, vpart, v_stride, split_stride, (int)blockIdx.y, slab);
}

// ------------------------------------------------------------------ expand
constexpr int kCols = 128;                 // output columns of one pass (32 per wave)
constexpr int kSubPasses = 8;              // passes per workgroup (1024 columns)
constexpr int kBPitch = kCols + 4;         // B chunk row pitch in elements (bank spread)
constexpr int kChunkRows = kStep;          // B rows staged per chunk

// LDS of the expand template for KB 32-row chunks: v rows, then the B stages.
constexpr int expand_vs_elems(int kb) { return kTileRows * (kb * kStep + 8); }
constexpr int expand_bbufs(int kb) { return kb <= 2 ? 2 : 1; }  // two B stages: one barrier per pass
constexpr int expand_bs_elems(int kb) { return expand_bbufs(kb) * kb * kChunkRows * kBPitch; }

// One (tile, column block) with KB chunks of KS rows of the rank (rank <= KS * KB); KS is
// the k of one product: 32 (16x16x32), or 16 (16x16x16) for ranks up to 16.
// kCoherent: the partial sums are read at agent scope (written in the same launch).
template <int DT, int KB, int KS = kStep, bool kCoherent = false>
__device__ __forceinline__ void expand_tile(const Geom& g, const SgTile& tl,
                                            const int32_t* __restrict__ tok, int32_t ksplit,
                                            const float* __restrict__ vpart, int32_t v_stride,
                                            int64_t split_stride, uint16_t* __restrict__ y,
                                            int cblock, uint16_t* vs, uint16_t* bs) {
  static_assert(KS == 16 || KS == 32, "k per product");
  constexpr int kRp = KB * KS;        // padded rank
  constexpr int kVPitch = kRp + 8;    // v row pitch in elements
  constexpr int kBBufs = expand_bbufs(KB);
  constexpr int kChunk = KS;          // B rows staged per chunk
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kg = lane >> 4;
  const int r = tl.rank;
  const int col_begin = cblock * (kSubPasses * kCols);
  const int n_pass = min(kSubPasses, (g.d_out - col_begin + kCols - 1) / kCols);

  int tk[4];  // token of operand row tb * 16 + li (the v^T operand's column)
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) tk[tb] = tile_token(tl, tok, tb * 16 + li);

  // B staging: thread -> column slot (8 columns) and rows ch * KS + row0 + 16 i of every
  // chunk. A pass's rows are loaded in one go, a pass ahead; the page ids of the
  // thread's rows are kept while the pass's columns stay in the same page chunk.
  constexpr int kSlots = kCols / 8, kRowStep = 64 * kWaves / kSlots, kBLoads = kChunk / kRowStep;
  static_assert(kBLoads >= 1 && kBLoads * kRowStep == kChunk, "B staging split");
  const int slot = tid % kSlots, row0 = tid / kSlots;
  int pid_c = -1;
  int pids[KB][kBLoads];
  auto load_b = [&](uint4 (&b)[KB][kBLoads], int pass) {
    const int bcol = col_begin + pass * kCols + slot * 8;
    const bool live = bcol < g.d_out;
    const int bc = live ? bcol / g.P : 0;
    if (live && bc != pid_c) {
      const int64_t bbase = (int64_t)tl.pt_base + (int64_t)r * g.cA + bc;
#pragma unroll
      for (int ch = 0; ch < KB; ++ch)
#pragma unroll
        for (int i = 0; i < kBLoads; ++i) {
          const int kr = ch * kChunk + row0 + i * kRowStep;
          pids[ch][i] = kr < r ? g.pt[bbase + (int64_t)kr * g.cB] : -1;
        }
      pid_c = bc;
    }
#pragma unroll
    for (int ch = 0; ch < KB; ++ch)
#pragma unroll
      for (int i = 0; i < kBLoads; ++i) {
        const int kr = ch * kChunk + row0 + i * kRowStep;
        const uint16_t* p = fill_zero();
        if (live && kr < r) {
          const int page = pids[ch][i];
          p = (uint32_t)page < (uint64_t)g.n_pages ? g.pool + (int64_t)page * g.P + (bcol - bc * g.P)
                                                   : fill_nan<DT>();
        }
        b[ch][i] = ld16(p);
      }
  };
  auto store_b = [&](const uint4 (&b)[KB][kBLoads], int buf) {
#pragma unroll
    for (int ch = 0; ch < KB; ++ch)
#pragma unroll
      for (int i = 0; i < kBLoads; ++i) {
        uint2* d = reinterpret_cast<uint2*>(&bs[((buf * KB + ch) * kChunk + row0 + i * kRowStep) * kBPitch + slot * 8]);
        d[0] = make_uint2(b[ch][i].x, b[ch][i].y);
        d[1] = make_uint2(b[ch][i].z, b[ch][i].w);
      }
  };
  uint4 bn[KB][kBLoads];
  load_b(bn, 0);  // in flight while v is staged

  // v: the k-range partials added in range order, rounded once, into LDS. Thread:
  // row tid / 4, columns 16 q + 4 (tid % 4) + [0, 4); rows at or past the rank
  // were never written and read as zero.
  {
    const int row = tid >> 2, cq = (tid & 3) * 4;
    const int t = tile_token(tl, tok, row);
    const bool vec = (v_stride & 3) == 0;
#pragma unroll
    for (int q = 0; q < kRp / 16; ++q) {
      const int kk = q * 16 + cq;
      float4 a[kSgMaxSplit];
#pragma unroll
      for (int sp = 0; sp < kSgMaxSplit; ++sp) {
        a[sp] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (sp < ksplit && t >= 0 && kk < r) {
          const float* src = vpart + sp * split_stride + (int64_t)t * v_stride + kk;
          if constexpr (kCoherent) {  // 16-byte aligned rows (v_stride % 4 == 0 in apply calls)
            const unsigned long long* q = reinterpret_cast<const unsigned long long*>(src);
            const unsigned long long w0 = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned long long w1 = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            a[sp] = make_float4(__uint_as_float((unsigned)w0), __uint_as_float((unsigned)(w0 >> 32)),
                                __uint_as_float((unsigned)w1), __uint_as_float((unsigned)(w1 >> 32)));
          } else if (vec) {
            a[sp] = *reinterpret_cast<const float4*>(src);
          } else {
            a[sp].x = src[0];
            a[sp].y = kk + 1 < r ? src[1] : 0.f;
            a[sp].z = kk + 2 < r ? src[2] : 0.f;
            a[sp].w = kk + 3 < r ? src[3] : 0.f;
          }
        }
      }
      float4 sum = a[0];
#pragma unroll
      for (int sp = 1; sp < kSgMaxSplit; ++sp) {
        sum.x += a[sp].x; sum.y += a[sp].y; sum.z += a[sp].z; sum.w += a[sp].w;
      }
      sum.y = kk + 1 < r ? sum.y : 0.f;
      sum.z = kk + 2 < r ? sum.z : 0.f;
      sum.w = kk + 3 < r ? sum.w : 0.f;
      uint2 packed;
      packed.x = pack2<DT>(sum.x, sum.y);
      packed.y = pack2<DT>(sum.z, sum.w);
      *reinterpret_cast<uint2*>(&vs[row * kVPitch + kk]) = packed;
    }
  }

  const float s = tl.scale;
  // y0 of this lane's outputs in a pass: token tk[tb], columns cw + kg * 8 + [0, 8)
  auto load_y0 = [&](uint4 (&yv)[4], int pass) {
    const int col = col_begin + pass * kCols + wave * 32 + kg * 8;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      yv[tb] = ld16(tk[tb] >= 0 && col < g.d_out ? y + (int64_t)tk[tb] * g.d_out + col : fill_zero());
  };
  auto run_pass = [&](int pass, const uint4 (&yv)[4]) {
    f32x4 acc[2][4];  // [half][token block]
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[h][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // With two stages, the one this pass writes was last read in pass - 2, and every wave
    // had finished those reads before it passed pass - 1's barrier; one stage needs a
    // barrier here. Pass 0 waits for v to be staged.
    const int buf = kBBufs == 2 ? (pass & 1) : 0;
    if (kBBufs == 1 || pass == 0) __syncthreads();
    store_b(bn, buf);
    if (pass + 1 < n_pass) load_b(bn, pass + 1);
    __syncthreads();
#pragma unroll
    for (int ch = 0; ch < KB; ++ch) {
      const uint16_t* bsc = bs + (buf * KB + ch) * kChunk * kBPitch;
      constexpr int kPer = KS / 4;  // k of one lane's operand
      // B^T operand: output column (h, li) = (li / 4) * 8 + h * 4 + li % 4 of this wave's 32,
      // k = kg * kPer + [0, kPer) of the chunk; v^T operand: token tb * 16 + li, the same k
      if constexpr (KS == 32) {
        uint4 vo[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          vo[tb] = *reinterpret_cast<const uint4*>(&vs[(tb * 16 + li) * kVPitch + ch * KS + kg * kPer]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int colw = wave * 32 + (li >> 2) * 8 + h * 4 + (li & 3);
          const uint16_t* src = &bsc[(kg * kPer) * kBPitch + colw];
          uint4 bo;
          bo.x = (uint32_t)src[0 * kBPitch] | ((uint32_t)src[1 * kBPitch] << 16);
          bo.y = (uint32_t)src[2 * kBPitch] | ((uint32_t)src[3 * kBPitch] << 16);
          bo.z = (uint32_t)src[4 * kBPitch] | ((uint32_t)src[5 * kBPitch] << 16);
          bo.w = (uint32_t)src[6 * kBPitch] | ((uint32_t)src[7 * kBPitch] << 16);
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) acc[h][tb] = mfma<DT>(bo, vo[tb], acc[h][tb]);
        }
      } else {
        uint2 vo[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          vo[tb] = *reinterpret_cast<const uint2*>(&vs[(tb * 16 + li) * kVPitch + ch * KS + kg * kPer]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int colw = wave * 32 + (li >> 2) * 8 + h * 4 + (li & 3);
          const uint16_t* src = &bsc[(kg * kPer) * kBPitch + colw];
          uint2 bo;
          bo.x = (uint32_t)src[0 * kBPitch] | ((uint32_t)src[1 * kBPitch] << 16);
          bo.y = (uint32_t)src[2 * kBPitch] | ((uint32_t)src[3 * kBPitch] << 16);
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) acc[h][tb] = mfma16<DT>(bo, vo[tb], acc[h][tb]);
        }
      }
    }
    // lane: token tk[tb], columns col + h * 4 + q
    const int col = col_begin + pass * kCols + wave * 32 + kg * 8;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if (tk[tb] < 0 || col >= g.d_out) continue;
      const uint4 y0 = yv[tb];
      const f32x4 a = acc[0][tb], b = acc[1][tb];
      uint4 o;
      o.x = pack2<DT>(fmaf(s, a[0], lo_f32<DT>(y0.x)), fmaf(s, a[1], hi_f32<DT>(y0.x)));
      o.y = pack2<DT>(fmaf(s, a[2], lo_f32<DT>(y0.y)), fmaf(s, a[3], hi_f32<DT>(y0.y)));
      o.z = pack2<DT>(fmaf(s, b[0], lo_f32<DT>(y0.z)), fmaf(s, b[1], hi_f32<DT>(y0.z)));
      o.w = pack2<DT>(fmaf(s, b[2], lo_f32<DT>(y0.w)), fmaf(s, b[3], hi_f32<DT>(y0.w)));
      st16(y + (int64_t)tk[tb] * g.d_out + col, o);
    }
  };

  // y0 of the next pass loads while a pass multiplies (two named buffers), except in
  // the widest template, which is short of registers: there one y0 buffer is loaded as
  // its pass begins and arrives while the pass stages B and multiplies
  if constexpr (KB >= 4) {
    uint4 ya[4];
    for (int pass = 0; pass < n_pass; ++pass) {
      load_y0(ya, pass);
      run_pass(pass, ya);
    }
  } else {
    uint4 ya[4], yb[4];
    load_y0(ya, 0);
    for (int pass = 0; pass < n_pass; pass += 2) {
      if (pass + 1 < n_pass) load_y0(yb, pass + 1);
      run_pass(pass, ya);
      if (pass + 1 >= n_pass) break;
      if (pass + 2 < n_pass) load_y0(ya, pass + 2);
      run_pass(pass + 1, yb);
    }
  }
}

// The narrowest expand body that holds the tile's rank, within a launch whose widest is KBM
// (the widest launch keeps its one body, see below).
template <int DT, int KBM, bool kCoherent>
__device__ __forceinline__ void expand_any(const Geom& g, const SgTile& tl,
                                           const int32_t* __restrict__ tok, int32_t ksplit,
                                           const float* vpart, int32_t v_stride,
                                           int64_t split_stride, uint16_t* __restrict__ y,
                                           int cblock, uint16_t* vs, uint16_t* bs) {
  if constexpr (KBM >= 4) {
    expand_tile<DT, 4, kStep, kCoherent>(g, tl, tok, ksplit, vpart, v_stride, split_stride, y, cblock, vs, bs);
  } else {
    if (KBM >= 2 && tl.rank > 32) expand_tile<DT, KBM, kStep, kCoherent>(g, tl, tok, ksplit, vpart, v_stride, split_stride, y, cblock, vs, bs);
    else if (tl.rank > 16) expand_tile<DT, 1, kStep, kCoherent>(g, tl, tok, ksplit, vpart, v_stride, split_stride, y, cblock, vs, bs);
    else expand_tile<DT, 1, 16, kCoherent>(g, tl, tok, ksplit, vpart, v_stride, split_stride, y, cblock, vs, bs);
  }
}

// KBM: the widest template of the launch (its registers, LDS and occupancy); each tile
// runs the narrowest one that holds its rank (uniform per workgroup, taken once). The
// widest launch (ranks above 64) keeps its one body: next to the narrower bodies its
// register spills grew (36 -> 44 bytes per lane) and mixed_13b's expand slowed
// (60.2 -> 62.6 us), while the narrower launches gained (prefill_sgmv expand 90.5 ->
// 88.1 us, shrink 50.9 -> 49.8 us; mlp_asym shrink 121.8 -> 117.5 us).
template <int DT, int KBM>
__global__ __launch_bounds__(64 * kWaves, expand_waves(KBM)) void sgmv_expand_kernel(
    Geom g, const SgTile* __restrict__ tiles, const int32_t* __restrict__ tok, int32_t ksplit,
    const float* __restrict__ vpart, int32_t v_stride, int64_t split_stride,
    uint16_t* __restrict__ y) {
  constexpr int kBsMax = expand_bs_elems(KBM) > expand_bs_elems(2) ? expand_bs_elems(KBM) : expand_bs_elems(2);
  __shared__ uint16_t vs[expand_vs_elems(KBM)];
  __shared__ uint16_t bs[KBM >= 2 ? kBsMax : expand_bs_elems(1)];
  const SgTile tl = tiles[blockIdx.x];
  expand_any<DT, KBM, false>(g, tl, tok, ksplit, vpart, v_stride, split_stride, y, (int)blockIdx.y, vs, bs);
}

// ------------------------------------------------------------------ fused (apply calls)
// Shrink and expand of one projection in one launch. The first workgroups are shrink
// items, the rest expand items (tile, column block), tile-major. Shrink items are
// (tile, k-range) with one exception: in a launch over ranks above 64 (NBM = 4, KBM = 4),
// each of the first n_wide tiles (those of rank above 64; tiles come in descending rank)
// is shrunk as two 64-row blocks, items (tile, block, k-range), so that the launch needs
// the 64-row shrink body only and keeps the expand's occupancy (3 workgroups per CU,
// where the 128-row body's 64 KB slab allows 2). Each block writes its own rows of the
// k-range's partial sums. Shrink item i stores its partial sums at agent scope, waits
// until they are performed, then stores the call's tag into flags[i]; an expand item
// polls its tile's flags (bounded; a give-up is recorded in the workspace header) and
// reads the partial sums at agent scope. Workgroups are dispatched in index order and
// shrink items never wait, so every shrink item an expand item waits for has been
// dispatched before it and finishes. The expand items take the slots the shrink items
// free at the end of their phase, which two launches would leave idle.
constexpr int fused_waves(int nbm, int kbm) {
  return shrink_waves(nbm) < expand_waves(kbm) ? shrink_waves(nbm) : expand_waves(kbm);
}
// LDS of a fused launch: the larger of its shrink slab and its expand stages (v rows,
// then B stages sized as the expand kernel sizes them).
constexpr int fused_lds_bytes(int nbm, int kbm) {
  const int slab = 2 * 16 * nbm * kSegs * 16;
  const int bs_wide = expand_bs_elems(kbm) > expand_bs_elems(2) ? expand_bs_elems(kbm) : expand_bs_elems(2);
  const int stages = (expand_vs_elems(kbm) + (kbm >= 2 ? bs_wide : expand_bs_elems(1))) * 2;
  return slab > stages ? slab : stages;
}

// A fused launch's segment work (kernel arguments). n_wide: the leading tiles shrunk in
// two 64-row blocks (used only by the NBM = 4, KBM = 4 template).
struct SgWork {
  const SgTile* tiles;
  const int32_t* tok;
  int32_t kc, ksplit, n_tiles, n_wide;
  float* vpart;
  int32_t v_stride;
  int64_t split_stride;
  uint32_t* flags;
};

template <int NBM, int KBM>
__device__ __forceinline__ int sg_wide(const SgWork& w) { return NBM == 4 && KBM == 4 ? w.n_wide : 0; }
template <int NBM, int KBM>
__device__ __forceinline__ int sg_shrink_items(const SgWork& w) { return (w.n_tiles + sg_wide<NBM, KBM>(w)) * w.ksplit; }
__device__ __forceinline__ int sg_expand_blocks(const Geom& g) {
  return (g.d_out + kSubPasses * kCols - 1) / (kSubPasses * kCols);
}

// Shrink item L: its partial sums, then its flag word.
template <int DT, int NBM, int KBM>
__device__ __forceinline__ void sg_shrink_item(const Geom& g, const SgWork& w,
                                               const uint16_t* __restrict__ x, uint32_t tag, int L,
                                               uint4* lds) {
  const int nw = sg_wide<NBM, KBM>(w);
  const int n_wide_items = 2 * nw * w.ksplit;
  if (NBM == 4 && KBM == 4 && L < n_wide_items) {
    const SgTile tl = w.tiles[L / (2 * w.ksplit)];
    shrink_tile<DT, 4, true>(g, tl, w.tok, w.kc, x, w.vpart, w.v_stride, w.split_stride,
                             L % w.ksplit, lds, 64 * ((L / w.ksplit) & 1));
  } else {
    const int l2 = L - n_wide_items;
    const SgTile tl = w.tiles[nw + l2 / w.ksplit];
    shrink_any<DT, NBM, true>(g, tl, w.tok, w.kc, x, w.vpart, w.v_stride, w.split_stride,
                              l2 % w.ksplit, lds);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are performed
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(w.flags + L, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Expand item E (tile E / column blocks, column block E % column blocks): waits for the
// tile's flags, then expands.
template <int DT, int NBM, int KBM>
__device__ __forceinline__ void sg_expand_item(const Geom& g, const SgWork& w, uint32_t tag,
                                               int32_t spin_limit, unsigned long long* err,
                                               uint16_t* __restrict__ y, int E, uint4* lds) {
  const int nw = sg_wide<NBM, KBM>(w);
  const int ncb = sg_expand_blocks(g);
  const int t = E / ncb;
  const int f0 = t < nw ? 2 * t * w.ksplit : 2 * nw * w.ksplit + (t - nw) * w.ksplit;
  const int nf = t < nw ? 2 * w.ksplit : w.ksplit;
  if (threadIdx.x < 64) {
    const int lane = (int)threadIdx.x;
    for (int spins = 0;; ++spins) {
      const bool ok = lane >= nf ||
                      __hip_atomic_load(w.flags + f0 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
      if (__all(ok)) break;
      if (spins >= spin_limit) {
        if (lane == 0) __hip_atomic_store(err, (unsigned long long)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  const SgTile tl = w.tiles[t];
  uint16_t* vs = reinterpret_cast<uint16_t*>(lds);
  expand_any<DT, KBM, true>(g, tl, w.tok, w.ksplit, w.vpart, w.v_stride, w.split_stride, y, E % ncb,
                            vs, vs + expand_vs_elems(KBM));
}

template <int DT, int NBM, int KBM>
__global__ __launch_bounds__(64 * kWaves, fused_waves(NBM, KBM)) void sgmv_fused_kernel(
    Geom g, const SgTile* __restrict__ tiles, const int32_t* __restrict__ tok, int32_t kc,
    int32_t ksplit, int32_t n_tiles, int32_t n_wide, const uint16_t* __restrict__ x,
    float* vpart, int32_t v_stride, int64_t split_stride, uint32_t* flags, uint32_t tag,
    int32_t spin_limit, unsigned long long* err, uint16_t* __restrict__ y) {
  __shared__ uint4 lds[(fused_lds_bytes(NBM, KBM) + 15) / 16];
  const SgWork w{tiles, tok, kc, ksplit, n_tiles, n_wide, vpart, v_stride, split_stride, flags};
  const int L = (int)blockIdx.x;
  const int n_shrink = sg_shrink_items<NBM, KBM>(w);
  if (L < n_shrink) sg_shrink_item<DT, NBM, KBM>(g, w, x, tag, L, lds);
  else sg_expand_item<DT, NBM, KBM>(g, w, tag, spin_limit, err, y, L - n_shrink, lds);
}

// ------------------------------------------------------------------ both families, several projections
// A call with decode groups (MBGMV items) and segment tiles runs both families in one
// launch, so that one family's ramp and tail overlap the other's work and the stream
// has one launch instead of two; a call over several projections of one batch (same
// routing and adapters, one page table, x, y and workspace region each) runs all of
// them in that launch too. Workgroups: [MBGMV shrink items][segment shrink items]
// [MBGMV expand items][segment expand items]; inside a part the projections take turns
// item by item, so the launch runs every projection's costliest items (groups and tiles
// come by descending rank) before any projection's cheapest, and its tail is short
// (item i of projection p is workgroup part_start + i * n_proj + p). Every shrink
// item of either family and any projection comes before every expand item and none
// waits, so the in-order-dispatch argument holds for every hand-off (v words for
// MBGMV, flags for the segments, each in its projection's workspace region); they
// share the call's tag and the first region's give-up word. LDS is the larger of the
// two families' needs.
struct Projs {
  ProjIO p[kMaxProj];
};

template <int DT, bool kUniformChunk, int NBM, int KBM>
__global__ __launch_bounds__(64 * kWaves, fused_waves(NBM, KBM)) void mixed_fused_kernel(
    Geom g, SgWork w, const MbItem* __restrict__ items, int32_t n_mb, int32_t n_mb_shrink,
    Projs pr, int32_t n_proj, uint32_t tag, int32_t spin_limit, unsigned long long* err) {
  constexpr int kMbBytes = mb::kRedBytes > kMbGroup * mb::kBatchVecs * 16 ? mb::kRedBytes : kMbGroup * mb::kBatchVecs * 16;
  constexpr int kBytes = fused_lds_bytes(NBM, KBM) > kMbBytes ? fused_lds_bytes(NBM, KBM) : kMbBytes;
  __shared__ uint4 lds[(kBytes + 15) / 16];
  const int a = n_mb_shrink, b = sg_shrink_items<NBM, KBM>(w), c = n_mb - n_mb_shrink;
  int L = (int)blockIdx.x, part, p, i;
  if (L < n_proj * a) {
    part = 0, p = L % n_proj, i = L / n_proj;
  } else if ((L -= n_proj * a) < n_proj * b) {
    part = 1, p = L % n_proj, i = L / n_proj;
  } else if ((L -= n_proj * b) < n_proj * c) {
    part = 2, p = L % n_proj, i = L / n_proj;
  } else {
    L -= n_proj * c;
    part = 3, p = L % n_proj, i = L / n_proj;
  }
  const ProjIO io = pr.p[p];
  Geom gp = g;
  gp.pt = io.pt;
  const uint16_t* x = static_cast<const uint16_t*>(io.x);
  uint16_t* y = static_cast<uint16_t*>(io.y);
  if (part == 0 || part == 2) {
    const MbItem it = mb::load_item(items, part == 0 ? i : a + i);
    mb::run_item<DT, kUniformChunk, true, false>(gp, it, x, io.v_mb, y, tag, err, spin_limit, lds);
    return;
  }
  SgWork wp = w;
  wp.vpart = io.vpart;
  wp.flags = io.flags;
  if (part == 1) sg_shrink_item<DT, NBM, KBM>(gp, wp, x, tag, i, lds);
  else sg_expand_item<DT, NBM, KBM>(gp, wp, tag, spin_limit, err, y, i, lds);
}

template <int DT>
hipError_t shrink_dt(const Geom& g, const int32_t* tok, const SgTile* tiles, int32_t n_tiles,
                     int32_t ksplit, int32_t kc, int32_t nb, const void* x, float* vpart,
                     int32_t v_stride, int64_t split_stride, hipStream_t s, const LaunchEvents& ev) {
  const dim3 grid((unsigned)n_tiles, (unsigned)ksplit), block(64 * kWaves);
  const size_t lds = 0;
  const uint16_t* xp = (const uint16_t*)x;
  switch (nb) {
    case 1: hipExtLaunchKernelGGL((sgmv_shrink_kernel<DT, 1>), grid, block, lds, s, ev.start, ev.stop, 0, g, tiles, tok, kc, xp, vpart, v_stride, split_stride); break;
    case 2: hipExtLaunchKernelGGL((sgmv_shrink_kernel<DT, 2>), grid, block, lds, s, ev.start, ev.stop, 0, g, tiles, tok, kc, xp, vpart, v_stride, split_stride); break;
    case 4: hipExtLaunchKernelGGL((sgmv_shrink_kernel<DT, 4>), grid, block, lds, s, ev.start, ev.stop, 0, g, tiles, tok, kc, xp, vpart, v_stride, split_stride); break;
    default: hipExtLaunchKernelGGL((sgmv_shrink_kernel<DT, 8>), grid, block, lds, s, ev.start, ev.stop, 0, g, tiles, tok, kc, xp, vpart, v_stride, split_stride); break;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t expand_dt(const Geom& g, const int32_t* tok, const SgTile* tiles, int32_t n_tiles,
                     int32_t ksplit, int32_t kb, const float* vpart, int32_t v_stride,
                     int64_t split_stride, void* y, hipStream_t s, const LaunchEvents& ev) {
  const int per_wg = kSubPasses * kCols;
  const dim3 grid((unsigned)n_tiles, (unsigned)((g.d_out + per_wg - 1) / per_wg)), block(64 * kWaves);
  uint16_t* yp = (uint16_t*)y;
  switch (kb) {
    case 1: hipExtLaunchKernelGGL((sgmv_expand_kernel<DT, 1>), grid, block, 0, s, ev.start, ev.stop, 0, g, tiles, tok, ksplit, vpart, v_stride, split_stride, yp); break;
    case 2: hipExtLaunchKernelGGL((sgmv_expand_kernel<DT, 2>), grid, block, 0, s, ev.start, ev.stop, 0, g, tiles, tok, ksplit, vpart, v_stride, split_stride, yp); break;
    default: hipExtLaunchKernelGGL((sgmv_expand_kernel<DT, 4>), grid, block, 0, s, ev.start, ev.stop, 0, g, tiles, tok, ksplit, vpart, v_stride, split_stride, yp); break;
  }
  return hipGetLastError();
}

// Both launchers: the grid, the segment work and, for a launch of both families, the
// MBGMV items (n_mb = 0: segments only), for n_proj projections.
struct MbPart {
  const MbItem* items;
  int32_t n_mb, n_mb_shrink;
};

template <int DT, int NBM, int KBM>
hipError_t fused_launch(const Geom& g, const SgWork& w, const MbPart& mp, const Projs& pr,
                        int32_t n_proj, uint32_t tag, int32_t spin_limit, unsigned long long* err,
                        hipStream_t s, const LaunchEvents& ev) {
  const int per_wg = kSubPasses * kCols;
  const int64_t ncb = (g.d_out + per_wg - 1) / per_wg;
  const int64_t wide = NBM == 4 && KBM == 4 ? w.n_wide : 0;
  const int64_t n = ((int64_t)(w.n_tiles + wide) * w.ksplit + (int64_t)w.n_tiles * ncb + mp.n_mb) * n_proj;
  if (n > INT32_MAX) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  if (mp.n_mb == 0 && n_proj == 1) {
    const ProjIO& io = pr.p[0];
    hipExtLaunchKernelGGL((sgmv_fused_kernel<DT, NBM, KBM>), dim3((unsigned)n), dim3(64 * kWaves), 0, s,
                          ev.start, ev.stop, 0, g, w.tiles, w.tok, w.kc, w.ksplit, w.n_tiles, w.n_wide,
                          (const uint16_t*)io.x, io.vpart, w.v_stride, w.split_stride, io.flags, tag,
                          spin_limit, err, (uint16_t*)io.y);
    return hipGetLastError();
  }
  if constexpr (NBM == 8) {
    if (mp.n_mb > 0) return hipErrorInvalidValue;  // both families take the 3-per-CU wide template
    hipExtLaunchKernelGGL((mixed_fused_kernel<DT, true, NBM, KBM>), dim3((unsigned)n), dim3(64 * kWaves), 0, s,
                          ev.start, ev.stop, 0, g, w, mp.items, 0, 0, pr, n_proj, tag, spin_limit, err);
  } else if (g.P % 512 == 0) {
    hipExtLaunchKernelGGL((mixed_fused_kernel<DT, true, NBM, KBM>), dim3((unsigned)n), dim3(64 * kWaves), 0, s,
                          ev.start, ev.stop, 0, g, w, mp.items, mp.n_mb, mp.n_mb_shrink, pr, n_proj, tag,
                          spin_limit, err);
  } else {
    hipExtLaunchKernelGGL((mixed_fused_kernel<DT, false, NBM, KBM>), dim3((unsigned)n), dim3(64 * kWaves), 0, s,
                          ev.start, ev.stop, 0, g, w, mp.items, mp.n_mb, mp.n_mb_shrink, pr, n_proj, tag,
                          spin_limit, err);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t fused_dt(const Geom& g, SgWork w, int32_t max_rank, const MbPart& mp, const Projs& pr,
                    int32_t n_proj, uint32_t tag, int32_t spin_limit, unsigned long long* err,
                    hipStream_t s, const LaunchEvents& ev) {
  w.n_wide = 0;
  if (max_rank <= 16) return fused_launch<DT, 1, 1>(g, w, mp, pr, n_proj, tag, spin_limit, err, s, ev);
  if (max_rank <= 32) return fused_launch<DT, 2, 1>(g, w, mp, pr, n_proj, tag, spin_limit, err, s, ev);
  if (max_rank <= 64) return fused_launch<DT, 4, 2>(g, w, mp, pr, n_proj, tag, spin_limit, err, s, ev);
  // ranks above 64: the tiles that have them come first (descending rank; the tile
  // records are in host-visible pinned memory). Beside narrower tiles they are shrunk in
  // two 64-row blocks, so that the whole launch keeps 3 workgroups per CU; a launch of
  // such tiles alone keeps the 128-row body, which reads each x row once.
  while (w.n_wide < w.n_tiles && w.tiles[w.n_wide].rank > 64) ++w.n_wide;
  for (int32_t i = w.n_wide; i < w.n_tiles; ++i)
    if (w.tiles[i].rank > 64) return hipErrorInvalidValue;
  if (w.n_wide == w.n_tiles && mp.n_mb == 0)
    return fused_launch<DT, 8, 4>(g, w, mp, pr, n_proj, tag, spin_limit, err, s, ev);
  return fused_launch<DT, 4, 4>(g, w, mp, pr, n_proj, tag, spin_limit, err, s, ev);
}

}  // namespace

hipError_t launch_multi_fused(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit, int32_t kc,
                              int32_t v_stride, int64_t split_stride, const ProjIO* io,
                              int32_t n_proj, uint32_t tag, int32_t spin_limit,
                              unsigned long long* err, hipStream_t s, const LaunchEvents& ev,
                              const MbItem* mb_items, int32_t n_mb, int32_t n_mb_shrink,
                              int32_t mb_max_tok) {
  if (n_tiles < 0 || n_mb < 0 || n_mb_shrink < 0 || n_mb_shrink > n_mb || n_proj < 1 ||
      n_proj > kMaxProj || !io || !err || tag == 0)
    return hipErrorInvalidValue;
  if (n_tiles > 0 && (max_rank < 1 || max_rank > kMaxRank || ksplit < 1 || ksplit > kSgMaxSplit ||
                      kc % kRound || (v_stride & 3) || !tiles))
    return hipErrorInvalidValue;
  if (n_mb > 0 && (!mb_items || mb_max_tok < 1 || mb_max_tok > kMbGroup)) return hipErrorInvalidValue;
  Projs pr{};
  for (int32_t p = 0; p < n_proj; ++p) {
    pr.p[p] = io[p];
    if (!io[p].pt || !io[p].x || !io[p].y || (n_tiles > 0 && (!io[p].vpart || !io[p].flags)) ||
        (n_mb > 0 && !io[p].v_mb))
      return hipErrorInvalidValue;
  }
  const SgWork w{tiles, tok, kc, n_tiles > 0 ? ksplit : 1, n_tiles, 0, nullptr, v_stride, split_stride, nullptr};
  const MbPart mp{mb_items, n_mb, n_mb_shrink};
  const int32_t mr = n_tiles > 0 ? max_rank : 1;
  return g.dtype == SLORA_F16
             ? fused_dt<SLORA_F16>(g, w, mr, mp, pr, n_proj, tag, spin_limit, err, s, ev)
             : fused_dt<SLORA_BF16>(g, w, mr, mp, pr, n_proj, tag, spin_limit, err, s, ev);
}

hipError_t launch_sgmv_fused(const Geom& g, const int32_t* tok, const SgTile* tiles,
                             int32_t n_tiles, int32_t max_rank, int32_t ksplit, int32_t kc,
                             const void* x, float* vpart, int32_t v_stride, int64_t split_stride,
                             uint32_t* flags, uint32_t tag, int32_t spin_limit,
                             unsigned long long* err, void* y, hipStream_t s,
                             const LaunchEvents& ev, const MbItem* mb_items, int32_t n_mb,
                             int32_t n_mb_shrink, int32_t mb_max_tok, void* v_mb) {
  if (n_tiles <= 0) return hipSuccess;
  const ProjIO io{g.pt, x, y, v_mb, vpart, flags};
  return launch_multi_fused(g, tok, tiles, n_tiles, max_rank, ksplit, kc, v_stride, split_stride,
                            &io, 1, tag, spin_limit, err, s, ev, mb_items, n_mb, n_mb_shrink,
                            mb_max_tok);
}

int sgmv_shrink_resident(int32_t max_rank, int32_t dtype) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, int> cache;
  const int nb = shrink_nb(max_rank);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_tuple(dev, nb, (int)dtype);
  auto f = cache.find(key);
  if (f != cache.end()) return f->second;
  const void* k = nullptr;
  if (dtype == SLORA_F16)
    k = nb == 1 ? (const void*)sgmv_shrink_kernel<SLORA_F16, 1> : nb == 2 ? (const void*)sgmv_shrink_kernel<SLORA_F16, 2>
      : nb == 4 ? (const void*)sgmv_shrink_kernel<SLORA_F16, 4> : (const void*)sgmv_shrink_kernel<SLORA_F16, 8>;
  else
    k = nb == 1 ? (const void*)sgmv_shrink_kernel<SLORA_BF16, 1> : nb == 2 ? (const void*)sgmv_shrink_kernel<SLORA_BF16, 2>
      : nb == 4 ? (const void*)sgmv_shrink_kernel<SLORA_BF16, 4> : (const void*)sgmv_shrink_kernel<SLORA_BF16, 8>;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * kWaves, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cache[key] = per_cu * cus;
}

SgSplit sg_split(int32_t d_in, int32_t n_tiles, int32_t slots, int32_t n_proj) {
  SgSplit o;
  // k-ranges: a workgroup walks its range as a chain of dependent batches, and the
  // expand reads every range's partial sums. With one projection per launch, three
  // ranges measured best on the prefill batch (290 tiles), the MLP batch (~480 tiles)
  // and the mixed batch (~130 tiles, ranks to 128); with several projections in one
  // launch, whose other projections' items fill the tail of a short round, one (the
  // prefill and mixed batches' four-projection launches 2-4% faster than with three,
  // the MLP batch's two-projection launch within 1%). More are used only while every
  // (tile, k-range) workgroup of the launch still fits on the device at once, since a
  // launch that spills a little into a second round ends with a tail of lone chains.
  const int32_t items = n_tiles * std::max(n_proj, 1);
  const int32_t ks_min = n_proj > 1 ? kSgMinSplitMulti : kSgMinSplit;
  int32_t ks = n_tiles > 0 ? std::max(ks_min, slots / items) : 1;
  ks = std::max(1, std::min(ks, sg_max_split(d_in)));
  const int32_t per = (d_in + ks - 1) / ks;
  o.kc = (per + kRound - 1) / kRound * kRound;
  o.ksplit = (d_in + o.kc - 1) / o.kc;
  return o;
}

hipError_t launch_sgmv_shrink(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit, int32_t kc,
                              const void* x, float* vpart, int32_t v_stride, int64_t split_stride,
                              hipStream_t s, const LaunchEvents& ev) {
  if (n_tiles <= 0) return hipSuccess;
  if (max_rank < 1 || max_rank > kMaxRank || ksplit < 1 || ksplit > kSgMaxSplit || kc % kRound)
    return hipErrorInvalidValue;
  const int nb = shrink_nb(max_rank);
  return g.dtype == SLORA_F16
             ? shrink_dt<SLORA_F16>(g, tok, tiles, n_tiles, ksplit, kc, nb, x, vpart, v_stride, split_stride, s, ev)
             : shrink_dt<SLORA_BF16>(g, tok, tiles, n_tiles, ksplit, kc, nb, x, vpart, v_stride, split_stride, s, ev);
}

hipError_t launch_sgmv_expand(const Geom& g, const int32_t* tok, const SgTile* tiles,
                              int32_t n_tiles, int32_t max_rank, int32_t ksplit,
                              const float* vpart, int32_t v_stride, int64_t split_stride, void* y,
                              hipStream_t s, const LaunchEvents& ev) {
  if (n_tiles <= 0) return hipSuccess;
  if (max_rank < 1 || max_rank > kMaxRank || ksplit < 1 || ksplit > kSgMaxSplit)
    return hipErrorInvalidValue;
  const int kb = max_rank <= 32 ? 1 : max_rank <= 64 ? 2 : 4;
  return g.dtype == SLORA_F16
             ? expand_dt<SLORA_F16>(g, tok, tiles, n_tiles, ksplit, kb, vpart, v_stride, split_stride, y, s, ev)
             : expand_dt<SLORA_BF16>(g, tok, tiles, n_tiles, ksplit, kb, vpart, v_stride, split_stride, y, s, ev);
}

}  // namespace slora

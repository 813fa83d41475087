// Device helpers shared by the gfx950 kernels: fp16 / bf16 conversions, packed
// dot products, 16-byte loads and the wave-wide transposing reduction.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace slora {
namespace dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// quiet NaN in both halves of a dword: what a gather through an invalid page id reads
template <int DT>
__device__ __forceinline__ uint32_t nan2() {
  return DT == SLORA_F16 ? 0x7E007E00u : 0x7FC07FC0u;
}

// 16-byte fill vectors in device memory. Loads that must not touch the pool (rows
// past the rank, an invalid page id, lanes past the end of a row) are pointed at
// these instead of being predicated, so every load issues unconditionally and no
// loaded value is selected on before it is used. (Not const, so the compiler
// cannot fold these loads back into selects on loaded data.)
struct alignas(16) FillVectors {
  uint32_t zero[4];
  uint32_t nan_f16[4];
  uint32_t nan_bf16[4];
};
__device__ FillVectors kFill = {{0u, 0u, 0u, 0u},
                                      {0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u},
                                      {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u}};

__device__ __forceinline__ const uint16_t* fill_zero() {
  return reinterpret_cast<const uint16_t*>(kFill.zero);
}
template <int DT>
__device__ __forceinline__ const uint16_t* fill_nan() {
  return reinterpret_cast<const uint16_t*>(DT == SLORA_F16 ? kFill.nan_f16 : kFill.nan_bf16);
}

template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t w) {
  if constexpr (DT == SLORA_F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  else
    return __builtin_bit_cast(float, w << 16);
}

template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t w) {
  if constexpr (DT == SLORA_F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// fp32 -> storage type, round to nearest even (v_cvt_f16_f32 / v_cvt_pk_bf16_f32)
template <int DT>
__device__ __forceinline__ uint32_t to_bits(float f) {
  if constexpr (DT == SLORA_F16)
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
  else
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return to_bits<DT>(lo) | (to_bits<DT>(hi) << 16);
}

// c + a.lo * b.lo + a.hi * b.hi with fp32 accumulation (v_dot2_f32_f16 / _bf16)
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (DT == SLORA_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), c, false);
}

template <int DT>
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float c) {
  c = dot2<DT>(a.x, b.x, c);
  c = dot2<DT>(a.y, b.y, c);
  c = dot2<DT>(a.z, b.z, c);
  c = dot2<DT>(a.w, b.w, c);
  return c;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(uint16_t* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Read of a wave-uniform address through the scalar data cache (s_load). On a CU whose
// waves keep many vector loads in flight, a new vector load queues behind them; a scalar
// load reaches L2 on its own path. Only for memory that nothing writes while the kernel
// runs (work lists, page tables): the scalar cache is not kept coherent within a launch.
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}
// The same at a 32-bit byte offset from a base (the offset travels in one register).
template <typename T>
__device__ __forceinline__ T sload(const T* base, uint32_t byte_off) {
  return *(const __attribute__((address_space(4))) T*)((const char*)base + byte_off);
}

// Makes the compiler issue all 16 scalar loads of `a` before this point and wait for them
// once (it would otherwise wait for each load next to its use).
__device__ __forceinline__ void settle16(int (&a)[16]) {
  asm volatile(""
               : "+s"(a[0]), "+s"(a[1]), "+s"(a[2]), "+s"(a[3]), "+s"(a[4]), "+s"(a[5]),
                 "+s"(a[6]), "+s"(a[7]), "+s"(a[8]), "+s"(a[9]), "+s"(a[10]), "+s"(a[11]),
                 "+s"(a[12]), "+s"(a[13]), "+s"(a[14]), "+s"(a[15]));
}

// 16 int32 entries base[min(first + i, last) * stride] (i < 16), read through the scalar
// cache (every index wave-uniform, base[last * stride] in bounds), into lanes lane0 ..
// lane0 + 15 of `into`: all loads are issued before one wait, and the values leave the
// scalar registers right after.
__device__ __forceinline__ int sload16_to_lanes(const int32_t* base, int first, int last,
                                                int stride, int into, int lane0) {
  int a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = sload(base, (uint32_t)(min(first + i, last) * stride) * 4u);
  settle16(a);
#pragma unroll
  for (int i = 0; i < 16; ++i) into = (int)(threadIdx.x & 63) == lane0 + i ? a[i] : into;
  return into;
}

// Sum V values per lane (V a power of two, 1..64) over the 64 lanes of a wave,
// with no per-lane selects (which the compiler would turn into indexed scratch):
//   * v_permlane32_swap pairs value i with value i + V/2 across the lane halves:
//     after "swap(a[i], a[i + V/2]); a[i] = a[i] + a[i + V/2]", lanes 0-31 hold
//     the sum over (l, l ^ 32) of value i and lanes 32-63 that of value i + V/2;
//   * v_permlane16_swap does the same between rows 2j and 2j + 1 (16 lanes each);
//   * a DPP reduction inside each row of 16 lanes (rotate by 8 and 4, then quad
//     permutations) completes the sum.
// With one value left, a register is swapped with itself, which adds the two
// halves. Afterwards lane l holds in out[i] the total of value wave_sum_index<V>(l, i),
// replicated across every lane that wave_sum_writer<V> does not select. The order of
// the additions depends on lane numbers only, so results are reproducible.
template <int V>
struct WaveSum {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  static constexpr int kOut = V >= 4 ? V / 4 : 1;
};

__device__ __forceinline__ void swap_add32(float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  lo = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap_add16(float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  lo = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

template <int V>
__device__ __forceinline__ void wave_sum(float (&a)[V], float (&out)[WaveSum<V>::kOut]) {
  constexpr int K = WaveSum<V>::kOut;
  if constexpr (V >= 2) {
#pragma unroll
    for (int i = 0; i < V / 2; ++i) swap_add32(a[i], a[i + V / 2]);
  } else {
    float t = a[0];
    swap_add32(a[0], t);
  }
  if constexpr (V >= 4) {
#pragma unroll
    for (int i = 0; i < V / 4; ++i) swap_add16(a[i], a[i + V / 4]);
  } else {
    float t = a[0];
    swap_add16(a[0], t);
  }
#pragma unroll
  for (int i = 0; i < K; ++i) {
    float x = a[i];
    x = dpp_add<0x128>(x);  // row_ror:8
    x = dpp_add<0x124>(x);  // row_ror:4
    x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
    x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
    out[i] = x;
  }
}

template <int V>
__device__ __forceinline__ int wave_sum_index(int lane, int i) {
  int base = 0;
  if constexpr (V >= 2) base += ((lane >> 5) & 1) * (V / 2);
  if constexpr (V >= 4) base += ((lane >> 4) & 1) * (V / 4);
  return base + i;
}

template <int V>
__device__ __forceinline__ bool wave_sum_writer(int lane, int i) {
  if constexpr (V >= 4) return (lane & 15) == i;
  else if constexpr (V == 2) return (lane & 31) == 0;
  else return lane == 0;
}

}  // namespace dev
}  // namespace slora

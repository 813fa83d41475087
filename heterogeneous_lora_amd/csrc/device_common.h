// Device helpers shared by the gfx950 kernels: fp16 / bf16 conversions, packed
// dot products, 16-byte loads and the wave-wide transposing reduction.
#pragma once

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

// Sum V values per lane across the 64 lanes of a wave. Halving butterfly: at each
// step a lane trades the half of its values its partner keeps, so V values need
// V - 1 exchanges plus log2(64 / V) for the tail, instead of 6 V. Lane l returns
// the total of value index reduce_index<V>(l); lanes l and l ^ m for the tail masks
// m < 64 / V return the same total. The summation order is fixed by lane numbers.
template <int V>
__device__ __forceinline__ float xreduce(float (&a)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  int m = 32;
#pragma unroll
  for (int h = V / 2; h >= 1; h /= 2) {
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? a[i] : a[i + h];
      const float keep = up ? a[i + h] : a[i];
      a[i] = keep + __shfl_xor(send, m);
    }
    m >>= 1;
  }
  float r = a[0];
#pragma unroll
  for (; m >= 1; m >>= 1) r += __shfl_xor(r, m);
  return r;
}

template <int V>
__device__ __forceinline__ int reduce_index(int lane) {
  int idx = 0, m = 32;
#pragma unroll
  for (int h = V / 2; h >= 1; h /= 2) {
    if (lane & m) idx += h;
    m >>= 1;
  }
  return idx;
}

// lanes that write the reduced values (one per index)
template <int V>
__device__ __forceinline__ bool reduce_writer(int lane) {
  return (lane & (64 / V - 1)) == 0;
}

}  // namespace dev
}  // namespace slora

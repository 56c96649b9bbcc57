// 16-byte slices of a key row and their dot products with the matching
// slice of a query row: the arithmetic of every exact score in the library
// (the score scan and the 4-bit path's rescoring use this one definition, so
// their scores agree bit for bit).
#pragma once

#include "device_common.h"

namespace ctopk {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T>
struct Slice;

// bf16: 8 elements per 16-byte slice, dot2 on packed pairs.
template <>
struct Slice<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static __forceinline__ float dot(const uint4& k, const uint4& q) {
    float a = 0.0f;
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                        __builtin_bit_cast(bf16x2_t, q.x), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                        __builtin_bit_cast(bf16x2_t, q.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                        __builtin_bit_cast(bf16x2_t, q.z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                        __builtin_bit_cast(bf16x2_t, q.w), a, false);
    return a;
  }
  // The slice's elements as fp32 (exact), in order.
  __device__ static __forceinline__ void unpack(const uint4& k, float (&x)[kElems]) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// fp32: 4 elements per 16-byte slice.
template <>
struct Slice<float> {
  static constexpr int kElems = 4;
  __device__ static __forceinline__ float dot(const uint4& k, const uint4& q) {
    float a = __uint_as_float(k.x) * __uint_as_float(q.x);
    a = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), a);
    a = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), a);
    a = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), a);
    return a;
  }
  __device__ static __forceinline__ void unpack(const uint4& k, float (&x)[kElems]) {
    x[0] = __uint_as_float(k.x);
    x[1] = __uint_as_float(k.y);
    x[2] = __uint_as_float(k.z);
    x[3] = __uint_as_float(k.w);
  }
};

}  // namespace ctopk

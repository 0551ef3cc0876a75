// Device-side helpers shared by the KDA kernels: bf16 <-> fp32, small vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr uint32_t DEVERR_SLOT_RANGE = KDA_DEVERR_SLOT_RANGE;

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two fp32 values -> packed bf16 (lo in bits 0-15), round to nearest even (NaN stays NaN): one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 kda_bf16x2 __attribute__((ext_vector_type(2)));
typedef float kda_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const kda_f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, kda_bf16x2));
}

// Load N consecutive bf16 values as raw 16-bit words (N in {1, 2, 4, 8, 16}); the pointer
// must be aligned to 2*N bytes (N <= 8) or 16 bytes.
template <int N>
__device__ __forceinline__ void load_bf16_raw(const uint16_t* p, uint32_t (&w)[(N + 1) / 2]) {
  if constexpr (N == 1) {
    w[0] = *p;
  } else if constexpr (N == 2) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (N == 4) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else {
    static_assert(N % 8 == 0, "bf16 vector width");
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      uint4 x = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i + 0] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  }
}

template <int N>
__device__ __forceinline__ void store_bf16_raw(uint16_t* p, const uint32_t (&w)[(N + 1) / 2]) {
  if constexpr (N == 1) {
    *p = (uint16_t)w[0];
  } else if constexpr (N == 2) {
    *reinterpret_cast<uint32_t*>(p) = w[0];
  } else if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
    static_assert(N % 8 == 0, "bf16 vector width");
#pragma unroll
    for (int i = 0; i < N / 8; ++i)
      reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  }
}

template <int N>
__device__ __forceinline__ void unpack_bf16(const uint32_t (&w)[(N + 1) / 2], float (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] = bf2f((w[i / 2] >> (16 * (i & 1))) & 0xffffu);
}

template <int N>
__device__ __forceinline__ void load_f32(const float* p, float (&f)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      float4 x = reinterpret_cast<const float4*>(p)[i];
      f[4 * i] = x.x; f[4 * i + 1] = x.y; f[4 * i + 2] = x.z; f[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = p[i];
  }
}

template <int N>
__device__ __forceinline__ void store_f32(float* p, const float (&f)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = f[i];
  }
}

}  // namespace kda

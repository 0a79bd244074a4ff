// Device-side helpers shared by the wanattn kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 is the upper half of an fp32 word: widening is a shift.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 (one 16-byte vector) -> 8 fp32.
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16lo(v[i]);
    f[2 * i + 1] = bf16hi(v[i]);
  }
}

// 8 fp32 -> 8 bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u32x4 pack8(const float* f) {
  f32x8 x = {f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
  bf16x8 b = __builtin_convertvector(x, bf16x8);
  return __builtin_bit_cast(u32x4, b);
}

// Streaming 16-byte accesses for data touched once (nontemporal hint: the
// activations are read and written exactly once per call).
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store_stream(uint16_t* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Sum over aligned groups of 16 lanes.
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Workgroup id -> logical tile id such that each XCD (hardware places
// workgroup i on XCD i % 8) receives one contiguous range of logical ids.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n) {
  const uint32_t q = n >> 3, r = n & 7u, x = i & 7u;
  return x * q + (x < r ? x : r) + (i >> 3);
}

}  // namespace wan

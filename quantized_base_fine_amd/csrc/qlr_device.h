// Device-side helpers shared by the gfx950 kernels of the qlr library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlr {

// Codebook levels passed by value as a kernel argument (at most 2^8 levels).
struct Levels {
  float v[256];
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// float32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element i of a storage-dtype array, widened exactly to float32.
template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (DT == DT_F32) {
    return reinterpret_cast<const float*>(p)[i];
  } else if constexpr (DT == DT_F16) {
    return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Copy the NL codebook levels of the by-value kernel argument into LDS.  The
// loop index is the same for every lane, so the argument is read with scalar
// loads; indexing the argument per lane would turn into slow vector loads from
// the kernel-argument segment.  Callers synchronise the workgroup afterwards.
template <int NL>
__device__ __forceinline__ void stage_levels(const Levels& lv, float* sL) {
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) sL[i] = lv.v[i];
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

}  // namespace qlr

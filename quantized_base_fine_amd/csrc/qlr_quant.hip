// Blockwise quantile quantization with double quantization, and its inverse.
//
// QLoRA page ("QLoRA", aizip.shop methodologies), section "1. 4-bit NormalFloat
// (NF4) quantization" (codebook of normal quantiles) and section "2. Double
// Quantization" (absmax constants of 64-weight blocks, re-quantized to 8 bits).
//
// Every decision is exact: a code is the count of level midpoints strictly
// below w, compared as 2w > (L[i] + L[i+1]) * a in float64, where the sum needs
// at most 27 significant bits and the product at most 51, so nothing rounds.
// The 8-bit absmax code is the count of (m + 1/2) * s below a, also exact in
// float64.  Ties therefore go to the lower index on both levels.
#include "qlr_internal.h"

namespace qlr {

namespace {

constexpr int kThreads = 256;       // one workgroup per group of 256 blocks
constexpr int kBlocksPerPass = 32;  // 8 lanes per 64-element block, 8 elements per lane

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// 8 consecutive elements from e0 (all in range): the raw 16 or 32 bytes, then
// their widening to float32 (apart, so that every load can be issued first)
template <int DT>
struct Raw8 {
  uint4 u[DT == DT_F32 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ Raw8<DT> load8_raw(const void* W, int64_t e0) {
  Raw8<DT> r;
  if constexpr (DT == DT_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(W) + e0);
    r.u[0] = p[0];
    r.u[1] = p[1];
  } else {
    r.u[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(W) + e0);
  }
  return r;
}

template <int DT>
__device__ __forceinline__ void widen8(const Raw8<DT>& r, float (&w)[8]) {
  if constexpr (DT == DT_F32) {
    const uint32_t d[8] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w, r.u[1].x, r.u[1].y, r.u[1].z, r.u[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __uint_as_float(d[i]);
  } else {
    const uint32_t d[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_F16) {
        w[2 * i] = f16_bits_to_f32((uint16_t)(d[i] & 0xFFFFu));
        w[2 * i + 1] = f16_bits_to_f32((uint16_t)(d[i] >> 16));
      } else {
        w[2 * i] = bf16_bits_to_f32(d[i] & 0xFFFFu);
        w[2 * i + 1] = bf16_bits_to_f32(d[i] >> 16);
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void load8(const void* W, int64_t e0, int64_t numel, float (&w)[8],
                                      int& present) {
  if (e0 + 8 <= numel) {
    present = 8;
    if constexpr (DT == DT_F32) {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + e0);
      float4 a = p[0], b = p[1];
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
      uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(W) + e0);
      uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DT == DT_F16) {
          w[2 * i] = f16_bits_to_f32((uint16_t)(d[i] & 0xFFFFu));
          w[2 * i + 1] = f16_bits_to_f32((uint16_t)(d[i] >> 16));
        } else {
          w[2 * i] = bf16_bits_to_f32(d[i] & 0xFFFFu);
          w[2 * i + 1] = bf16_bits_to_f32(d[i] >> 16);
        }
      }
    }
  } else {
    present = (int)(e0 < numel ? numel - e0 : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (i < present) ? load_elem<DT>(W, e0 + i) : 0.0f;
  }
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* dst, uint64_t packed) {
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
  } else if constexpr (BITS == 4) {
    *reinterpret_cast<uint32_t*>(dst) = (uint32_t)packed;
  } else if constexpr (BITS == 8) {
    *reinterpret_cast<uint64_t*>(dst) = packed;
  } else {  // 3 bits: 24 bits per 8 codes, byte aligned only
    dst[0] = (uint8_t)packed;
    dst[1] = (uint8_t)(packed >> 8);
    dst[2] = (uint8_t)(packed >> 16);
  }
}

// One workgroup quantizes one group: 256 blocks of 64 elements (16384 elements).
template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void k_quantize(const void* __restrict__ W, int64_t numel,
                                                        Levels lv, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ q8,
                                                        float* __restrict__ cst,
                                                        uint32_t* __restrict__ flag) {
  constexpr int NL = 1 << BITS;
  __shared__ double sT[NL];  // level midpoints times two: L[i] + L[i+1] (exact)
  __shared__ float sA[256];  // first-level absmax of the group's blocks
  __shared__ float sMax[kThreads / 64];

  __shared__ float sL[NL];
  const int tid = threadIdx.x;
  stage_levels<NL>(lv, sL);
  __syncthreads();
  for (int i = tid; i < NL - 1; i += kThreads) sT[i] = (double)sL[i] + (double)sL[i + 1];
  const int64_t nblk_total = (numel + 63) / 64;
  const int64_t blk0 = (int64_t)blockIdx.x * 256;
  const int nblk_here = (int)min<int64_t>(256, nblk_total - blk0);
  __syncthreads();

  bool bad = false;
  const int q = tid & 7;  // lane within the block
  // block jj's absmax and codes from the lane's 8 elements w (present of them real)
  auto encode = [&](int jj, const float (&w)[8], int present) {
    const int64_t j = blk0 + jj;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bad |= !__builtin_isfinite(w[i]);
      m = fmaxf(m, fabsf(w[i]));
    }
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    if (q == 0 && jj < nblk_here) sA[jj] = m;

    const double a = (double)m;
    uint64_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double w2 = 2.0 * (double)w[i];
      int c = 0;
#pragma unroll
      for (int step = NL / 2; step >= 1; step >>= 1)
        if (w2 > sT[c + step - 1] * a) c += step;
      if (i >= present) c = 0;
      packed |= (uint64_t)c << (BITS * i);
    }
    if (jj < nblk_here) store_codes<BITS>(codes + j * (8 * BITS) + q * BITS, packed);
  };
  if (blk0 * 64 + 256 * 64 <= numel) {
    // a whole group (uniform): the loads of all passes in flight together
    Raw8<DT> raw[256 / kBlocksPerPass];
#pragma unroll
    for (int pass = 0; pass < 256 / kBlocksPerPass; ++pass)
      raw[pass] = load8_raw<DT>(W, (blk0 + pass * kBlocksPerPass + (tid >> 3)) * 64 + q * 8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pass = 0; pass < 256 / kBlocksPerPass; ++pass) {
      float w[8];
      widen8<DT>(raw[pass], w);
      encode(pass * kBlocksPerPass + (tid >> 3), w, 8);
    }
  } else {
#pragma unroll 1
    for (int pass = 0; pass < 256 / kBlocksPerPass; ++pass) {
      const int jj = pass * kBlocksPerPass + (tid >> 3);
      float w[8];
      int present = 0;
      if (jj < nblk_here) {
        load8<DT>(W, (blk0 + jj) * 64 + q * 8, numel, w, present);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.0f;
      }
      encode(jj, w, present);
    }
  }
  __syncthreads();

  // Double quantization of the group's absmax values.
  const float a = (tid < nblk_here) ? sA[tid] : 0.0f;
  float g = a;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) g = fmaxf(g, __shfl_xor(g, off, 64));
  if ((tid & 63) == 0) sMax[tid >> 6] = g;
  __syncthreads();
  g = fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3]));
  const float s = (float)((double)g / 255.0);  // one rounding: 53 >= 2*24 + 2
  if (tid < nblk_here) {
    const double ad = (double)a, sd = (double)s;
    int c = 0;
#pragma unroll
    for (int step = 128; step >= 1; step >>= 1)
      if (ad > (double)(2 * (c + step - 1) + 1) * sd * 0.5) c += step;
    q8[blk0 + tid] = (uint8_t)c;
  }
  if (tid == 0) cst[blockIdx.x] = s;
  if (__any(bad) && (tid & 63) == 0) atomicOr(flag, 1u);
}

template <int BITS>
__device__ __forceinline__ uint64_t load_codes8(const uint8_t* p) {
  if constexpr (BITS == 2) return *reinterpret_cast<const uint16_t*>(p);
  else if constexpr (BITS == 4) return *reinterpret_cast<const uint32_t*>(p);
  else if constexpr (BITS == 8) return *reinterpret_cast<const uint64_t*>(p);
  else return (uint64_t)p[0] | ((uint64_t)p[1] << 8) | ((uint64_t)p[2] << 16);
}

// Each thread dequantizes 8 consecutive elements: two float32 multiplies each.
template <int BITS, int ODT>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ q8,
                                                    const float* __restrict__ cst, int64_t numel,
                                                    Levels lv, void* __restrict__ out) {
  constexpr int NL = 1 << BITS;
  __shared__ float sL[NL];
  stage_levels<NL>(lv, sL);
  __syncthreads();
  const int64_t nchunk = (numel + 7) / 8;
  for (int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ch < nchunk;
       ch += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = ch >> 3;
    const int q = (int)(ch & 7);
    const float ap = (float)q8[j] * cst[j >> 8];
    const uint64_t bitsv = load_codes8<BITS>(codes + j * (8 * BITS) + q * BITS);
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = sL[(bitsv >> (BITS * i)) & (NL - 1)] * ap;
    const int64_t e0 = ch * 8;
    if (e0 + 8 <= numel) {
      if constexpr (ODT == DT_F32) {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e0);
        o[0] = make_float4(w[0], w[1], w[2], w[3]);
        o[1] = make_float4(w[4], w[5], w[6], w[7]);
      } else {
        uint4 u;
        u.x = pack_bf16x2(w[0], w[1]);
        u.y = pack_bf16x2(w[2], w[3]);
        u.z = pack_bf16x2(w[4], w[5]);
        u.w = pack_bf16x2(w[6], w[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + e0) = u;
      }
    } else {
      for (int i = 0; i < 8 && e0 + i < numel; ++i) {
        if constexpr (ODT == DT_F32) reinterpret_cast<float*>(out)[e0 + i] = w[i];
        else reinterpret_cast<uint16_t*>(out)[e0 + i] = (uint16_t)f32_to_bf16_bits(w[i]);
      }
    }
  }
}

template <int BITS>
hipError_t launch_quantize_b(const void* W, int wdt, int64_t numel, const Levels& lv,
                             uint8_t* codes, uint8_t* q8, float* cst, uint32_t* flag,
                             hipStream_t s) {
  const int64_t ngroups = ((numel + 63) / 64 + 255) / 256;
  dim3 grid((unsigned)ngroups), block(kThreads);
  if (wdt == DT_F32)
    hipLaunchKernelGGL((k_quantize<BITS, DT_F32>), grid, block, 0, s, W, numel, lv, codes, q8, cst, flag);
  else if (wdt == DT_F16)
    hipLaunchKernelGGL((k_quantize<BITS, DT_F16>), grid, block, 0, s, W, numel, lv, codes, q8, cst, flag);
  else
    hipLaunchKernelGGL((k_quantize<BITS, DT_BF16>), grid, block, 0, s, W, numel, lv, codes, q8, cst, flag);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_dequantize_b(const uint8_t* codes, const uint8_t* q8, const float* cst,
                               int64_t numel, const Levels& lv, void* out, int odt,
                               hipStream_t s) {
  const int64_t nchunk = (numel + 7) / 8;
  const int64_t want = (nchunk + 255) / 256;
  dim3 grid((unsigned)std::min<int64_t>(want, 256 * 64)), block(256);
  if (odt == DT_F32)
    hipLaunchKernelGGL((k_dequantize<BITS, DT_F32>), grid, block, 0, s, codes, q8, cst, numel, lv, out);
  else
    hipLaunchKernelGGL((k_dequantize<BITS, DT_BF16>), grid, block, 0, s, codes, q8, cst, numel, lv, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* W, int wdt, int64_t numel, int bits, const Levels& lv,
                           uint8_t* codes, uint8_t* q8, float* cst, uint32_t* flag,
                           hipStream_t s) {
  switch (bits) {
    case 2: return launch_quantize_b<2>(W, wdt, numel, lv, codes, q8, cst, flag, s);
    case 3: return launch_quantize_b<3>(W, wdt, numel, lv, codes, q8, cst, flag, s);
    case 4: return launch_quantize_b<4>(W, wdt, numel, lv, codes, q8, cst, flag, s);
    default: return launch_quantize_b<8>(W, wdt, numel, lv, codes, q8, cst, flag, s);
  }
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* q8, const float* cst,
                             int64_t numel, int bits, const Levels& lv, void* out, int odt,
                             hipStream_t s) {
  switch (bits) {
    case 2: return launch_dequantize_b<2>(codes, q8, cst, numel, lv, out, odt, s);
    case 3: return launch_dequantize_b<3>(codes, q8, cst, numel, lv, out, odt, s);
    case 4: return launch_dequantize_b<4>(codes, q8, cst, numel, lv, out, odt, s);
    default: return launch_dequantize_b<8>(codes, q8, cst, numel, lv, out, odt, s);
  }
}

}  // namespace qlr

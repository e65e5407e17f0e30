// Level lookup shared by the MFMA kernels: a lane-private LDS table of bf16
// level pairs.  Entry e of lane L sits at byte e*256 + 4L, so the 64 lanes of a
// wave read 64 different banks.  For 2/3/4-bit codes an entry holds the levels
// of two neighbouring codes (index = their packed bits, the lower code in the
// low half); for 8-bit codes an entry holds one level in its low half.
#pragma once

#include "qlr_device.h"

namespace qlr {

template <int BITS>
struct PairTable {
  // entries per lane copy: 2 codes per entry, except 8-bit (one code, bf16 in the low half)
  static constexpr int kEntries = (BITS == 8) ? 256 : (1 << (2 * BITS));
  static constexpr int kBytes = kEntries * 256;
};

// Fill the lane-private table from the levels staged in LDS (sL).
template <int BITS>
__device__ __forceinline__ void build_table(uint32_t* tbl, const float* sL, int tid, int nthreads) {
  constexpr int NL = 1 << BITS;
  constexpr int E = PairTable<BITS>::kEntries;
  for (int idx = tid; idx < E * 64; idx += nthreads) {
    const int e = idx >> 6;
    uint32_t v;
    if constexpr (BITS == 8) v = f32_to_bf16_bits(sL[e]);
    else v = pack_bf16x2(sL[e & (NL - 1)], sL[e >> BITS]);
    tbl[idx] = v;
  }
}

__device__ __forceinline__ uint32_t lds_u32(const uint32_t* base, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + byte_addr);
}

// Raw code bits of a lane's 16 weights of one block.
template <int BITS>
struct Raw;
template <> struct Raw<2> { uint32_t v; };
template <> struct Raw<3> { uint32_t lo, hi; };
template <> struct Raw<4> { uint32_t a, b; };
template <> struct Raw<8> { uint32_t a, b, c, d; };

template <int BITS>
__device__ __forceinline__ Raw<BITS> load_raw(const uint8_t* blk, int g) {
  Raw<BITS> r;
  if constexpr (BITS == 2) {
    r.v = *reinterpret_cast<const uint32_t*>(blk + 4 * g);
  } else if constexpr (BITS == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(blk + 8 * g);
    r.a = u.x; r.b = u.y;
  } else if constexpr (BITS == 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(blk + 16 * g);
    r.a = u.x; r.b = u.y; r.c = u.z; r.d = u.w;
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(blk + 6 * g);
    r.lo = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
    r.hi = p[2];
  }
  return r;
}

// Unscaled bf16 levels of the lane's 16 weights: b0 = elements 0..7, b1 = 8..15.
template <int BITS>
__device__ __forceinline__ void decode16(const Raw<BITS>& r, const uint32_t* tbl, uint32_t lane4,
                                         u32x4_t& b0, u32x4_t& b1) {
  if constexpr (BITS == 4) {
    // address = (code byte << 8) | lane*4, built with one byte permute
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + i) << 8);
      b0[i] = lds_u32(tbl, __builtin_amdgcn_perm(r.a, lane4, sel));
      b1[i] = lds_u32(tbl, __builtin_amdgcn_perm(r.b, lane4, sel));
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b0[i] = lds_u32(tbl, (((r.v >> (4 * i)) & 15u) << 8) | lane4);
      b1[i] = lds_u32(tbl, (((r.v >> (16 + 4 * i)) & 15u) << 8) | lane4);
    }
  } else if constexpr (BITS == 3) {
    const uint64_t v = (uint64_t)r.lo | ((uint64_t)r.hi << 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b0[i] = lds_u32(tbl, ((uint32_t)((v >> (6 * i)) & 63u) << 8) | lane4);
      b1[i] = lds_u32(tbl, ((uint32_t)((v >> (24 + 6 * i)) & 63u) << 8) | lane4);
    }
  } else {
    const uint32_t w[4] = {r.a, r.b, r.c, r.d};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d0 = w[i >> 1], d1 = w[2 + (i >> 1)];
      const int sh = 16 * (i & 1);
      const uint32_t lo0 = lds_u32(tbl, (((d0 >> sh) & 255u) << 8) | lane4);
      const uint32_t hi0 = lds_u32(tbl, (((d0 >> (sh + 8)) & 255u) << 8) | lane4);
      const uint32_t lo1 = lds_u32(tbl, (((d1 >> sh) & 255u) << 8) | lane4);
      const uint32_t hi1 = lds_u32(tbl, (((d1 >> (sh + 8)) & 255u) << 8) | lane4);
      b0[i] = lo0 | (hi0 << 16);
      b1[i] = lo1 | (hi1 << 16);
    }
  }
}


// Unscaled bf16 levels of 8 consecutive codes, given as 8*BITS bits starting at
// bit 0 of `v` (v holds at most 64 bits): 4 dwords of bf16 pairs.
template <int BITS>
__device__ __forceinline__ u32x4_t decode8(uint64_t v, const uint32_t* tbl, uint32_t lane4) {
  u32x4_t b;
  if constexpr (BITS == 4) {
    const uint32_t d = (uint32_t)v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b[i] = lds_u32(tbl, __builtin_amdgcn_perm(d, lane4, 0x0C0C0000u | ((uint32_t)(4 + i) << 8)));
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = lds_u32(tbl, ((uint32_t)((v >> (4 * i)) & 15u) << 8) | lane4);
  } else if constexpr (BITS == 3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = lds_u32(tbl, ((uint32_t)((v >> (6 * i)) & 63u) << 8) | lane4);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = lds_u32(tbl, ((uint32_t)((v >> (16 * i)) & 255u) << 8) | lane4);
      const uint32_t hi = lds_u32(tbl, ((uint32_t)((v >> (16 * i + 8)) & 255u) << 8) | lane4);
      b[i] = lo | (hi << 16);
    }
  }
  return b;
}

// float32 level pairs for the prefill dequantizer: entry e (e = two packed
// codes, or one 8-bit code) of copy c at byte e*256 + 8c, c = lane % 32, so a
// wave's lanes 0..15 / 16..31 / 32..47 / 48..63 each read 16 different 8-byte
// bank pairs.  For 8-bit codes the entry holds one level (second float unused).
template <int BITS>
struct PairTableF32 {
  static constexpr int kEntries = (BITS == 8) ? 256 : (1 << (2 * BITS));
  static constexpr int kBytes = kEntries * 256;
};

template <int BITS>
__device__ __forceinline__ void build_table_f32(uint32_t* tbl, const float* sL, int tid, int nthreads) {
  constexpr int NL = 1 << BITS;
  constexpr int E = PairTableF32<BITS>::kEntries;
  float2* t2 = reinterpret_cast<float2*>(tbl);
  for (int idx = tid; idx < E * 32; idx += nthreads) {
    const int e = idx >> 5;
    float2 v;
    if constexpr (BITS == 8) v = make_float2(sL[e], 0.0f);
    else v = make_float2(sL[e & (NL - 1)], sL[e >> BITS]);
    t2[idx] = v;
  }
}

__device__ __forceinline__ float2 lds_f2(const uint32_t* base, uint32_t byte_addr) {
  return *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(base) + byte_addr);
}

}  // namespace qlr

// Level lookup of the decode kernels' MFMA path (several x rows, or 3-bit codes
// on their own at M = 1): a table in LDS of bf16 levels, each level carried as
// two bf16 halves, hi = bf16(L) and lo = bf16(L - hi).  Together they hold L
// to about 16 significant bits, so a product with a bf16 x (exact in
// float32 either way) is within 2^-16 of the exact one relative to |x L|; hi
// alone can be off by up to 2^-8, which is more than the layer's 1e-3 budget
// when every term of a sum has the same sign.
//   * 2-, 3- and 4-bit codes: entry e = the packed bits of two neighbouring codes
//     (the lower code in the low bits), 8 bytes: the hi pair (lower code in the
//     low half), then the lo pair.  Copy c = lane % 32 of entry e sits at byte
//     e*256 + 8c, so the 16 or 32 lanes an LDS cycle serves hit distinct banks.
//   * 8-bit codes: entry e = one code, 4 bytes: hi in the low half, lo in the
//     high half.  Copy L = lane of entry e sits at byte e*256 + 4L.
// The table sits at LDS address 0: a lookup address is (entry << 8) | table_lane.
#pragma once

#include "qlr_device.h"

namespace qlr {

template <int BITS>
struct PairTable {
  static constexpr int kEntries = (BITS == 8) ? 256 : (1 << (2 * BITS));
  static constexpr int kBytes = kEntries * 256;
};

// Byte offset of a lane's copy inside an entry.
template <int BITS>
__device__ __forceinline__ uint32_t table_lane(int lane) {
  return BITS == 8 ? 4u * (uint32_t)lane : 8u * ((uint32_t)lane & 31u);
}

// bf16 halves of a float32 level: hi = round-to-nearest-even bf16, lo = the
// same rounding of the (exact) remainder.
__device__ __forceinline__ uint32_t level_hi(float v) { return f32_to_bf16_bits(v); }
__device__ __forceinline__ uint32_t level_lo(float v) { return f32_to_bf16_bits(v - bf16_bits_to_f32(f32_to_bf16_bits(v))); }

// One 32-bit word / one 8-byte entry of LDS at byte address `addr`.
__device__ __forceinline__ uint32_t lds_word(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((uintptr_t)addr);
}
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2v_t lds_entry(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x2v_t*>((uintptr_t)addr);
}

// 8-bit entries of two codes -> (hi pair, lo pair), the first code in the low halves.
__device__ __forceinline__ u32x2v_t split8(uint32_t w0, uint32_t w1) {
  return u32x2v_t{__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w1, w0, 0x07060302u)};
}

// Raw code bits of a lane's 16 weights of one block.
template <int BITS>
struct Raw;
template <> struct Raw<2> { uint32_t v; };
template <> struct Raw<3> { uint32_t lo, hi; };
template <> struct Raw<4> { uint32_t a, b; };
template <> struct Raw<8> { uint32_t a, b, c, d; };

// bf16 level halves of the lane's 16 weights: b0 = elements 0..7, b1 = 8..15
// (h = hi halves, l = lo halves, pairs in element order).
template <int BITS>
__device__ __forceinline__ void decode16(const Raw<BITS>& r, uint32_t tl, u32x4_t& b0h, u32x4_t& b0l, u32x4_t& b1h,
                                         u32x4_t& b1l) {
  auto put = [&](int i, u32x2v_t e0, u32x2v_t e1) {
    b0h[i] = e0.x; b0l[i] = e0.y;
    b1h[i] = e1.x; b1l[i] = e1.y;
  };
  if constexpr (BITS == 4) {
    // address built with one byte permute: code byte i into bits 8..15
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + i) << 8);
      put(i, lds_entry(__builtin_amdgcn_perm(r.a, tl, sel)), lds_entry(__builtin_amdgcn_perm(r.b, tl, sel)));
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      put(i, lds_entry((((r.v >> (4 * i)) & 15u) << 8) | tl), lds_entry((((r.v >> (16 + 4 * i)) & 15u) << 8) | tl));
  } else if constexpr (BITS == 3) {
    const uint64_t v = (uint64_t)r.lo | ((uint64_t)r.hi << 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      put(i, lds_entry(((uint32_t)((v >> (6 * i)) & 63u) << 8) | tl),
          lds_entry(((uint32_t)((v >> (24 + 6 * i)) & 63u) << 8) | tl));
  } else {
    const uint32_t w[4] = {r.a, r.b, r.c, r.d};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d0 = w[i >> 1], d1 = w[2 + (i >> 1)];
      const int sh = 16 * (i & 1);
      const uint32_t e00 = lds_word((((d0 >> sh) & 255u) << 8) | tl);
      const uint32_t e01 = lds_word((((d0 >> (sh + 8)) & 255u) << 8) | tl);
      const uint32_t e10 = lds_word((((d1 >> sh) & 255u) << 8) | tl);
      const uint32_t e11 = lds_word((((d1 >> (sh + 8)) & 255u) << 8) | tl);
      put(i, split8(e00, e01), split8(e10, e11));
    }
  }
}

// Level table of the single-row decode path: each level as one fp16 number
// (11 significant bits, so within 2^-11 of the level relative to it; every
// level of the 2-, 3-, 4- and 8-bit codebooks is a normal fp16 number), and
// the x row converted to fp16 with an exact power-of-two scale, so one packed
// fp16 dot product gives two exact level x products.
//   * 2-, 3- and 4-bit codes: entry e = the packed bits of two neighbouring
//     codes (the lower code in the low bits), one word: the two fp16 levels,
//     the lower code's in the low half.
//   * 8-bit codes: entry e = one code, its fp16 level in the low half.
// Copy L = lane of entry e sits at byte e*256 + 4L: no two lanes of a wave ever
// read the same bank.  Like PairTable it sits at LDS address 0, and a lookup
// address is (entry << 8) | table_lane_h(lane).
template <int BITS>
struct LevelTableH {
  static constexpr int kEntries = (BITS == 8) ? 256 : (1 << (2 * BITS));
  static constexpr int kBytes = kEntries * 256;
};
__device__ __forceinline__ uint32_t table_lane_h(int lane) { return 4u * (uint32_t)lane; }

// float32 level pairs for the prefill dequantizer: entry e (e = two packed
// codes, or one 8-bit code) of copy c at byte e*256 + 8c, c = lane % 32, so a
// wave's lanes 0..15 / 16..31 / 32..47 / 48..63 each read 16 different 8-byte
// bank pairs.  For 8-bit codes the entry holds one level (second float unused).
template <int BITS>
struct PairTableF32 {
  static constexpr int kEntries = (BITS == 8) ? 256 : (1 << (2 * BITS));
  static constexpr int kBytes = kEntries * 256;
};

}  // namespace qlr

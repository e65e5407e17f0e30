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

// One 32-bit word of LDS at byte address `addr`.
__device__ __forceinline__ uint32_t lds_word(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((uintptr_t)addr);
}

// Raw code bits of a lane's 16 weights of one block.
template <int BITS>
struct Raw;
template <> struct Raw<2> { uint32_t v; };
template <> struct Raw<3> { uint32_t lo, hi; };
template <> struct Raw<4> { uint32_t a, b; };
template <> struct Raw<8> { uint32_t a, b, c, d; };

// Unscaled bf16 levels of the lane's 16 weights: b0 = elements 0..7, b1 = 8..15.
// The table sits at LDS address 0, so a lookup address is (entry << 8) | lane*4.
template <int BITS>
__device__ __forceinline__ void decode16(const Raw<BITS>& r, uint32_t lane4, u32x4_t& b0, u32x4_t& b1) {
  if constexpr (BITS == 4) {
    // address built with one byte permute: code byte i into bits 8..15
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + i) << 8);
      b0[i] = lds_word(__builtin_amdgcn_perm(r.a, lane4, sel));
      b1[i] = lds_word(__builtin_amdgcn_perm(r.b, lane4, sel));
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b0[i] = lds_word((((r.v >> (4 * i)) & 15u) << 8) | lane4);
      b1[i] = lds_word((((r.v >> (16 + 4 * i)) & 15u) << 8) | lane4);
    }
  } else if constexpr (BITS == 3) {
    const uint64_t v = (uint64_t)r.lo | ((uint64_t)r.hi << 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b0[i] = lds_word(((uint32_t)((v >> (6 * i)) & 63u) << 8) | lane4);
      b1[i] = lds_word(((uint32_t)((v >> (24 + 6 * i)) & 63u) << 8) | lane4);
    }
  } else {
    const uint32_t w[4] = {r.a, r.b, r.c, r.d};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d0 = w[i >> 1], d1 = w[2 + (i >> 1)];
      const int sh = 16 * (i & 1);
      const uint32_t lo0 = lds_word((((d0 >> sh) & 255u) << 8) | lane4);
      const uint32_t hi0 = lds_word((((d0 >> (sh + 8)) & 255u) << 8) | lane4);
      const uint32_t lo1 = lds_word((((d1 >> sh) & 255u) << 8) | lane4);
      const uint32_t hi1 = lds_word((((d1 >> (sh + 8)) & 255u) << 8) | lane4);
      b0[i] = lo0 | (hi0 << 16);
      b1[i] = lo1 | (hi1 << 16);
    }
  }
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

}  // namespace qlr

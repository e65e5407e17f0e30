// Decode path (M <= 16, bf16 x): the dequantizing GEMV of the frozen base with
// the unmerged adapter added in the epilogue (t = x A^T comes from the
// adapter-product kernel launched just before; measured on this chip, a second
// launch costs less than handing t between workgroups of one launch, whose
// cross-XCD round trips sit on the critical path).
//
// The frozen base is read once, as packed k-bit codes (QLoRA page,
// memory-decomposition equation: the 4-bit base takes about half a byte per
// weight), so the kernel is bound by HBM bandwidth; the dequantization the
// QLoRA page's limitations section mentions is fused into the load path.
//
// Work decomposition: a persistent grid of 512-thread workgroups (one per CU)
// walks 16-row tiles of W; inside a workgroup the 8 waves split K (whole
// 64-element blocks) and are reduced through LDS at the end of every tile.
// Each wave streams its K slice in chunks of 4 blocks and keeps the next chunk
// in flight (in registers) while it computes the current one, across tile
// boundaries too.
//
// Loads are shaped for the vector memory pipeline, which serves a group of 4
// consecutive lanes per cycle when they read one 64-byte segment: the code
// bytes of a chunk (16 rows x 4 blocks) are read as 16-byte pieces, 8
// consecutive lanes per row, through a buffer resource (rows past N read as
// zero), and staged in a wave-private LDS slice; the absmax codes and group
// constants are read one (row, block) per lane, 4 consecutive blocks of a row
// per lane quad, turned into scales and staged beside them.
//
// Layout on the 16x16x32 bf16 MFMA (A = x rows, B = unscaled levels):
//   lane l: x row / weight row (l & 15), lane group g = l >> 4 owns the 16
//   consecutive elements [16g, 16g+16) of each 64-element block; one MFMA pair
//   takes elements [16g, 16g+8), another [16g+8, 16g+16).  All MFMAs of a
//   block stay inside that block, so the block's dequantized absmax
//   multiplies the 16x16 product afterwards (one FMA per output and block)
//   instead of every weight.
// Levels are looked up in an LDS table indexed by the packed code bits of two
// neighbouring weights, with a copy per lane position so that lanes never
// collide on a bank (qlr_lut.h).  A level rounded to bf16 alone is off by up
// to 2^-8 of its value, and with x and the weights of one sign those errors
// add up to more than the layer's 1e-3 bound.  So on the MFMA path each level
// enters as two bf16 halves, hi and lo (two MFMAs), which carry the float32
// level to about 2^-16; the single-row path takes it as one fp16 number
// (within 2^-11) and x as fp16 numbers with an exact power-of-two scale per
// block, one packed fp16 dot product per level pair (half the lookups and the
// products of two halves).
#include <algorithm>
#include <type_traits>

#include "qlr_internal.h"
#include "qlr_lut.h"

namespace qlr {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int CH = 4;  // blocks per chunk and wave

// Per-chunk geometry for BITS-bit codes: the code bytes of 16 rows x CH blocks
// are loaded as PB-byte pieces (8 bytes for 3-bit codes, whose 24-byte blocks
// are only 8-byte aligned) and staged with a row stride RS chosen to keep the
// MFMA-layout reads within 2-way bank conflicts.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int BITS>
struct ChunkGeo {
  static constexpr int kRowBytes = CH * 8 * BITS;
  static constexpr int PB = (BITS == 3) ? 8 : 16;
  static constexpr int PR = kRowBytes / PB;          // pieces per row
  static constexpr int NP = (16 * PR + 63) / 64;     // pieces per lane
  static constexpr int RS = kRowBytes + (BITS == 8 ? 16 : 8);
  static constexpr int kStage = 16 * RS + 16 * CH * 4;  // codes + scales, one buffer
  typedef typename std::conditional<PB == 16, u32x4_t, u32x2_t>::type Piece;
};

// One chunk of a wave's stream held in registers between its loads and its
// staging: raw code pieces, the (row, block) absmax code and group constant of
// this lane and the x fragments of the chunk's blocks (when x is not in LDS).
template <int BITS, bool XLDS>
struct Chunk {
  typename ChunkGeo<BITS>::Piece piece[ChunkGeo<BITS>::NP];
  uint32_t q8;
  float sc;
  u32x4_t x[XLDS ? 1 : CH][2];  // x fragments (unused when x is staged in LDS)
};
// 16-byte pieces of B rows each thread of the decode kernel loads up front:
// all the B rows of a workgroup's tiles (2 r pieces per tile) when they number
// at most kBPre * 512.
constexpr int kBPre = 2;

// Chunks a wave keeps in flight (the ring depth D): 4 for long streams, 2 when
// a wave's whole stream is at most 2 chunks or x rides with the chunks.  Every
// load instruction costs address-unit time even when it reads out of range,
// so the ring is no deeper than the stream.

// Largest x (bytes) staged once per workgroup in LDS instead of being read per
// chunk in the MFMA layout (which repeats every x row 16 times per wave).
constexpr size_t kXLdsMax = 32 * 1024;
// Adapter partial sums (float32) prefetched into registers, per thread: all of
// them, as the adapter-product split count guarantees (kTPartsMax).
constexpr int kTPre = kTPartsMax / kThreads;
static_assert(kTPre * kThreads == kTPartsMax, "prefetch covers every partial sum");
// the single-row path's fp16 table takes the place of the MFMA path's hi/lo table
static_assert(LevelTableH<2>::kBytes == PairTable<2>::kBytes && LevelTableH<3>::kBytes == PairTable<3>::kBytes &&
                  LevelTableH<4>::kBytes == PairTable<4>::kBytes && LevelTableH<8>::kBytes == PairTable<8>::kBytes,
              "one LDS layout for both tables");

// How the epilogue gets the adapter product t = x A^T: from the split partial
// sums of the adapter-product kernel (T_GLOBAL, T_LOOP, T_PREFETCH), or
// computed by every workgroup itself (T_FUSED, single row, r <= kFuseR).
enum { T_GLOBAL = 0, T_LOOP = 1, T_PREFETCH = 2, T_FUSED = 3 };
constexpr int kFuseR = 16;

struct Params {
  LinearArgs a;
  int64_t ntiles;
  int tmode;     // T_GLOBAL: summed per output from global memory; T_LOOP: summed
                 // into LDS after the first barrier; T_PREFETCH: partials loaded
                 // with the first chunks, summed into LDS; T_FUSED: x A^T
                 // computed in the kernel (per-wave sums at sTP)
  int bpre;      // the B rows of all of a workgroup's tiles are loaded into LDS up front
  uint32_t sT;   // LDS byte addresses: summed t (M x r), raw partials, B tile, x
  uint32_t sTP;
  uint32_t sB;
  uint32_t sX;
  uint32_t sXh;  // single-row path: the x row as fp16 numbers x 2^s_b
  uint32_t sXs;  // and its per-block exponents s_b (int32, kXsBad: not exact)
  uint32_t sZ;   // 128 zero bytes (x fragments of rows past M)
  uint32_t sW;   // float32 transform of the x row (Walsh-Hadamard side channel)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOOB = 0xFFFFFFF0u;  // buffer offset past every resource: reads zero, writes dropped

// `ok ? off : kOOB`, with `off` computed unconditionally: the pin keeps the
// compiler from turning the select into a branch around the access (which
// would give the accesses of one stream different counts on different paths
// and force full waits on the memory counter).
__device__ __forceinline__ uint32_t buf_off(bool ok, uint32_t off) {
  asm volatile("" : "+v"(off));
  return ok ? off : kOOB;
}

// LDS byte address in the dynamic block (which starts at LDS address 0: the
// kernel has no static LDS).
__device__ __forceinline__ u32x4_t lds_rd128(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((uintptr_t)addr);
}
__device__ __forceinline__ void lds_wr128(uint32_t addr, u32x4_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>((uintptr_t)addr) = v;
}
__device__ __forceinline__ uint2 lds_rd64(uint32_t addr) {
  const u32x2_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>((uintptr_t)addr);
  return uint2{v.x, v.y};
}
__device__ __forceinline__ void lds_wr64(uint32_t addr, uint2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>((uintptr_t)addr) = u32x2_t{v.x, v.y};
}
__device__ __forceinline__ uint32_t lds_rd32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((uintptr_t)addr);
}
__device__ __forceinline__ uint32_t lds_rd16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>((uintptr_t)addr);
}

// Raw codes of lane group g (16 codes) of block u of staged row at `row_addr`.
template <int BITS>
__device__ __forceinline__ Raw<BITS> raw_from_lds(uint32_t row_addr, int u, int g) {
  Raw<BITS> r;
  const uint32_t ad = row_addr + (uint32_t)(u * 8 * BITS + g * 2 * BITS);
  if constexpr (BITS == 2) {
    r.v = lds_rd32(ad);
  } else if constexpr (BITS == 4) {
    const uint2 v = lds_rd64(ad);
    r.a = v.x; r.b = v.y;
  } else if constexpr (BITS == 8) {
    const u32x4_t v = lds_rd128(ad);
    r.a = v[0]; r.b = v[1]; r.c = v[2]; r.d = v[3];
  } else {
    r.lo = lds_rd16(ad) | (lds_rd16(ad + 2) << 16);
    r.hi = lds_rd16(ad + 4);
  }
  return r;
}

// The level table (layout in qlr_lut.h), built straight from the by-value
// levels: wave w writes entries [w E/8, (w+1) E/8) of every copy, so an entry's
// level indices are uniform across the wave; for 3- and 4-bit codes the low
// level index runs over all levels within a wave and is a compile-time index
// (one batched scalar load), the high one takes E/8/NL values per wave.  For
// paired widths lane L writes word L >> 5 (hi pair or lo pair) of copy L % 32.
template <int BITS>
__device__ __forceinline__ void build_table_kernarg(uint32_t* tbl, const Levels& lv, int tid) {
  constexpr int NL = 1 << BITS;
  constexpr int E = PairTable<BITS>::kEntries;
  constexpr int EPW = E / kWaves;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lo_half = lane >= 32;
  uint32_t* t = tbl + (w * EPW) * 64 + (BITS == 8 ? lane : 2 * (lane & 31) + (lane >> 5));
  auto word = [&](float a, float b) {
    const uint32_t h = level_hi(a) | (level_hi(b) << 16);
    const uint32_t l = level_lo(a) | (level_lo(b) << 16);
    return lo_half ? l : h;
  };
  if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < EPW; ++i) {
      const float v = lv.v[w * EPW + i];
      t[i * 64] = level_hi(v) | (level_lo(v) << 16);
    }
  } else if constexpr (EPW >= NL) {
    float lo[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) lo[j] = lv.v[j];
#pragma unroll
    for (int i = 0; i < EPW; ++i) t[i * 64] = word(lo[i & (NL - 1)], lv.v[w * (EPW / NL) + (i >> BITS)]);
  } else {
#pragma unroll
    for (int i = 0; i < EPW; ++i) {
      const int e = w * EPW + i;
      t[i * 64] = word(lv.v[e & (NL - 1)], lv.v[e >> BITS]);
    }
  }
}

// The fp16 level table of the single-row path (layout in qlr_lut.h), from the
// by-value levels: wave w writes entries [w E/8, (w+1) E/8), one 256-byte entry
// (64 copies of one word) per store instruction, so an entry's level indices
// are uniform across the wave (batched scalar loads).  For 2-bit codes (16
// entries) waves 0 and 1 write them all.
template <int BITS>
__device__ __forceinline__ void build_table_h(uint32_t* tbl, const Levels& lv, int tid) {
  constexpr int NL = 1 << BITS;
  constexpr int E = LevelTableH<BITS>::kEntries;
  constexpr int EPW = (E / kWaves > 0) ? E / kWaves : 1;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (w * EPW >= E) return;
  uint32_t* t = tbl + (w * EPW) * 64 + lane;
  auto h16 = [](float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v); };
#pragma unroll
  for (int i = 0; i < EPW; ++i) {
    const int e = w * EPW + i;
    if constexpr (BITS == 8) {
      const uint32_t hv = h16(lv.v[e]);
      t[i * 64] = hv | (hv << 16);
    } else {
      t[i * 64] = h16(lv.v[e & (NL - 1)]) | (h16(lv.v[e >> BITS]) << 16);
    }
  }
}

// Sum over aligned groups of G consecutive lanes (G = 2, 4, 8 or 16), every
// lane of a group getting the group's sum, by row-local data-parallel moves:
// neighbour pairs, then quads, then the mirrored half of an 8-lane group, then
// the mirrored half of the 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2, 4, 8 or 16 lanes");
  v += dpp_mov<0xB1>(v);                      // lane ^ 1
  if constexpr (G >= 4) v += dpp_mov<0x4E>(v);  // lane ^ 2
  if constexpr (G >= 8) v += dpp_mov<0x141>(v); // 7 - lane within 8
  if constexpr (G >= 16) v += dpp_mov<0x140>(v);  // 15 - lane within 16
  return v;
}

// x rows for the MFMA path are loaded with each quad of lanes in one 64-byte
// segment (lane l: 16 bytes of row l / 4, piece l % 4 of the block's first
// half in h0 and of its second half in h1; a piece is 8 columns), the rate the
// address unit sustains; the 16x16x32 A fragments want lane 16 g + n to hold
// pieces 2 g (f0) and 2 g + 1 (f1) of row n.  Quad moves gather the even
// pieces of a row into one register and the odd ones into another (lane
// 4 n + q holding pieces (0, 4, 2, 6)[q] and (1, 5, 3, 7)[q]), and one lane
// permute per word moves them into place.
__device__ __forceinline__ void x_frag(const u32x4_t& h0, const u32x4_t& h1, int lane, u32x4_t& f0, u32x4_t& f1) {
  const bool odd = (lane & 1) != 0;
  const int g = lane >> 4;
  const int src = (4 * (lane & 15) + (((g & 1) << 1) | (g >> 1))) << 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // the quad moves run on every lane (their sources are the lane's neighbours),
    // then plain selects
    const uint32_t m1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h1[j], 0xA0, 0xF, 0xF, false);
    const uint32_t m0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h0[j], 0xF5, 0xF, 0xF, false);
    const uint32_t e = odd ? m1 : h0[j];
    const uint32_t o = odd ? h1[j] : m0;
    f0[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)e);
    f1[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)o);
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// Single-row products: sum over the codes of one piece (16 bytes of 2-, 4- or
// 8-bit codes) of level(code) * x, the levels looked up in the fp16 table (at
// LDS address 0) and paired with the matching x pairs (xv holds the piece's x
// values in order, 8 per 16-byte vector).  H: x is the fp16 row (scaled), one
// packed fp16 dot product per pair; otherwise x is the bf16 row and each pair
// takes two float32 multiply-adds (fp16 level and bf16 x are both exact in
// float32).  Two accumulation chains, added at the end.
template <bool H>
struct PairAcc {
  float s0 = 0.0f, s1 = 0.0f;
  // e: the two fp16 levels, xp: the two x values (both lower element in the low half)
  __device__ __forceinline__ void add(uint32_t e, uint32_t xp, bool odd) {
    float& s = odd ? s1 : s0;
    if constexpr (H) {
      s = dot2h(e, xp, s);
    } else {
      s = fmaf(f16_bits_to_f32((uint16_t)(e & 0xFFFFu)), bf16_bits_to_f32(xp & 0xFFFFu), s);
      s = fmaf(f16_bits_to_f32((uint16_t)(e >> 16)), bf16_bits_to_f32(xp >> 16), s);
    }
  }
  __device__ __forceinline__ float sum() const { return s0 + s1; }
};
// LDS address of entry (byte b of w) for the lane: one byte permute puts the
// byte into bits 8..15 over the lane's copy offset.
__device__ __forceinline__ uint32_t entry_addr(uint32_t w, uint32_t tl, int b) {
  return __builtin_amdgcn_perm(w, tl, 0x0C0C0000u | ((uint32_t)(4 + b) << 8));
}
template <int BITS, bool H>
__device__ __forceinline__ float dot_piece(const u32x4_t& pc, const u32x4_t* xv, uint32_t tl) {
  PairAcc<H> acc;
  if constexpr (BITS == 4) {
    // byte b of word w = pair 4w + b
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc.add(lds_word(entry_addr(pc[w], tl, b)), xv[w][b], b & 1);
  } else if constexpr (BITS == 2) {
    // nibble n of word w = pair 8w + n; the even nibbles spread into bytes by one
    // mask, the odd ones by a shift and the mask
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t ev = pc[w] & 0x0F0F0F0Fu, od = (pc[w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int n = 0; n < 8; ++n)
        acc.add(lds_word(entry_addr((n & 1) ? od : ev, tl, n >> 1)), xv[2 * w + (n >> 2)][n & 3], n & 1);
    }
  } else {
    // byte b of word w = code 4w + b; codes 2p and 2p + 1 make x pair p
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t e0 = lds_word(entry_addr(pc[w], tl, 2 * j));
        const uint32_t e1 = lds_word(entry_addr(pc[w], tl, 2 * j + 1));
        acc.add(__builtin_amdgcn_perm(e1, e0, 0x05040100u), xv[w >> 1][2 * (w & 1) + j], j);
      }
  }
  return acc.sum();
}

// x as scaled fp16 numbers, per 64-column block b of the row: x 2^s_b, with s_b
// the power of two that puts the block's largest |x| in [2^14, 2^15).  A block
// is exact when each of its values is then a normal fp16 number or zero, so
// that every product with an fp16 level is exact in float32; a block holding
// Inf or NaN, or whose largest |x| is below 2^-126, is not.  The 8 pieces of a
// block sit in 8 neighbouring lanes (the staging order), which reduce its
// largest |x| and its exactness among themselves.  kXsBad marks a block that
// is not exact in the scale array.
constexpr int kXsBad = 0x7FFFFFFF;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t group_max8(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // lane ^ 1
  v = max(v, dpp_u32<0x4E>(v));   // lane ^ 2
  return max(v, dpp_u32<0x141>(v));  // 7 - lane within 8
}
__device__ __forceinline__ uint32_t group_min8(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));
  v = min(v, dpp_u32<0x4E>(v));
  return min(v, dpp_u32<0x141>(v));
}
// h: the piece's 8 values as fp16 x 2^s_b; returns s_b, or kXsBad.  On the bf16
// bits: a value 1.m x 2^(E - 127) (exponent field E, 7-bit m) becomes 1.m x
// 2^(E - 127 + s), whose fp16 exponent field is E - 112 + s, so the fp16 bits
// without the sign are ((E << 7 | m) + (s - 112) 128) << 3; it is a normal fp16
// number when that field is at least 1, i.e. when E << 7 | m >= max(1, 113 - s)
// 128 (subnormal bf16 values, E = 0, never pass).  The field is at most 29 for
// the block's largest value, so the sums stay below 2^12 per 16-bit half.
__device__ __forceinline__ int x_piece_f16(const u32x4_t& xb, u32x4_t& h) {
  typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
  u16x2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};  // largest |x| bits; smallest |x| bits - 1 (0 wraps to 0xFFFF)
  u16x2_t a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = __builtin_bit_cast(u16x2_t, xb[j] & 0x7FFF7FFFu);
    mx = __builtin_elementwise_max(mx, a[j]);
    mn = __builtin_elementwise_min(mn, a[j] - (u16x2_t){1, 1});
  }
  const uint32_t m = group_max8(max((uint32_t)mx.x, (uint32_t)mx.y));
  const uint32_t lo = group_min8(min((uint32_t)mn.x, (uint32_t)mn.y));
  // |x| bits >= 0x7F80: Inf or NaN; below 0x0080 (and not 0): a subnormal largest |x|
  const bool scalable = m < 0x7F80u && (m == 0u || m >= 0x0080u);
  const int s = m == 0u ? 0 : 141 - (int)(m >> 7);
  const uint32_t tmin = (uint32_t)max(1, 113 - s) * 128u;
  const bool ok = scalable && (lo == 0xFFFFu || lo + 1u >= tmin);
  const uint16_t bias = (uint16_t)((s - 112) * 128);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u16x2_t v = (a[j] + (u16x2_t){bias, bias}) << (u16x2_t){3, 3};
    v = v * __builtin_elementwise_min(a[j], (u16x2_t){1, 1});  // zeros stay zero
    h[j] = __builtin_bit_cast(uint32_t, v) | (xb[j] & 0x80008000u);
  }
  return ok ? s : kXsBad;
}
// Whether every block [b0, b1) of the row (at most 64) is exact, uniformly over the wave.
__device__ __forceinline__ bool x_blocks_exact(uint32_t sxs, int64_t b0, int64_t b1, int lane) {
  const int64_t b = b0 + lane;
  const int v = b < b1 ? (int)lds_rd32(sxs + (uint32_t)b * 4u) : 0;
  return __builtin_amdgcn_ballot_w64(v == kXsBad) == 0;
}

// ADP: the call has an adapter branch (r > 0); calls without one run a separate
// instantiation, which also gives it its own kernel name.
// DOT (a single x row, 2-, 4- or 8-bit codes): the codes are used straight from
// the registers they were loaded into, each lane taking 16-byte pieces of
// rows; level pairs are looked up and multiplied with x pairs by packed fp16
// dot products (a wave whose x blocks are not all exact in fp16 takes float32
// products of the same levels with the bf16 row), and the row sums are
// reduced across the lanes of a row and the waves at the end of a tile.  Otherwise the codes are staged through LDS into
// the 16x16x32 MFMA layout (x rows as the A operand).
//
// Every global access of the chunk stream is issued unconditionally (out-of-
// range pieces read zero through buffer resources), so the compiler's memory
// counters see the same outstanding loads on every path and a chunk's compute
// waits for that chunk only, never for the chunks issued after it.
// TF (single-row path, adapter rank <= 16, one 512-element K sweep per wave):
// every workgroup also computes t = x A^T itself, from A rows read after the
// code stream has been issued (L2-resident after the first workgroup of each
// XCD), instead of reading the partial sums of a separate kernel.
// XR (MFMA path, x read from global memory, exactly two chunks per wave and
// tile, 40..64 blocks per row): the wave's x fragments (its 8 blocks of the 16
// x rows in the MFMA layout, 64 registers) are loaded once, before the chunk
// stream, instead of riding with every chunk: a chunk's loads are then its
// code pieces and scales only, and x is read once per workgroup, not per tile.
template <int BITS, int YDT, bool XLDS, bool ADP, int D, bool DOT, bool TF, int SPX, bool DBA, bool XR>
__global__ __launch_bounds__(kThreads, 1) void k_gemv(Params P, Levels lv) {
  static_assert(!DOT || (XLDS && BITS != 3), "the single-row path reads x from LDS and 16-byte pieces of whole codes");
  static_assert(!TF || (DOT && ADP), "the fused adapter product belongs to the single-row path");
  static_assert(SPX == 0 || DOT, "the fused side channel belongs to the single-row path");
  static_assert(!DBA || TF, "the double-binary branch is fused through the adapter product");
  static_assert(!XR || (!XLDS && !DOT && (D == 2 || D == 4)), "x in registers: MFMA path, x from global memory");
  // per-wave LDS staging buffer: codes and scales, or scales only (single-row path)
  constexpr uint32_t kStageW = DOT ? 16 * CH * 4 : ChunkGeo<BITS>::kStage;
  using G = ChunkGeo<BITS>;
  using Ch = Chunk<BITS, XLDS || XR>;
  constexpr int ES = (YDT == DT_F32) ? 4 : 2;
  extern __shared__ uint32_t smem[];
  const LinearArgs& a = P.a;
  const int64_t N = a.N, K = a.K, nb = K >> 6;
  const int M = (int)a.M;
  const int r = ADP ? a.r : 0;
  const int mr = M * r;
  uint32_t* tbl = smem;
  // LDS: level table | per-wave staging (2 buffers) | sRed (waves x 256) | t | t partials | B tile | x
  const uint32_t stage0 = (uint32_t)PairTable<BITS>::kBytes;
  float* sRed = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + stage0 + kWaves * 2 * kStageW);
  float* sT = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + P.sT);

  const int tid = threadIdx.x;
  // (the wave index is uniform within a wave: saying so keeps the chunk loops scalar)
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const uint32_t tlane = DOT ? table_lane_h(lane) : table_lane<BITS>(lane);
  const int64_t kb0 = nb * wave / kWaves, kb1 = nb * (wave + 1) / kWaves;
  const int nchunk = (int)((kb1 - kb0 + CH - 1) / CH);
  const int nitem = nchunk > 0 ? nchunk : 1;  // items (chunks) per tile for this wave
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // x row of this lane's A fragments: in LDS, lanes of rows past M read a
  // 128-byte zero strip at a fixed address; from global memory, they are zeroed
  // after the load
  const bool xvalid = nl < M;
  const uint32_t xlane = xvalid ? P.sX + (uint32_t)(nl * (K + 8) * 2 + 32 * g) : P.sZ + 32u * g;
  const uint32_t xstep = xvalid ? 128u : 0u;
  // coalesced x pieces of row lane / 4 (clamped into x), moved into the
  // fragment layout by x_frag where they are used
  const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x) + (int64_t)min(lane >> 2, M - 1) * K + 8 * (lane & 3);
  const __amdgpu_buffer_rsrc_t cr = rsrc(a.codes, N * nb * 8 * BITS);
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.q8, N * nb);
  const __amdgpu_buffer_rsrc_t sr = rsrc(a.cst, ((N * nb + 255) >> 8) * 4);
  const uint32_t wstage = stage0 + (uint32_t)wave * 2 * kStageW;
  // scale-loading lane: (row lane / 4, block lane % 4) of a chunk
  const int srow = lane >> 2, sblk = lane & 3;

  // Byte offsets of this lane's loads at chunk 0 of tile blockIdx.x, formed
  // once; chunk c of a tile adds c * CH blocks, each later tile of the
  // workgroup gridDim.x * 16 rows (32-bit adds only).  Rows past N, and the
  // tiles past the last that the ring loads ahead, lie past the end of the
  // buffer resources and read zero, or (offsets wrapping past 2^32) bytes of
  // other rows: either way only sums that are never stored see them, so the
  // loads need no bounds test.  Blocks past the wave's K range are read and not
  // added.
  const uint32_t nb32 = (uint32_t)nb;
  const uint32_t kb032 = (uint32_t)kb0;
  const uint32_t rowb = nb32 * (8u * BITS);  // code bytes per weight row
  const uint32_t row_first = (uint32_t)blockIdx.x * 16u;
  uint32_t coff0[G::NP];
#pragma unroll
  for (int i = 0; i < G::NP; ++i) {
    const int p = i * 64 + lane;
    coff0[i] = (row_first + (uint32_t)(p / G::PR)) * rowb + kb032 * (8u * BITS) + (uint32_t)((p % G::PR) * G::PB);
  }
  const uint32_t qoff0 = (row_first + (uint32_t)srow) * nb32 + kb032 + (uint32_t)sblk;
  const uint32_t tstep_c = (uint32_t)gridDim.x * 16u * rowb, tstep_q = (uint32_t)gridDim.x * 16u * nb32;
  // load cursor: its tile, chunk, and the tile's offset from tile blockIdx.x
  int64_t ltile = blockIdx.x;
  int lc = 0;
  uint32_t lct = 0, lqt = 0;
  auto load_chunk = [&](Ch& ch) {
    const int c = lc;
    const uint32_t cb = (uint32_t)c * (uint32_t)CH;
    // code pieces: piece p -> row p / PR, byte (p % PR) * PB of the chunk row
#pragma unroll
    for (int i = 0; i < G::NP; ++i) {
      uint32_t off = coff0[i] + lct + cb * (8u * BITS);
      asm volatile("" : "+v"(off));
      if constexpr (G::PB == 16) {
        ch.piece[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cr, off, 0, 0));
      } else {
        ch.piece[i] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(cr, off, 0, 0));
      }
    }
    // absmax code and group constant of (row srow, block kbs + sblk)
    {
      uint32_t blk = qoff0 + lqt + cb;
      asm volatile("" : "+v"(blk));
      ch.q8 = __builtin_amdgcn_raw_buffer_load_b8(qr, blk, 0, 0);
      ch.sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, (blk >> 8) << 2, 0, 0));
    }
    // x fragments of the chunk's blocks (clamped into the row; unused past kb1)
    if constexpr (!XLDS && !XR) {
      const int64_t kbs = kb0 + (int64_t)c * CH;
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int64_t kb = min(kbs + u, nb - 1);
        ch.x[u][0] = *reinterpret_cast<const u32x4_t*>(xg + kb * 64);
        ch.x[u][1] = *reinterpret_cast<const u32x4_t*>(xg + kb * 64 + 32);
      }
    }
    if (++lc == nitem) {
      lc = 0;
      ltile += gridDim.x;
      lct += tstep_c;
      lqt += tstep_q;
    }
  };

  // Sparse side channel (SPX, a single x row; SPX = 1: the entries multiply x,
  // SPX = 2: they multiply the Walsh-Hadamard transform of x, formed in LDS).
  // Tile row o = tid >> 5 belongs to 32 consecutive lanes (half a wave); lane
  // i = tid & 31 holds the row's CSR offsets and its entries i + 32 e, e < 8
  // (clamped, unconditional loads: each load instruction reads two contiguous
  // runs), so 256 entries per row are in registers and the row's sum is a
  // reduction across its 32 lanes.  The first tile's offsets are loaded before
  // everything else and its entries right after x is in LDS, so both have long
  // arrived when the tile ends; later tiles load theirs at the tile's end.
  constexpr int kSpE = 8;
  int64_t sp0 = 0, sp1 = 0;
  int32_t spc[kSpE];
  float spv[kSpE];
  auto sp_rows = [&](int64_t tile) {
    const int64_t n = min(tile * 16 + (tid >> 5), N - 1);
    // offsets clamped into range: a malformed CSR gives wrong sums, never a stray access
    sp0 = min<int64_t>(max<int64_t>(a.sp_row_ptr[n], 0), a.sp_nnz);
    sp1 = max<int64_t>(sp0, min<int64_t>(a.sp_row_ptr[n + 1], a.sp_nnz));
  };
  auto sp_entries = [&]() {
#pragma unroll
    for (int e = 0; e < kSpE; ++e) {
      const int64_t j = min(sp0 + (tid & 31) + 32 * e, a.sp_nnz - 1);
      spc[e] = min<int32_t>(max<int32_t>(a.sp_col[j], 0), (int32_t)(K - 1));
      spv[e] = a.sp_val[j];
    }
  };
  // (SPX = 2) the x row's 16-byte pieces 8 (tid + 512 g) .. + 7, loaded first
  constexpr int kWG = 4;  // pieces per thread: up to 4 x 4096 columns
  u32x4_t wx[kWG];
  if constexpr (SPX == 2) {
    const uint16_t* x0 = reinterpret_cast<const uint16_t*>(a.x);
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
      const int64_t e0 = 4096 * g + 8 * (int64_t)tid;
      wx[g] = *reinterpret_cast<const u32x4_t*>(x0 + (e0 < K ? e0 : 0));
    }
  }
  if constexpr (SPX != 0) sp_rows(blockIdx.x);

  // Small x: one coalesced copy into LDS per workgroup (rows at stride K + 8),
  // loaded first, so that waiting for it does not wait for the code stream.
  // Load i is issued only if some thread has a piece in it (a workgroup-wide
  // condition).
  constexpr int kXPer = (int)(kXLdsMax / 16 / kThreads);  // 16-byte pieces per thread (4)
  u32x4_t xst[kXPer];
  const int64_t xpieces = (int64_t)M * (K / 8);
  if constexpr (XLDS) {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      if ((int64_t)i * kThreads < xpieces) {
        const int64_t q = tid + (int64_t)i * kThreads;
        const int64_t qc = q < xpieces ? q : 0;
        xst[i] = *reinterpret_cast<const u32x4_t*>(x + qc * 8);
      }
    }
  }
  // (adapter) the B rows of this workgroup's tiles, 16 x r bf16 each (tile g of
  // the workgroup, blockIdx.x + g gridDim.x, at sB + 32 r g): piece p = tid +
  // 512 i, issued after x and before the chunk stream, written to LDS before
  // the first barrier
  const int64_t ntl = (P.ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;  // tiles of this workgroup
  const int bpieces = (ADP && !DBA && (TF || P.bpre)) ? (int)ntl * 2 * r : 0;
  u32x4_t bpv[ADP ? kBPre : 1];
  if constexpr (ADP) {
    const __amdgpu_buffer_rsrc_t brs = rsrc(a.B, N * r * 2);
#pragma unroll
    for (int i = 0; i < kBPre; ++i) {
      const int p = tid + i * kThreads;
      const int gt = p / (2 * max(r, 1)), pc = p - gt * 2 * r;
      const uint32_t off = ((uint32_t)blockIdx.x + (uint32_t)gt * gridDim.x) * (uint32_t)(32 * r) + (uint32_t)pc * 16u;
      bpv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, buf_off(p < bpieces, off), 0, 0));
    }
  }
  // adapter partials, when prefetched: element tid + 512 i of the splits x M x r array
  float tp[kTPre];
  const int tcount = (ADP && !TF && P.tmode == T_PREFETCH) ? a.t_splits * mr : 0;
  if constexpr (ADP && !TF) {
    const __amdgpu_buffer_rsrc_t trs = rsrc(a.t, (int64_t)tcount * 4);
#pragma unroll
    for (int i = 0; i < kTPre; ++i) {
      const int q = tid + i * kThreads;
      tp[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(trs, buf_off(q < tcount, (uint32_t)q * 4u), 0, 0));
    }
  }

  // (XR) the x fragments of the wave's blocks kb0 .. kb0 + 7 (clamped into the
  // row; those past kb1 are never added), before the chunk stream
  u32x4_t xr[XR ? 2 * CH : 1][2];
  if constexpr (XR) {
#pragma unroll
    for (int u = 0; u < 2 * CH; ++u) {
      const int64_t kb = min(kb0 + u, nb - 1);
      xr[u][0] = *reinterpret_cast<const u32x4_t*>(xg + kb * 64);
      xr[u][1] = *reinterpret_cast<const u32x4_t*>(xg + kb * 64 + 32);
    }
  }

  // the first D chunks of this wave's stream (tiles blockIdx.x, + gridDim.x, ...)
  Ch ring[D];
#pragma unroll
  for (int s = 0; s < D; ++s) load_chunk(ring[s]);

  if constexpr (SPX == 2) {
    // Transform of the x row in blocks of P = 2^lp columns, float32 at sW
    // (unscaled), part 1: piece g of thread tid covers columns 8 (tid + 512 g) ..
    // + 7, so a wave holds 512 consecutive columns; column bits 0-2 are combined
    // in registers and bits 3-8 across the wave's lanes.  No barrier: it runs
    // while the first chunks are in flight, and the prologue's barrier ends it.
    const int lp = a.sp_wht_lp;
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
      const int64_t e0 = 4096 * g + 8 * (int64_t)tid;
      if (4096 * g >= K) break;  // uniform
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = bf16_bits_to_f32((wx[g][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
#pragma unroll
      for (int st = 1; st < 8; st <<= 1)
        if ((1 << lp) > st) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (!(j & st)) {
              const float u = v[j], w = v[j + st];
              v[j] = u + w;
              v[j + st] = u - w;
            }
        }
      // lane bits 0-1: DPP quad permutations; 2-3: swizzles (xor within 32
      // lanes); 4-5: half swaps, which hand every lane both operands (a = the
      // lower lane's value, b = the upper's) so that the pair becomes (a + b, a - b)
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
        if (lp > 3 + sb) {
          const bool up = (lane >> sb) & 1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int vi = __float_as_int(v[j]);
            int oi;
            if (sb == 0) oi = __builtin_amdgcn_mov_dpp(vi, 0xB1, 0xF, 0xF, false);
            else if (sb == 1) oi = __builtin_amdgcn_mov_dpp(vi, 0x4E, 0xF, 0xF, false);
            else if (sb == 2) oi = __builtin_amdgcn_ds_swizzle(vi, (4 << 10) | 0x1F);
            else oi = __builtin_amdgcn_ds_swizzle(vi, (8 << 10) | 0x1F);
            const float o = __int_as_float(oi);
            v[j] = up ? o - v[j] : v[j] + o;
          }
        }
      if (lp > 7) {
        const bool up = (lane >> 4) & 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
          const float lo = __uint_as_float(sw[0]), hi = __uint_as_float(sw[1]);
          v[j] = up ? lo - hi : lo + hi;
        }
      }
      if (lp > 8) {
        const bool up = (lane >> 5) & 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
          const float lo = __uint_as_float(sw[0]), hi = __uint_as_float(sw[1]);
          v[j] = up ? lo - hi : lo + hi;
        }
      }
      if (e0 < K) {
        lds_wr128(P.sW + (uint32_t)e0 * 4u, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                  __float_as_uint(v[2]), __float_as_uint(v[3])});
        lds_wr128(P.sW + (uint32_t)e0 * 4u + 16u, u32x4_t{__float_as_uint(v[4]), __float_as_uint(v[5]),
                                                        __float_as_uint(v[6]), __float_as_uint(v[7])});
      }
    }
  }
  if constexpr (DOT) build_table_h<BITS>(tbl, lv, tid);
  else build_table_kernarg<BITS>(tbl, lv, tid);
  if constexpr (XLDS) {
    if (tid < 8) lds_wr128(P.sZ + 16u * tid, zero);
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int64_t q = tid + (int64_t)i * kThreads;
      if constexpr (DOT) {
        // (single row) also the fp16 form, and block q / 8's exponent from its first lane
        if ((int64_t)i * kThreads < xpieces) {
          u32x4_t xh;
          const int sb = x_piece_f16(q < xpieces ? xst[i] : zero, xh);
          if (q < xpieces) {
            lds_wr128(P.sX + (uint32_t)q * 16u, xst[i]);
            lds_wr128(P.sXh + (uint32_t)q * 16u, xh);
            if ((q & 7) == 0) *reinterpret_cast<__attribute__((address_space(3))) int*>((uintptr_t)(P.sXs + (uint32_t)(q >> 3) * 4u)) = sb;
          }
        }
      } else if (q < xpieces) {
        const int64_t m = q / (K / 8), c8 = q % (K / 8);
        lds_wr128(P.sX + (uint32_t)((m * (K + 8) + c8 * 8) * 2), xst[i]);
      }
    }
  }
  if constexpr (ADP) {
#pragma unroll
    for (int i = 0; i < kBPre; ++i) {
      const int p = tid + i * kThreads;
      if (p < bpieces) lds_wr128(P.sB + (uint32_t)p * 16u, bpv[i]);
    }
  }
  if constexpr (ADP && !TF) {
    float* sTP = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + P.sTP);
#pragma unroll
    for (int i = 0; i < kTPre; ++i) {
      const int q = tid + i * kThreads;
      if (q < tcount) sTP[q] = tp[i];
    }
  }
  if constexpr (SPX != 0) sp_entries();
  // fused adapter product: lane's 8 elements k0 .. k0 + 7 of every A row j < 16
  // (rows past r and elements past the wave's range read as zero), issued after
  // the table and x are in LDS (issuing them holds the wave for a while)
  u32x4_t afr[TF && !DBA ? kFuseR : 1];
  const int64_t tk0 = kb0 * 64 + 8 * lane;
  const bool tkv = tk0 < kb1 * 64;
  // (DBA) the double-binary branch in place of A: gamma at the lane's 8 columns
  // (fp16) and, per row j of B2, the 8 sign bits of those columns
  u32x4_t dg = {0u, 0u, 0u, 0u};
  uint32_t dbits[DBA ? kFuseR : 1];
  if constexpr (DBA) {
    const int64_t kc = tkv ? tk0 : 0;
    dg = *reinterpret_cast<const u32x4_t*>(a.dba_gamma + kc);
    const int64_t w2 = (K + 31) / 32;
#pragma unroll
    for (int j = 0; j < kFuseR; ++j) {
      const uint32_t wd = a.dba_b2[(int64_t)(j < r ? j : 0) * w2 + (kc >> 5)];
      dbits[j] = (wd >> (kc & 31)) & 0xFFu;
    }
  } else if constexpr (TF) {
    const __amdgpu_buffer_rsrc_t ars = rsrc(a.A, (int64_t)r * K * 2);
#pragma unroll
    for (int j = 0; j < kFuseR; ++j)
      afr[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               ars, buf_off(tkv && j < r, (uint32_t)((j * K + tk0) * 2)), 0, 0));
  }
  __syncthreads();
  if constexpr (SPX == 2) {
    // part 2: column bits 9 and up, in LDS rounds of up to 3 bits (each ends
    // with a barrier, the last one before any epilogue reads the transform)
    const int lp = a.sp_wht_lp;
    for (int b = 9; b < lp; b += 3) {
      const int nbit = min(3, lp - b);
      const int R = 1 << nbit;
      const int64_t h = int64_t(1) << b;
      for (int64_t t = tid; t < (K >> nbit); t += kThreads) {
        const int64_t c0 = ((t >> b) << (b + nbit)) | (t & (h - 1));
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < R) v[j] = __uint_as_float(lds_rd32(P.sW + (uint32_t)(c0 + j * h) * 4u));
#pragma unroll
        for (int st = 1; st < 8; st <<= 1)
          if (st < R) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (j < R && !(j & st)) {
                const float u = v[j], w = v[j + st];
                v[j] = u + w;
                v[j + st] = u - w;
              }
          }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < R)
            *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)(P.sW + (uint32_t)(c0 + j * h) * 4u)) =
                v[j];
      }
      __syncthreads();
    }
  }
  // sT[i] = sum over parts of src[part][i], in part order, staged through sRed
  auto stage_t = [&](const float* src, int nparts) {
    const int per = mr > 0 ? max(1, (kWaves * 256) / mr) : 1;
    for (int p0 = 0; p0 < nparts; p0 += per) {
      const int np = min(per, nparts - p0);
      for (int idx = tid; idx < np * mr; idx += kThreads) sRed[idx] = src[(int64_t)p0 * mr + idx];
      __syncthreads();
      for (int i = tid; i < mr; i += kThreads) {
        float acc = (p0 == 0) ? 0.0f : sT[i];
        for (int q = 0; q < np; ++q) acc += sRed[q * mr + i];
        sT[i] = acc;
      }
      __syncthreads();
    }
  };
  if constexpr (ADP && !TF) {
    if (P.tmode == T_PREFETCH) {
      // summed in part order; read by the epilogue after the first tile's barrier
      const float* sTP = reinterpret_cast<const float*>(reinterpret_cast<const char*>(smem) + P.sTP);
      for (int i = tid; i < mr; i += kThreads) {
        float acc = 0.0f;
        for (int q = 0; q < a.t_splits; ++q) acc += sTP[q * mr + i];
        sT[i] = acc;
      }
    } else if (P.tmode == T_LOOP) {
      stage_t(a.t, a.t_splits);
    }
  }

  // (single-row path) the wave multiplies the fp16 x row when all its blocks are
  // exact (hx), else the bf16 row
  bool hx = false;
  if constexpr (DOT) hx = x_blocks_exact(P.sXs, kb0, kb1, lane);

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float accd[G::NP];  // single-row path: one row sum per piece
#pragma unroll
  for (int i = 0; i < G::NP; ++i) accd[i] = 0.0f;
  constexpr int CP = 128 / BITS;                   // codes per 16-byte piece
  constexpr int PPB = (BITS == 3) ? 1 : 64 / CP;   // pieces per block

  // Single-row chunk: lane's pieces i cover rows (64 i + lane) / PR, the same
  // K range (piece column lane % PR), so one x read serves all of them.
  auto compute_dot = [&](const Ch& ch, int64_t tl, int c, int buf) {
    if constexpr (DOT) {
      const uint32_t sscale = wstage + (uint32_t)buf * kStageW;
      {
        const bool nvalid = tl * 16 + srow < N;
        const float ap = nvalid ? (float)ch.q8 * ch.sc : 0.0f;
        *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)(sscale + (uint32_t)(srow * CH + sblk) * 4)) = ap;
      }
      const int64_t kbs = kb0 + (int64_t)c * CH;
      const int col = lane % G::PR;
      const int u = col / PPB;
      const bool bval = kbs + u < kb1;  // blocks past the wave's range are read but not added
      const uint32_t xa = (hx ? P.sXh : P.sX) + (uint32_t)((kbs * 64 + col * CP) * 2);
      u32x4_t xv[CP / 8];
  #pragma unroll
      for (int q = 0; q < CP / 8; ++q) xv[q] = lds_rd128(xa + 16u * q);
      // the pieces' block scales and the lane's block exponent (blocks past the row read the
      // array's padding, never added), read before the products so their latency is hidden
      float ap[G::NP];
  #pragma unroll
      for (int i = 0; i < G::NP; ++i)
        ap[i] = __uint_as_float(lds_rd32(sscale + (uint32_t)(((i * 64 + lane) / G::PR) * CH + u) * 4));
      const int sb = (int)lds_rd32(P.sXs + (uint32_t)(kbs + u) * 4u);
      float sp[G::NP];
      if (hx) {
  #pragma unroll
        for (int i = 0; i < G::NP; ++i)
          sp[i] = ldexpf(dot_piece<BITS, true>(__builtin_bit_cast(u32x4_t, ch.piece[i]), xv, tlane), -sb);
      } else {
  #pragma unroll
        for (int i = 0; i < G::NP; ++i) sp[i] = dot_piece<BITS, false>(__builtin_bit_cast(u32x4_t, ch.piece[i]), xv, tlane);
      }
  #pragma unroll
      for (int i = 0; i < G::NP; ++i) accd[i] = fmaf(ap[i], bval ? sp[i] : 0.0f, accd[i]);
    }
  };

  // Stage a chunk's codes and scales in this wave's LDS buffer `buf` (only this
  // wave reads them, and a wave's LDS instructions run in order), then compute.
  // (XR: `slot` is the ring slot, whose chunk index within its tile is slot % 2)
  auto compute = [&](const Ch& ch, int64_t tl, int c, int buf, int slot) {
    const uint32_t sb = wstage + (uint32_t)buf * G::kStage;
#pragma unroll
    for (int i = 0; i < G::NP; ++i) {
      const int p = i * 64 + lane;
      if (p < 16 * G::PR) {
        const uint32_t ad = sb + (uint32_t)((p / G::PR) * G::RS + (p % G::PR) * G::PB);
        if constexpr (G::PB == 16) lds_wr128(ad, ch.piece[i]);
        else lds_wr64(ad, uint2{ch.piece[i].x, ch.piece[i].y});
      }
    }
    const uint32_t sscale = sb + 16 * G::RS;
    {
      const bool nvalid = tl * 16 + srow < N;
      const float ap = nvalid ? (float)ch.q8 * ch.sc : 0.0f;
      *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)(sscale + (uint32_t)(srow * CH + sblk) * 4)) = ap;
    }
    const u32x4_t aps = lds_rd128(sscale + (uint32_t)nl * (CH * 4));
    const uint32_t rowad = sb + (uint32_t)nl * G::RS;
    const int64_t kbs = kb0 + (int64_t)c * CH;
    // block u of the chunk: two 16x16x32 products of the lane's x and level fragments
    auto block = [&](int u) {
      u32x4_t x0, x1;
      if constexpr (XLDS) {
        const uint32_t xa = xlane + (uint32_t)(kbs + u) * xstep;
        x0 = lds_rd128(xa);
        x1 = lds_rd128(xa + 16);
      } else if constexpr (XR) {
        x0 = xvalid ? xr[(slot & 1) * CH + u][0] : zero;
        x1 = xvalid ? xr[(slot & 1) * CH + u][1] : zero;
      } else {
        x_frag(ch.x[u][0], ch.x[u][1], lane, x0, x1);
        x0 = xvalid ? x0 : zero;
        x1 = xvalid ? x1 : zero;
      }
      u32x4_t b0h, b0l, b1h, b1l;
      decode16<BITS>(raw_from_lds<BITS>(rowad, u, g), tlane, b0h, b0l, b1h, b1l);
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
      d = mfma16x16x32(as_bf16x8(x0), as_bf16x8(b0h), d);
      d = mfma16x16x32(as_bf16x8(x1), as_bf16x8(b1h), d);
      d = mfma16x16x32(as_bf16x8(x0), as_bf16x8(b0l), d);
      return mfma16x16x32(as_bf16x8(x1), as_bf16x8(b1l), d);
    };
    auto accumulate = [&](int u, const f32x4_t& d) {
      const float ap = __uint_as_float(aps[u]);
      acc[0] = fmaf(ap, d[0], acc[0]);
      acc[1] = fmaf(ap, d[1], acc[1]);
      acc[2] = fmaf(ap, d[2], acc[2]);
      acc[3] = fmaf(ap, d[3], acc[3]);
    };
    if (kbs + CH <= kb1) {
      // whole chunk in the wave's K range: no branches between the blocks, so
      // their LDS reads, lookups and products overlap
      f32x4_t d[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) d[u] = block(u);
#pragma unroll
      for (int u = 0; u < CH; ++u) accumulate(u, d[u]);
    } else {
#pragma unroll
      for (int u = 0; u < CH; ++u)
        if (kbs + u < kb1) accumulate(u, block(u));
    }
  };

  const __amdgpu_buffer_rsrc_t yr = rsrc(a.y, (int64_t)M * N * ES);
  // Reduce the K slices of a finished tile and write its outputs.  All 512
  // threads run the epilogue (threads 256.. repeat outputs 0..255 and store out
  // of range), so the stores are issued on every path.
  // Fused adapter product, per wave: t_j over the wave's K range, reduced over
  // the 64 lanes by halving exchanges (lane l ends with j = l >> 2), written
  // to the wave's 16 slots at sTP; the waves are summed after the next barrier.
  auto compute_t = [&]() {
    if constexpr (TF) {
      const u32x4_t xv = lds_rd128(P.sX + (uint32_t)(tkv ? tk0 * 2 : 0));
      float v[kFuseR];
      if constexpr (DBA) {
        // t'_j over the lane's columns: sum of +-gamma_k x_k by the sign bits of B2 row j
        // (gamma_k x_k is exact in float32: 11 by 8 significant bits)
        float gx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          gx[e] = f16_bits_to_f32((dg[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) *
                  bf16_bits_to_f32((xv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
#pragma unroll
        for (int j = 0; j < kFuseR; ++j) {
          float sj = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sj += ((dbits[j] >> e) & 1u) ? gx[e] : -gx[e];
          v[j] = tkv && j < r ? sj : 0.0f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kFuseR; ++j) {
          float sj = 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q) sj = dot2(afr[j][q], xv[q], sj);
          v[j] = tkv ? sj : 0.0f;
        }
      }
      // exchange distances 32 and 16: swaps of lane halves (lanes without the
      // distance bit keep value i, the others value i + n/2, each summed with
      // its partner's)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]), false, false);
        v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]), false, false);
        v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      // lanes of row R (lane / 16) now hold j = 4R .. 4R + 3 summed over 4
      // lanes; the row sums complete them, and lane 16R writes the four
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = group_sum<16>(v[i]);
      if ((lane & 15) == 0)
        lds_wr128(P.sTP + 4u * (wave * kFuseR + (lane >> 2)),
                  u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
    }
  };

  uint32_t sBt = P.sB;  // LDS B rows of the tile being finished
  // Output (m, row nn = tile row l15) = s + scale * sum_j t[m][j] B[nn][j], stored
  // when ov (else out of range).
  auto epilogue = [&](int m, int l15, int64_t nn, bool ov, float s) {
    float lo = 0.0f;
    if constexpr (ADP) {
      const int mc = m < M ? m : M - 1;
      const int64_t nc = nn < N ? nn : N - 1;
      // (the fused product always has t and the B tile in LDS)
      const bool bpre = TF || P.bpre;
      const bool tlds = TF || P.tmode != T_GLOBAL;
      if (bpre) {
        const uint32_t brow = sBt + (uint32_t)(l15 * r * 2);
        if (tlds && (r & 7) == 0) {
          // 8 ranks per step from 16-byte LDS reads (t rows and B rows are
          // 16-byte aligned when r is a multiple of 8), same order of sums
          const uint32_t trow = P.sT + (uint32_t)(mc * r * 4);
#pragma unroll 2
          for (int j = 0; j < r; j += 8) {
            const u32x4_t t0 = lds_rd128(trow + 4u * j), t1 = lds_rd128(trow + 4u * j + 16u);
            const u32x4_t bb = lds_rd128(brow + 2u * j);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              lo = fmaf(__uint_as_float(q < 2 ? t0[2 * q] : t1[2 * q - 4]), bf16_bits_to_f32(bb[q] & 0xFFFFu), lo);
              lo = fmaf(__uint_as_float(q < 2 ? t0[2 * q + 1] : t1[2 * q - 3]), bf16_bits_to_f32(bb[q] >> 16), lo);
            }
          }
        } else if (tlds) {
          const float* tr = sT + mc * r;
          for (int j = 0; j < r; ++j) lo = fmaf(tr[j], bf16_bits_to_f32(lds_rd16(brow + 2 * j)), lo);
        } else {
          for (int j = 0; j < r; ++j) {
            float tj = 0.0f;
            for (int sp = 0; sp < a.t_splits; ++sp) tj += a.t[((int64_t)sp * M + mc) * r + j];
            lo = fmaf(tj, bf16_bits_to_f32(lds_rd16(brow + 2 * j)), lo);
          }
        }
      } else {
        const uint16_t* br = reinterpret_cast<const uint16_t*>(a.B) + nc * r;
        if (tlds) {
          const float* tr = sT + mc * r;
          for (int j = 0; j < r; ++j) lo = fmaf(tr[j], bf16_bits_to_f32(br[j]), lo);
        } else {
          for (int j = 0; j < r; ++j) {
            float tj = 0.0f;
            for (int sp = 0; sp < a.t_splits; ++sp) tj += a.t[((int64_t)sp * M + mc) * r + j];
            lo = fmaf(tj, bf16_bits_to_f32(br[j]), lo);
          }
        }
      }
    }
    float out = fmaf(a.scale, lo, s);
    if (a.addend && ov) out += a.addend[(int64_t)m * N + nn];
    const uint32_t yo = buf_off(ov, (uint32_t)(((int64_t)m * N + nn) * ES));
    if constexpr (YDT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), yr, yo, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(out), yr, yo, 0, 0);
  };

  // Reduce the K slices of a finished tile and write its outputs.  All 512
  // threads run the epilogue (threads past the outputs repeat one and store
  // out of range), so the stores are issued on every path.
  // row o's side-channel term (SPX = 2: times 1 / P, exact)
  auto sp_sum = [&](int o) {
    float t = sRed[256 + o];
    if constexpr (SPX == 2) t *= 1.0f / (float)(1 << a.sp_wht_lp);
    return t;
  };
  auto finish_tile = [&](int64_t tl) {
    if constexpr (DOT) {
#pragma unroll
      for (int i = 0; i < G::NP; ++i) {
        const float v = group_sum<G::PR>(accd[i]);
        if (lane % G::PR == 0) sRed[wave * 16 + (i * 64 + lane) / G::PR] = v;
        accd[i] = 0.0f;
      }
      if constexpr (SPX != 0) {
        // side-channel sum of tile row o = tid >> 5: lane i adds its entries
        // i + 32 e in e order (then i + 256 + 32 k), the 32 lanes are summed by
        // a fixed butterfly, and lane 0 writes sRed slot 256 + o
        if (tl != blockIdx.x) {
          sp_rows(tl);
          sp_entries();
        }
        auto src = [&](int32_t c) {
          if constexpr (SPX == 1) return bf16_bits_to_f32(lds_rd16(P.sX + (uint32_t)c * 2u));
          else return __uint_as_float(lds_rd32(P.sW + (uint32_t)c * 4u));
        };
        const int64_t li = tid & 31;
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < kSpE; ++e)
          if (sp0 + li + 32 * e < sp1) sum = fmaf(spv[e], src(spc[e]), sum);
        for (int64_t j = sp0 + li + 32 * kSpE; j < sp1; j += 32)
          sum = fmaf(a.sp_val[j], src(min<int32_t>(max<int32_t>(a.sp_col[j], 0), (int32_t)(K - 1))), sum);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) sum += __shfl_xor(sum, o, 64);
        if (li == 0) sRed[256 + (tid >> 5)] = sum;
      }
      __syncthreads();
      if constexpr (TF) {
        // thread (o, j) = (tid / 16 % 16, tid % 16): t_j (the waves' sums, in
        // wave order) times B[row o][j], summed over the 16 j lanes; lane j = 0
        // adds the row sum and stores output o (threads 256.. repeat, out of range)
        const int o = (tid >> 4) & 15, j = tid & 15;
        float tj = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          tj += *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)(P.sTP + 4u * (w * kFuseR + j)));
        float bj;
        if constexpr (DBA) {
          // alpha_n beta_j times the sign of B1[n][j] (R <= 16: one word per row)
          const int64_t n = min(tl * 16 + o, N - 1);
          const uint32_t w1 = a.dba_b1[n];
          const float ab = f16_bits_to_f32(a.dba_alpha[n]) * f16_bits_to_f32(a.dba_beta[j < r ? j : 0]);
          bj = j < r ? (((w1 >> j) & 1u) ? ab : -ab) : 0.0f;
        } else {
          bj = j < r ? bf16_bits_to_f32(lds_rd16(sBt + (uint32_t)((o * r + j) * 2))) : 0.0f;
        }
        const float lo = group_sum<16>(tj * bj);
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sRed[w * 16 + o];
        const int64_t nn = tl * 16 + o;
        float out = fmaf(a.scale, lo, s);
        if constexpr (SPX != 0) out += sp_sum(o);
        if (a.addend && tid < 256 && j == 0 && nn < N) out += a.addend[nn];
        const uint32_t yo = buf_off(tid < 256 && j == 0 && nn < N, (uint32_t)(nn * ES));
        if constexpr (YDT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), yr, yo, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(out), yr, yo, 0, 0);
      } else if (ADP && P.bpre && P.tmode != T_GLOBAL) {
        // output o = tid / 32 by a half-wave: lane q sums t_j B[o][j] over
        // j = q, q + 32, ..., the 32 lanes are added by a fixed butterfly, and
        // lane 0 adds the row sum and stores
        const int o = tid >> 5, q = tid & 31;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sRed[w * 16 + o];
        if constexpr (SPX != 0) s += sp_sum(o);
        float lo = 0.0f;
        for (int j = q; j < r; j += 32)
          lo = fmaf(sT[j], bf16_bits_to_f32(lds_rd16(sBt + (uint32_t)((o * r + j) * 2))), lo);
#pragma unroll
        for (int d = 1; d < 32; d <<= 1) lo += __shfl_xor(lo, d, 64);
        const int64_t nn = tl * 16 + o;
        const bool ov = q == 0 && nn < N;
        float out = fmaf(a.scale, lo, s);
        if (a.addend && ov) out += a.addend[nn];
        const uint32_t yo = buf_off(ov, (uint32_t)(nn * ES));
        if constexpr (YDT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), yr, yo, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(out), yr, yo, 0, 0);
      } else {
        const int o = tid & 15;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sRed[w * 16 + o];
        const int64_t nn = tl * 16 + o;
        if constexpr (SPX != 0) s += sp_sum(o);
        epilogue(0, o, nn, tid < 16 && nn < N, s);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) sRed[wave * 256 + lane * 4 + v] = acc[v];
      acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      if (ADP && P.bpre && P.tmode != T_GLOBAL && (r & 7) == 0) {
        // output o = tid / 2 by two neighbouring lanes, each summing every other
        // group of 8 ranks (16-byte LDS reads of t and B), added by one exchange
        const int o = tid >> 1, hh = tid & 1;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sRed[w * 256 + o];
        const int l = o >> 2, v = o & 3;
        const int m = 4 * (l >> 4) + v;  // MFMA output row (x row)
        const int l15 = l & 15;
        const int64_t nn = tl * 16 + l15;
        const int mc = m < M ? m : M - 1;
        const uint32_t trow = P.sT + (uint32_t)(mc * r * 4), brow = sBt + (uint32_t)(l15 * r * 2);
        float lo = 0.0f;
        for (int j = 8 * hh; j < r; j += 16) {
          const u32x4_t t0 = lds_rd128(trow + 4u * j), t1 = lds_rd128(trow + 4u * j + 16u);
          const u32x4_t bb = lds_rd128(brow + 2u * j);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lo = fmaf(__uint_as_float(q < 2 ? t0[2 * q] : t1[2 * q - 4]), bf16_bits_to_f32(bb[q] & 0xFFFFu), lo);
            lo = fmaf(__uint_as_float(q < 2 ? t0[2 * q + 1] : t1[2 * q - 3]), bf16_bits_to_f32(bb[q] >> 16), lo);
          }
        }
        lo += __shfl_xor(lo, 1, 64);
        const bool ov = hh == 0 && m < M && nn < N;
        float out = fmaf(a.scale, lo, s);
        if (a.addend && ov) out += a.addend[(int64_t)m * N + nn];
        const uint32_t yo = buf_off(ov, (uint32_t)(((int64_t)m * N + nn) * ES));
        if constexpr (YDT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), yr, yo, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(out), yr, yo, 0, 0);
      } else {
        const int o = tid & 255;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sRed[w * 256 + o];
        const int l = o >> 2, v = o & 3;
        const int m = 4 * (l >> 4) + v;  // MFMA output row (x row)
        const int64_t nn = tl * 16 + (l & 15);
        epilogue(m, l & 15, nn, tid < 256 && m < M && nn < N, s);
      }
    }
    sBt += (uint32_t)(32 * r);  // the next tile's B rows
    // the next tile reuses sRed; after the workgroup's last tile nothing is reused
    if (tl + gridDim.x < P.ntiles) __syncthreads();
  };

  // The stream: chunk j is item j % nitem of tile blockIdx.x + (j / nitem) gridDim.x;
  // slot j % D of the ring is computed and then refilled with chunk j + D.
  const int64_t T = (P.ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const int64_t total = T * nitem;
  int64_t ctile = blockIdx.x;
  int cc = 0, buf = 0;
  // compute slot s (chunk j = j0 + s) and finish its tile at the tile's last chunk
  auto consume = [&](int s, int64_t j) {
    if (j < total) {
      if (nchunk > 0) {
        if constexpr (DOT) compute_dot(ring[s], ctile, cc, buf);
        else compute(ring[s], ctile, cc, buf, s);
      }
      buf ^= 1;
      if (cc == nitem - 1) {
        if constexpr (TF) {
          if (ctile == blockIdx.x) compute_t();
        }
        finish_tile(ctile);
        cc = 0;
        ctile += gridDim.x;
      } else {
        ++cc;
      }
    }
  };
  if constexpr (XR) {
    // the x fragments into the MFMA layout, once (their loads were issued
    // before the ring's, so the first chunk's wait covers them)
#pragma unroll
    for (int u = 0; u < 2 * CH; ++u) {
      u32x4_t f0, f1;
      x_frag(xr[u][0], xr[u][1], lane, f0, f1);
      xr[u][0] = f0;
      xr[u][1] = f1;
    }
  }
  if constexpr (TF) {
    // the whole stream is in the ring (at most D chunks): straight-line, no refills
#pragma unroll
    for (int s = 0; s < D; ++s) consume(s, s);
  } else {
    for (int64_t j0 = 0; j0 < total; j0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        consume(s, j0 + s);
        load_chunk(ring[s]);
      }
    }
  }
}

// Geometry of the grouped single-row kernel: 16-byte pieces of whole codes, and
// for 3-bit codes 12-byte pieces (32 codes; a 24-byte block is two of them,
// 4-byte aligned), 8 lanes per 96-byte chunk row.
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
template <int BITS>
struct DotGeo {
  static constexpr int kRowBytes = CH * 8 * BITS;
  static constexpr int PB = (BITS == 3) ? 12 : 16;
  static constexpr int PR = kRowBytes / PB;       // pieces per chunk row
  static constexpr int NP = (16 * PR + 63) / 64;  // pieces per lane
  static constexpr int CP = PB * 8 / BITS;        // codes per piece
  typedef typename std::conditional<BITS == 3, u32x3_t, u32x4_t>::type Piece;
};
template <int BITS>
struct DChunk {
  typename DotGeo<BITS>::Piece piece[DotGeo<BITS>::NP];
  uint32_t q8;
  float sc;
  u32x4_t bp;
};

// dot_piece for a 12-byte piece of 32 3-bit codes: pair p (codes 2p, 2p + 1)
// is the 6-bit field at bits [6p, 6p + 6), an index of the 64-entry table; the
// fields of pairs 5 and 10 straddle a word boundary (funnel shift).
template <bool H>
__device__ __forceinline__ float dot_piece3(const u32x3_t& pc, const u32x4_t* xv, uint32_t tl) {
  PairAcc<H> acc;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int bit = 6 * p, w = bit >> 5, sh = bit & 31;
    uint32_t e;
    if (sh <= 26) e = (pc[w] >> sh) & 63u;
    else e = __builtin_amdgcn_alignbit(pc[w + 1], pc[w], (uint32_t)sh) & 63u;
    acc.add(lds_word((e << 8) | tl), xv[p >> 2][p & 3], p & 1);
  }
  return acc.sum();
}

// ---------------------------------------------------------------- grouped single-row decode
//
// Up to kGvGroupMax independent linears of one code width at M = 1 in one
// launch (a mixed stack's decode; AutoQRA page, section 3.1: each layer has its
// own bits and rank).  The work units are the layers' 16-row tiles, each costing
// its layer's blocks per row; workgroup b takes the contiguous run of units
// whose start cost lies in [b C / G, (b + 1) C / G) (C the group's total), so
// the workgroups stream about the same number of bytes and each crosses only a
// few layer boundaries.  Within a layer it is the single-row path of k_gemv:
// when a workgroup enters a layer it issues that layer's first chunks, then
// stages the x row (and the adapter product, summed over its splits) in LDS;
// the 8 waves split K, each keeps a ring of D chunks in flight (never past its
// run: loads beyond it read nothing), and every tile ends with the cross-wave
// reduction and the epilogue (adapter term spread over the threads).
constexpr int kGvGroupMax = 16;
struct GvLayer {
  const uint16_t* x;     // 1 x K bf16
  const uint8_t* codes;
  const uint8_t* q8;
  const float* cst;
  const float* t;        // t_splits x r float32 partial sums of x A^T (r > 0)
  const uint16_t* B;     // N x r bf16
  void* y;               // 1 x N
  int32_t N, nb, r, t_splits;
  float scale;
  int32_t ntiles;
  int64_t cost0;         // units before this layer: sum of ntiles x nb
};
struct GvParams {
  int32_t nl;
  int64_t total;
  uint32_t sT, sTP, sB, sX;  // LDS byte addresses: summed t, its partials, the tile's B rows, the x row
  uint32_t sXh, sXs;         // the x row as fp16 numbers x 2^s_b, and the block exponents s_b
  GvLayer L[kGvGroupMax];
};

template <int BITS, int YDT, bool ADP, int D>
__global__ __launch_bounds__(kThreads, 1) void k_gemv_group(GvParams P, Levels lv) {
  using G = DotGeo<BITS>;
  using Ch = DChunk<BITS>;
  constexpr uint32_t kStageW = 16 * CH * 4;
  constexpr int ES = (YDT == DT_F32) ? 4 : 2;
  constexpr int CP = G::CP;      // codes per piece
  constexpr int PPB = 64 / CP;   // pieces per block
  extern __shared__ uint32_t smem[];
  const int tid = threadIdx.x;
  // (the wave index is uniform within a wave: saying so keeps the chunk loops scalar)
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t tlane = table_lane_h(lane);
  const uint32_t stage0 = (uint32_t)LevelTableH<BITS>::kBytes;
  float* sRed = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + stage0 + kWaves * 2 * kStageW);
  const float* sT = reinterpret_cast<const float*>(reinterpret_cast<const char*>(smem) + P.sT);
  const uint32_t wstage = stage0 + (uint32_t)wave * 2 * kStageW;
  const int srow = lane >> 2, sblk = lane & 3;
  build_table_h<BITS>(smem, lv, tid);  // complete at the first segment's barrier
  const int64_t c_begin = P.total * blockIdx.x / gridDim.x, c_end = P.total * (blockIdx.x + 1) / gridDim.x;
  for (int l = 0; l < P.nl; ++l) {
    const GvLayer& L = P.L[l];
    const int64_t nb = L.nb, lo = c_begin - L.cost0, hi = c_end - L.cost0;
    if (hi <= 0 || lo >= (int64_t)L.ntiles * nb) continue;
    // the units u of this layer whose start cost u nb lies in [lo, hi)
    const int32_t t0 = (int32_t)(lo <= 0 ? 0 : (lo + nb - 1) / nb);
    const int32_t t1 = (int32_t)min<int64_t>(L.ntiles, (hi + nb - 1) / nb);
    if (t0 >= t1) continue;
    const int64_t N = L.N, K = nb * 64;
    const int r = ADP ? L.r : 0;
    const int64_t kb0 = nb * wave / kWaves, kb1 = nb * (wave + 1) / kWaves;
    const int nchunk = (int)((kb1 - kb0 + CH - 1) / CH);
    const int nitem = nchunk > 0 ? nchunk : 1;
    const int64_t total = (int64_t)(t1 - t0) * nitem;
    const __amdgpu_buffer_rsrc_t cr = rsrc(L.codes, N * nb * 8 * BITS);
    const __amdgpu_buffer_rsrc_t qr = rsrc(L.q8, N * nb);
    const __amdgpu_buffer_rsrc_t sr = rsrc(L.cst, ((N * nb + 255) >> 8) * 4);
    const __amdgpu_buffer_rsrc_t brs = rsrc(L.B, ADP ? N * r * 2 : 0);
    const __amdgpu_buffer_rsrc_t yr = rsrc(L.y, N * ES);
    const uint32_t nb32 = (uint32_t)nb, kb032 = (uint32_t)kb0;
    const uint32_t rowb = nb32 * (8u * BITS);
    uint32_t coff0[G::NP];
#pragma unroll
    for (int i = 0; i < G::NP; ++i) {
      const int p = i * 64 + lane;
      coff0[i] = ((uint32_t)t0 * 16u + (uint32_t)(p / G::PR)) * rowb + kb032 * (8u * BITS) +
                 (uint32_t)((p % G::PR) * G::PB);
    }
    const uint32_t qoff0 = ((uint32_t)t0 * 16u + (uint32_t)srow) * nb32 + kb032 + (uint32_t)sblk;
    int32_t ltile = t0;
    int lc = 0;
    uint32_t lct = 0, lqt = 0;
    // chunk lc of tile ltile (nothing read once the cursor is past the run)
    auto load_chunk = [&](Ch& ch) __attribute__((always_inline)) {
      const bool in = ltile < t1;
      const uint32_t cb = (uint32_t)lc * (uint32_t)CH;
#pragma unroll
      for (int i = 0; i < G::NP; ++i) {
        const uint32_t off = buf_off(in, coff0[i] + lct + cb * (8u * BITS));
        if constexpr (BITS == 3) ch.piece[i] = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(cr, off, 0, 0));
        else ch.piece[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cr, off, 0, 0));
      }
      const uint32_t blk = qoff0 + lqt + cb;
      ch.q8 = __builtin_amdgcn_raw_buffer_load_b8(qr, buf_off(in, blk), 0, 0);
      ch.sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, buf_off(in, (blk >> 8) << 2), 0, 0));
      if constexpr (ADP) {
        const int pc = wave * 64 + lane;
        const bool bv = in && lc == nitem - 1 && pc < 2 * r;
        ch.bp = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                brs, buf_off(bv, (uint32_t)ltile * (uint32_t)(32 * r) + (uint32_t)pc * 16u),
                                                0, 0));
      }
      if (++lc == nitem) {
        lc = 0;
        ++ltile;
        lct += 16u * rowb;
        lqt += 16u * nb32;
      }
    };
    // the previous segment's tiles are done with x, t and B in LDS (and, the first time, the table is written)
    __syncthreads();
    Ch ring[D];
#pragma unroll
    for (int q = 0; q < D; ++q) load_chunk(ring[q]);
    {
      // the x row (K <= 16384: at most 4 pieces per thread) and the adapter partials (at most 8 per
      // thread), every load issued before any is used
      constexpr int kXP = (int)(kXLdsMax / 16 / kThreads), kTP = kTPartsMax / kThreads;
      const uint16_t* xg = L.x;
      const int64_t xpieces = K / 8;
      u32x4_t xs[kXP];
#pragma unroll
      for (int i = 0; i < kXP; ++i) {
        const int64_t q = tid + (int64_t)i * kThreads;
        if (i * kThreads < xpieces) xs[i] = *reinterpret_cast<const u32x4_t*>(xg + (q < xpieces ? q : 0) * 8);
      }
      float tpv[kTP];
      const int tc = ADP ? L.t_splits * r : 0;
      if constexpr (ADP) {
#pragma unroll
        for (int i = 0; i < kTP; ++i) {
          const int q = tid + i * kThreads;
          tpv[i] = q < tc ? L.t[q] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < kXP; ++i) {
        const int64_t q = tid + (int64_t)i * kThreads;
        if (i * kThreads < xpieces) {
          u32x4_t xh;
          const int sb = x_piece_f16(q < xpieces ? xs[i] : u32x4_t{0u, 0u, 0u, 0u}, xh);
          if (q < xpieces) {
            lds_wr128(P.sX + (uint32_t)q * 16u, xs[i]);
            lds_wr128(P.sXh + (uint32_t)q * 16u, xh);
            if ((q & 7) == 0) *reinterpret_cast<__attribute__((address_space(3))) int*>((uintptr_t)(P.sXs + (uint32_t)(q >> 3) * 4u)) = sb;
          }
        }
      }
      if constexpr (ADP) {
        float* sTPw = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + P.sTP);
#pragma unroll
        for (int i = 0; i < kTP; ++i) {
          const int q = tid + i * kThreads;
          if (q < tc) sTPw[q] = tpv[i];
        }
      }
    }
    __syncthreads();
    if constexpr (ADP) {
      // t_j = its partials summed in split order (read by the first tile's epilogue, after a barrier)
      float* sTw = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + P.sT);
      const float* sTPr = reinterpret_cast<const float*>(reinterpret_cast<const char*>(smem) + P.sTP);
      for (int j = tid; j < r; j += kThreads) {
        float acc = 0.0f;
        for (int q = 0; q < L.t_splits; ++q) acc += sTPr[q * r + j];
        sTw[j] = acc;
      }
    }
    // the wave multiplies the fp16 x row when all its blocks are exact (hx), else the bf16 row
    const bool hx = x_blocks_exact(P.sXs, kb0, kb1, lane);
    float accd[G::NP];
#pragma unroll
    for (int i = 0; i < G::NP; ++i) accd[i] = 0.0f;
    auto compute_dot = [&](const Ch& ch, int32_t tl, int c, int buf) __attribute__((always_inline)) {
      const uint32_t sscale = wstage + (uint32_t)buf * kStageW;
      {
        const bool nvalid = (int64_t)tl * 16 + srow < N;
        const float ap = nvalid ? (float)ch.q8 * ch.sc : 0.0f;
        *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)(sscale + (uint32_t)(srow * CH + sblk) * 4)) = ap;
      }
      const int64_t kbs = kb0 + (int64_t)c * CH;
      const int col = lane % G::PR;
      const int u = col / PPB;
      const bool bval = kbs + u < kb1;  // blocks past the wave's range are read but not added
      const uint32_t xa = (hx ? P.sXh : P.sX) + (uint32_t)((kbs * 64 + col * CP) * 2);
      u32x4_t xv[CP / 8];
#pragma unroll
      for (int q = 0; q < CP / 8; ++q) xv[q] = lds_rd128(xa + 16u * q);
      // the pieces' block scales and the lane's block exponent (blocks past the row read the
      // array's padding, never added), read before the products so their latency is hidden
      float ap[G::NP];
#pragma unroll
      for (int i = 0; i < G::NP; ++i)
        ap[i] = __uint_as_float(lds_rd32(sscale + (uint32_t)(((i * 64 + lane) / G::PR) * CH + u) * 4));
      const int sb = (int)lds_rd32(P.sXs + (uint32_t)(kbs + u) * 4u);
      float sp[G::NP];
      if (hx) {
#pragma unroll
        for (int i = 0; i < G::NP; ++i) {
          float v;
          if constexpr (BITS == 3) v = dot_piece3<true>(ch.piece[i], xv, tlane);
          else v = dot_piece<BITS, true>(ch.piece[i], xv, tlane);
          sp[i] = ldexpf(v, -sb);
        }
      } else {
#pragma unroll
        for (int i = 0; i < G::NP; ++i) {
          if constexpr (BITS == 3) sp[i] = dot_piece3<false>(ch.piece[i], xv, tlane);
          else sp[i] = dot_piece<BITS, false>(ch.piece[i], xv, tlane);
        }
      }
#pragma unroll
      for (int i = 0; i < G::NP; ++i) accd[i] = fmaf(ap[i], bval ? sp[i] : 0.0f, accd[i]);
    };
    auto finish_tile = [&](int32_t tl) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < G::NP; ++i) {
        const float v = group_sum<G::PR>(accd[i]);
        if (lane % G::PR == 0) sRed[wave * 16 + (i * 64 + lane) / G::PR] = v;
        accd[i] = 0.0f;
      }
      __syncthreads();
      // output o = tid / 32 by a half-wave (adapter ranks q, q + 32, ... per lane, then a butterfly)
      const int o = tid >> 5, q = tid & 31;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += sRed[w * 16 + o];
      float lo2 = 0.0f;
      if constexpr (ADP) {
        for (int j = q; j < r; j += 32)
          lo2 = fmaf(sT[j], bf16_bits_to_f32(lds_rd16(P.sB + (uint32_t)((o * r + j) * 2))), lo2);
#pragma unroll
        for (int d = 1; d < 32; d <<= 1) lo2 += __shfl_xor(lo2, d, 64);
      }
      const int64_t nn = (int64_t)tl * 16 + o;
      const float out = fmaf(L.scale, lo2, sum);
      const uint32_t yo = buf_off(q == 0 && nn < N, (uint32_t)nn * (uint32_t)ES);
      if constexpr (YDT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), yr, yo, 0, 0);
      else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(out), yr, yo, 0, 0);
      __syncthreads();  // sRed and the B tile are reused by the next tile
    };
    int32_t ctile = t0;
    int cc = 0, buf = 0;
    // (the counters advance by value selects: a store to a selected counter would keep both in memory)
    auto consume = [&](int q, int64_t j) __attribute__((always_inline)) {
      if (j < total) {
        if (nchunk > 0) compute_dot(ring[q], ctile, cc, buf);
        buf ^= 1;
        const bool last = cc == nitem - 1;
        if (last) {
          if constexpr (ADP) {
            const int pc = wave * 64 + lane;
            if (pc < 2 * r) lds_wr128(P.sB + (uint32_t)pc * 16u, ring[q].bp);
          }
          finish_tile(ctile);
        }
        cc = last ? 0 : cc + 1;
        ctile += last ? 1 : 0;
      }
    };
    for (int64_t j0 = 0; j0 < total; j0 += D) {
#pragma unroll
      for (int q = 0; q < D; ++q) {
        consume(q, j0 + q);
        load_chunk(ring[q]);
      }
    }
  }
}

constexpr size_t kLdsMax = 160 * 1024;

int device_cus() {
  static int cus = 0;  // one device per process
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cus = std::max(n, 1);
    else
      return 1;
  }
  return cus;
}

template <int BITS, int YDT, bool XLDS, bool ADP, int D, bool DOT = false, bool TF = false, int SPX = 0,
          bool DBA = false, bool XR = false>
hipError_t launch_k(const Params& P, int64_t grid, size_t shmem, const Levels& lv, hipStream_t s) {
  auto kern = k_gemv<BITS, YDT, XLDS, ADP, D, DOT, TF, SPX, DBA, XR>;
  static bool attr = false;
  if (!attr) {
    // the kernel addresses LDS from 0: it must not have static LDS
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsMax);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), shmem, s, P, lv);
  return hipGetLastError();
}

// Launch plan of one call: parameters, grid, dynamic LDS and the variant.
struct Plan {
  Params P;
  int64_t grid = 0;
  size_t lds = 0;
  bool ok = false;    // 32-bit buffer addressing holds
  bool xlds = false;  // x staged in LDS
  bool deep = false;  // a wave's chunk stream is longer than 2 (ring depth 4)
  bool dot = false;   // single-row path
  bool tf = false;    // fused adapter product
  bool xr = false;    // MFMA path: each wave's x fragments in registers (two chunks per wave and tile)
  bool spw = false;   // room for the transform of the x row (Walsh-Hadamard side channel)
};

template <int BITS>
Plan plan_gemv(const LinearArgs& a) {
  Plan pl;
  Params& P = pl.P;
  P.a = a;
  P.ntiles = (a.N + 15) / 16;
  const int64_t r = a.r > 0 ? a.r : 0;
  const int64_t ES = (a.ydt == DT_F32) ? 4 : 2;
  // codes, absmax codes, y, A and B rows are addressed with 32-bit buffer offsets
  const int64_t lim = int64_t(1) << 31;
  if (a.N * (a.K / 64) * 8 * a.bits >= lim || a.M * a.N * ES >= lim || a.N * r * 2 >= lim || r * a.K * 2 >= lim)
    return pl;
  pl.ok = true;
  pl.grid = std::min<int64_t>(P.ntiles, device_cus());
  // longest chunk stream of a wave: tiles per workgroup x chunks per tile
  const int64_t nb = a.K / 64;
  const int64_t stream = ((P.ntiles + pl.grid - 1) / pl.grid) * std::max<int64_t>(1, ((nb + kWaves - 1) / kWaves + CH - 1) / CH);
  pl.deep = stream > 2;
  auto r16 = [](size_t b) { return (b + 15) & ~(size_t)15; };
  for (int attempt = 0; attempt < 2; ++attempt) {
    const bool dot = attempt == 0 && BITS != 3 && a.M == 1 && (size_t)a.K * 2 <= kXLdsMax;
    const bool dbaf = a.dba_b2 != nullptr;  // the double-binary branch through the fused product
    const bool tf = dot && r > 0 && r <= kFuseR && nb <= 8 * kWaves && !pl.deep &&
                    (dbaf || (a.A != nullptr && (reinterpret_cast<uintptr_t>(a.A) & 15) == 0));
    const size_t stage = dot ? 16 * CH * 4 : ChunkGeo<BITS>::kStage;
    size_t lds = PairTable<BITS>::kBytes + (size_t)kWaves * 2 * stage + (size_t)kWaves * 256 * sizeof(float);
    // single-row path: the x row as fp16 numbers (read up to 256 elements past its end, like the bf16
    // row) and its block exponents (read up to CH blocks past the row)
    P.sXh = P.sXs = 0;
    if (dot) {
      P.sXh = (uint32_t)lds;
      lds += (size_t)(a.K + 8) * 2 + 512;
      P.sXs = (uint32_t)lds;
      lds += r16((size_t)(nb + 8) * 4);
    }
    // adapter product: fused, partials prefetched when they fit the registers, else summed by a loop
    const size_t mr = (size_t)a.M * (size_t)r;
    const size_t tparts = (size_t)a.t_splits * mr;
    P.tmode = T_GLOBAL;
    P.sT = P.sTP = P.sB = P.sX = P.sZ = 0;
    P.bpre = 0;
    if (r > 0) {
      P.sT = (uint32_t)lds;
      if (tf) {
        P.tmode = T_FUSED;
        lds += r16(mr * 4);
        P.sTP = (uint32_t)lds;
        lds += (size_t)kWaves * kFuseR * 4;
      } else if (tparts <= (size_t)kTPre * kThreads && lds + r16(mr * 4) + r16(tparts * 4) <= kLdsMax) {
        P.tmode = T_PREFETCH;
        lds += r16(mr * 4);
        P.sTP = (uint32_t)lds;
        lds += r16(tparts * 4);
      } else if (lds + r16(mr * 4) <= kLdsMax) {
        P.tmode = T_LOOP;
        lds += r16(mr * 4);
      }
      // the B rows of every tile of a workgroup (2 r 16-byte pieces per tile, at most
      // kBPre per thread), from a 16-byte aligned B
      const int64_t tpw = (P.ntiles + pl.grid - 1) / pl.grid;
      if (tpw * 2 * r <= (int64_t)kBPre * kThreads && (reinterpret_cast<uintptr_t>(a.B) & 15) == 0 &&
          lds + r16((size_t)(32 * r * tpw)) <= kLdsMax) {
        P.bpre = 1;
        P.sB = (uint32_t)lds;
        lds += r16((size_t)(32 * r * tpw));
      }
    }
    // x staged in LDS (rows at stride K + 8 bf16) when small enough (+512 bytes:
    // the single-row path reads up to 256 elements past a row's end, for
    // blocks it does not add), after a 128-byte zero strip
    const size_t xbytes = (size_t)a.M * (size_t)(a.K + 8) * 2 + 512;
    const bool xlds = (size_t)a.M * (size_t)a.K * 2 <= kXLdsMax && lds + 128 + xbytes <= kLdsMax;
    if (dot && !xlds) continue;  // the single-row path needs x in LDS
    if (tf && (P.tmode != T_FUSED || (!P.bpre && !dbaf))) continue;
    P.sZ = (uint32_t)lds;
    lds += 128;
    P.sX = (uint32_t)lds;
    pl.xlds = xlds;
    pl.dot = dot;
    // every wave's K range is 5..8 blocks (two chunks): 40 <= nb <= 64
    pl.xr = !xlds && !dot && nb >= 5 * kWaves && nb <= 2 * CH * kWaves;
    pl.tf = tf && P.tmode == T_FUSED;
    pl.lds = lds + (xlds ? xbytes : 0);
    if (a.sp_row_ptr && a.sp_wht_lp >= 0 && dot) {
      P.sW = (uint32_t)r16(pl.lds);
      pl.spw = P.sW + (size_t)a.K * 4 <= kLdsMax;
      if (pl.spw) pl.lds = P.sW + (size_t)a.K * 4;
    }
    return pl;
  }
  pl.ok = false;
  return pl;
}

template <int BITS, int YDT>
hipError_t launch_gemv_b(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  const Plan pl = plan_gemv<BITS>(a);
  if (!pl.ok) return hipErrorInvalidValue;
  const Params& P = pl.P;
  const int64_t grid = pl.grid;
  const size_t lds = pl.lds;
  const bool adp = a.r > 0;
  if (a.dba_b2) {
    if constexpr (BITS != 3) {
      if (pl.tf) return launch_k<BITS, YDT, true, true, 2, true, true, 0, true>(P, grid, lds, lv, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.sp_row_ptr) {
    // the side channel is summed in the kernel only on the single-row path with a short stream
    if constexpr (BITS != 3) {
      if (pl.dot && !pl.deep && a.sp_nnz > 0) {
        if (a.sp_wht_lp >= 0) {
          if (!pl.spw || adp) return hipErrorInvalidValue;
          return launch_k<BITS, YDT, true, false, 2, true, false, 2>(P, grid, lds, lv, s);
        }
        if (pl.tf) return launch_k<BITS, YDT, true, true, 2, true, true, 1>(P, grid, lds, lv, s);
        if (adp) return launch_k<BITS, YDT, true, true, 2, true, false, 1>(P, grid, lds, lv, s);
        return launch_k<BITS, YDT, true, false, 2, true, false, 1>(P, grid, lds, lv, s);
      }
    }
    return hipErrorInvalidValue;
  }
  if constexpr (BITS != 3) {
    if (pl.dot) {
      if (pl.tf) return launch_k<BITS, YDT, true, true, 2, true, true>(P, grid, lds, lv, s);
      if (adp) {
        if (pl.deep) return launch_k<BITS, YDT, true, true, 4, true>(P, grid, lds, lv, s);
        return launch_k<BITS, YDT, true, true, 2, true>(P, grid, lds, lv, s);
      }
      if (pl.deep) return launch_k<BITS, YDT, true, false, 4, true>(P, grid, lds, lv, s);
      return launch_k<BITS, YDT, true, false, 2, true>(P, grid, lds, lv, s);
    }
  }
  if (adp) {
    if (pl.xlds) {
      if (pl.deep) return launch_k<BITS, YDT, true, true, 4>(P, grid, lds, lv, s);
      return launch_k<BITS, YDT, true, true, 2>(P, grid, lds, lv, s);
    }
    if (pl.xr) {
      if (pl.deep) return launch_k<BITS, YDT, false, true, 4, false, false, 0, false, true>(P, grid, lds, lv, s);
      return launch_k<BITS, YDT, false, true, 2, false, false, 0, false, true>(P, grid, lds, lv, s);
    }
    return launch_k<BITS, YDT, false, true, 2>(P, grid, lds, lv, s);
  }
  if (pl.xlds) {
    if (pl.deep) return launch_k<BITS, YDT, true, false, 4>(P, grid, lds, lv, s);
    return launch_k<BITS, YDT, true, false, 2>(P, grid, lds, lv, s);
  }
  if (pl.xr) {
    if (pl.deep) return launch_k<BITS, YDT, false, false, 4, false, false, 0, false, true>(P, grid, lds, lv, s);
    return launch_k<BITS, YDT, false, false, 2, false, false, 0, false, true>(P, grid, lds, lv, s);
  }
  return launch_k<BITS, YDT, false, false, 2>(P, grid, lds, lv, s);
}

template <int BITS>
hipError_t launch_gemv_y(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.ydt == DT_F32) return launch_gemv_b<BITS, DT_F32>(a, lv, s);
  return launch_gemv_b<BITS, DT_BF16>(a, lv, s);
}

}  // namespace

bool gemv_fuses_adapter(const LinearArgs& a) {
  if (a.r <= 0 || a.M <= 0) return false;
  switch (a.bits) {
    case 2: return plan_gemv<2>(a).tf;
    case 3: return plan_gemv<3>(a).tf;
    case 4: return plan_gemv<4>(a).tf;
    default: return plan_gemv<8>(a).tf;
  }
}

bool gemv_fuses_dba(const LinearArgs& a) {
  if (a.M != 1 || a.bits == 3 || !a.dba_b2 || a.r <= 0 || a.r > kFuseR) return false;
  Plan pl;
  switch (a.bits) {
    case 2: pl = plan_gemv<2>(a); break;
    case 4: pl = plan_gemv<4>(a); break;
    default: pl = plan_gemv<8>(a); break;
  }
  return pl.ok && pl.tf;
}

bool gemv_fuses_sparse(const LinearArgs& a) {
  if (a.M != 1 || a.bits == 3) return false;
  Plan pl;
  switch (a.bits) {
    case 2: pl = plan_gemv<2>(a); break;
    case 4: pl = plan_gemv<4>(a); break;
    default: pl = plan_gemv<8>(a); break;
  }
  return pl.ok && pl.dot && !pl.deep && (a.sp_wht_lp < 0 || (pl.spw && a.r <= 0));
}

namespace {

template <int BITS, int YDT, bool ADP, int D>
hipError_t launch_gv_group_k(const GvParams& P, int64_t grid, size_t shmem, const Levels& lv, hipStream_t s) {
  auto kern = k_gemv_group<BITS, YDT, ADP, D>;
  static bool attr = false;
  if (!attr) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsMax);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), shmem, s, P, lv);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_gv_group_b(const GvParams& P, int64_t grid, size_t shmem, bool adp, bool deep, int ydt,
                             const Levels& lv, hipStream_t s) {
  if (ydt == DT_F32) {
    if (adp) return deep ? launch_gv_group_k<BITS, DT_F32, true, 4>(P, grid, shmem, lv, s)
                         : launch_gv_group_k<BITS, DT_F32, true, 2>(P, grid, shmem, lv, s);
    return deep ? launch_gv_group_k<BITS, DT_F32, false, 4>(P, grid, shmem, lv, s)
                : launch_gv_group_k<BITS, DT_F32, false, 2>(P, grid, shmem, lv, s);
  }
  if (adp) return deep ? launch_gv_group_k<BITS, DT_BF16, true, 4>(P, grid, shmem, lv, s)
                       : launch_gv_group_k<BITS, DT_BF16, true, 2>(P, grid, shmem, lv, s);
  return deep ? launch_gv_group_k<BITS, DT_BF16, false, 4>(P, grid, shmem, lv, s)
              : launch_gv_group_k<BITS, DT_BF16, false, 2>(P, grid, shmem, lv, s);
}

}  // namespace

int gemv_group_max() { return kGvGroupMax; }

// Longest row of the grouped kernel: the bf16 and fp16 rows, the level table and
// the largest adapter staging (r = 256) then fill at most 152 KB of LDS.
constexpr int64_t kGvMaxK = 12288;

bool gemv_groupable(const LinearArgs& a) {
  const int64_t r = a.r > 0 ? a.r : 0;
  return a.M == 1 && a.xdt == DT_BF16 && a.K % 64 == 0 && a.K <= kGvMaxK &&
         r <= 256 && (r == 0 || (a.abdt == DT_BF16 && a.t != nullptr && (int64_t)a.t_splits * r <= kTPartsMax &&
                                 (reinterpret_cast<uintptr_t>(a.B) & 15) == 0)) &&
         a.N * (a.K / 64) * 8 * a.bits < (int64_t(1) << 31) && a.N * r * 2 < (int64_t(1) << 31) &&
         (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 && a.addend == nullptr && a.sp_row_ptr == nullptr &&
         a.dba_b2 == nullptr;
}

hipError_t launch_gemv_group(const LinearArgs* ls, int n, const Levels& lv, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n > kGvGroupMax) return hipErrorInvalidValue;
  GvParams P;
  P.nl = n;
  int64_t cost = 0, maxK = 0;
  int maxr = 0;
  bool adp = false;
  for (int i = 0; i < n; ++i) {
    const LinearArgs& a = ls[i];
    if (!gemv_groupable(a) || a.bits != ls[0].bits || a.ydt != ls[0].ydt) return hipErrorInvalidValue;
    GvLayer& L = P.L[i];
    L.x = reinterpret_cast<const uint16_t*>(a.x);
    L.codes = a.codes;
    L.q8 = a.q8;
    L.cst = a.cst;
    L.t = a.t;
    L.B = reinterpret_cast<const uint16_t*>(a.B);
    L.y = a.y;
    L.N = (int32_t)a.N;
    L.nb = (int32_t)(a.K / 64);
    L.r = a.r > 0 ? a.r : 0;
    L.t_splits = a.t_splits;
    L.scale = a.scale;
    L.ntiles = (int32_t)((a.N + 15) / 16);
    L.cost0 = cost;
    cost += (int64_t)L.ntiles * L.nb;
    maxK = std::max<int64_t>(maxK, a.K);
    maxr = std::max(maxr, L.r);
    adp = adp || L.r > 0;
  }
  P.total = cost;
  if (cost == 0) return hipSuccess;
  auto r16 = [](size_t b) { return (b + 15) & ~(size_t)15; };
  const int bits = ls[0].bits;
  size_t lds = bits == 2 ? PairTable<2>::kBytes : bits == 3 ? PairTable<3>::kBytes : bits == 4 ? PairTable<4>::kBytes
                                                                                           : PairTable<8>::kBytes;
  lds += (size_t)kWaves * 2 * (16 * CH * 4) + (size_t)kWaves * 256 * sizeof(float);
  P.sT = (uint32_t)lds;
  lds += r16((size_t)maxr * 4);
  P.sTP = (uint32_t)lds;
  if (adp) lds += (size_t)kTPartsMax * 4;
  P.sB = (uint32_t)lds;
  lds += r16((size_t)32 * maxr);
  P.sX = (uint32_t)lds;
  lds += (size_t)maxK * 2 + 512;  // the row reads up to 256 elements past its end, for blocks it does not add
  P.sXh = (uint32_t)lds;          // the same as fp16 numbers
  lds += (size_t)maxK * 2 + 512;
  P.sXs = (uint32_t)lds;          // block exponents (read up to CH blocks past the row)
  lds += r16((size_t)(maxK / 64 + 8) * 4);
  if (lds > kLdsMax) return hipErrorInvalidValue;
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) tiles += P.L[i].ntiles;
  const int64_t grid = std::min<int64_t>(device_cus(), tiles);
  // ring depth 4 unless a wave's share of its workgroup's run (cost / grid blocks over 8 waves) is at most 2 chunks
  const bool deep = cost / grid / (8 * CH) > 2;
  switch (ls[0].bits) {
    case 2: return launch_gv_group_b<2>(P, grid, lds, adp, deep, ls[0].ydt, lv, s);
    case 3: return launch_gv_group_b<3>(P, grid, lds, adp, deep, ls[0].ydt, lv, s);
    case 4: return launch_gv_group_b<4>(P, grid, lds, adp, deep, ls[0].ydt, lv, s);
    default: return launch_gv_group_b<8>(P, grid, lds, adp, deep, ls[0].ydt, lv, s);
  }
}

hipError_t launch_gemv(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_gemv_y<2>(a, lv, s);
    case 3: return launch_gemv_y<3>(a, lv, s);
    case 4: return launch_gemv_y<4>(a, lv, s);
    default: return launch_gemv_y<8>(a, lv, s);
  }
}

}  // namespace qlr

// Prefill path (bf16 x, any M): dequantizing GEMM on 32x32x16 bf16 MFMA with
// float32 accumulation, plus the unmerged adapter branch.
//
// QLoRA page, section "Limitations": the quantized base is dequantized every
// time it is used.  LoRDBA page, "adapter mode": the adapter stays a separate
// branch, y = x W'^T + scale (x A^T) B^T.
//
// Tiling.  A workgroup of 8 waves owns a 256 (M) x 128 (N) output tile: 4
// producer waves stage operands in LDS and 4 consumer waves multiply them.
// Consumer wave w = 2 nh + mh computes rows [128 mh, 128 mh + 128) x columns
// [64 nh, 64 nh + 64) (4 x 2 MFMA tiles of 32x32, 128 accumulator registers)
// over every 64-element K block.
//
// Operand staging.  Per 64-element K block the producers write two LDS tiles,
// both stored as 128-byte rows whose 16-byte chunks are XOR-swizzled by the row
// index: chunk c of row q sits at q*128 + ((c ^ g(q mod 16)) * 16) with
// g(r) = (r ^ bit2(r) ^ bit3(r)) mod 8.  Fragment reads (16 rows, one chunk)
// and both tile writes then hit distinct banks whether the LDS serves 8 lanes
// x 16 bytes over 32 banks or 16 lanes over 64 banks per cycle; a plain
// g(q) = q mod 8 leaves 2-way conflicts on the fragment reads in the latter:
//  * x: 256 rows, loaded with coalesced buffer loads (8 lanes per 128-byte row;
//    rows past M read as zero).  MFMA fragments loaded straight from global
//    memory would touch 32 rows per instruction, which the L1 serves at about a
//    third of the rate.
//  * W: the tile's 128 weight rows, dequantized by the 256 producer threads (two
//    per row, 32 codes each) to bf16 = round(level(code) * absmax).
// Tiles are triple-buffered (block k in buffer k mod 3, static in the 3-way
// unrolled loop): block k+2 is written while block k is multiplied, so the
// first fragments of block k+1 can be read before the barrier that ends block
// k.  One barrier per block.
//
// 4-bit levels are looked up in registers: the codebook is symmetric, so a
// code c selects one of the 8 positive levels (c - 8 or 7 - c) and the sign is
// bit 3 of c; the 8 scaled bf16 levels of a (row, block) form two 8-byte byte
// tables that v_perm indexes four codes at a time.  Other widths look up
// float32 levels in lane-private LDS tables.
//
// Tile order.  Workgroups are dealt to the 8 XCDs round robin; tile ids are
// remapped so that each XCD walks a contiguous, row-major range of tiles, which
// keeps one 256-row slab of x hot in that XCD's L2.
//
// Dense weights (BITS = 16: the weight given as bf16 values, the Walsh-Hadamard
// branch merged into it).  The producers load the weight tile by direct loads
// as they load x, with no dequantization; tiles are taken column-major, since
// 16-bit weights re-read by every XCD would cost more than x re-read by every XCD.
//
// Adapter.  t = x A^T (float32, from the adapter-product kernel) enters as
// extra K blocks after the last weight block, 32 adapter columns each: the x
// side holds [hi(s t) | lo(s t)] with hi = bf16(s t) and lo = bf16(s t - hi)
// (about 16 significant bits of s t), the weight side [B | B].  The producers
// build them in the steps where the pipeline has no weight block left to
// write, so their loads overlap the last weight blocks' products and the
// consumers run the same MFMA steps over them.
#include <algorithm>
#include <type_traits>

#include <climits>
#include <cstdint>

#include "qlr_internal.h"
#include "qlr_lut.h"

namespace qlr {

namespace {

constexpr int BM = 256, BN = 128;
constexpr uint32_t kXTile = BM * 128;  // bytes of one x tile (256 rows x 64 bf16)
constexpr uint32_t kWTile = BN * 128;  // bytes of one weight tile (128 rows x 64 bf16)
constexpr uint32_t kXOff = 0, kWOff = 3 * kXTile, kTOff = kWOff + 3 * kWTile;

// LDS bytes of the level table for each code width (4-bit levels live in registers).
template <int BITS>
struct GemmTable {
  static constexpr uint32_t kBytes = (BITS == 4) ? 0 : (BITS == 8) ? 256 * 16 * 4 : PairTableF32<BITS>::kBytes;
};
// BITS = 16: the weight is given as dense bf16 values (no codes, no table)
template <>
struct GemmTable<16> {
  static constexpr uint32_t kBytes = 0;
};
template <int BITS>
constexpr uint32_t gemm_lds_bytes() { return kTOff + GemmTable<BITS>::kBytes; }
static_assert(gemm_lds_bytes<3>() <= 160 * 1024 && gemm_lds_bytes<8>() <= 160 * 1024, "LDS budget");
// Outlier side channel of the forward (2- and 4-bit codes, whose level tables
// leave LDS free): after the tiles and the table, the tile's row offsets
// (kGemmTileRows + 1 int32, 528 bytes with padding), then its columns and values.
constexpr uint32_t kLdsAll = 160 * 1024;
template <int BITS>
constexpr uint32_t gemm_sp_off() { return (gemm_lds_bytes<BITS>() + 15u) & ~15u; }
template <int BITS>
constexpr int gemm_sp_cap() { return (BITS == 2 || BITS == 4) ? (int)((kLdsAll - gemm_sp_off<BITS>() - 528) / 8) : 0; }
static_assert(BN == kGemmTileRows, "the side channel's tile rows are the GEMM's");

// Raw codes of one thread for one block: the 32 codes [32h, 32h+32) of a weight row.
template <int BITS>
struct Codes32 {
  uint32_t w[BITS];  // 32*BITS bits
};

template <int BITS>
__device__ __forceinline__ Codes32<BITS> load_codes32(const uint8_t* p) {
  Codes32<BITS> c;
  if constexpr (BITS == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    c.w[0] = u.x; c.w[1] = u.y;
  } else if constexpr (BITS == 3) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);  // 12 bytes at a 4-byte boundary
    c.w[0] = q[0]; c.w[1] = q[1]; c.w[2] = q[2];
  } else if constexpr (BITS == 4) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    c.w[0] = u.x; c.w[1] = u.y; c.w[2] = u.z; c.w[3] = u.w;
  } else {
    const uint4 u0 = *reinterpret_cast<const uint4*>(p);
    const uint4 u1 = *reinterpret_cast<const uint4*>(p + 16);
    c.w[0] = u0.x; c.w[1] = u0.y; c.w[2] = u0.z; c.w[3] = u0.w;
    c.w[4] = u1.x; c.w[5] = u1.y; c.w[6] = u1.z; c.w[7] = u1.w;
  }
  return c;
}

// LDS accesses at a byte address of the dynamic LDS block, which starts at LDS
// address 0 (the kernel has no static LDS; the launcher checks this).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 lds_pair(uint32_t byte_addr) {
  const f32x2_t v = *reinterpret_cast<const __attribute__((address_space(3))) f32x2_t*>((uintptr_t)byte_addr);
  return make_float2(v.x, v.y);
}
__device__ __forceinline__ float lds_f32(uint32_t byte_addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)byte_addr);
}
__device__ __forceinline__ u32x4_t lds_u32x4(uint32_t byte_addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((uintptr_t)byte_addr);
}
__device__ __forceinline__ void lds_store_u32x4(uint32_t byte_addr, u32x4_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>((uintptr_t)byte_addr) = v;
}
__device__ __forceinline__ void lds_store_f32x4(uint32_t byte_addr, f32x4_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) f32x4_t*>((uintptr_t)byte_addr) = v;
}
__device__ __forceinline__ f32x4_t lds_f32x4(uint32_t byte_addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>((uintptr_t)byte_addr);
}
// LDS transpose read of 16-bit elements (ds_read_b64_tr_b16): within each group
// of 16 lanes, lane i receives element i % 4 of the 8-byte reads of lanes
// i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12, in that order.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef s16x4_t u16x4_t;
__device__ __forceinline__ u16x4_t lds_tr16(uint32_t byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>((uintptr_t)byte_addr));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// round-to-nearest-even bf16 pair of (a, b) in one packed conversion
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ uint32_t perm(uint32_t hi4, uint32_t lo4, uint32_t sel) {
  return __builtin_amdgcn_perm(hi4, lo4, sel);
}

// ---- 4-bit register lookup
// Byte tables of the 8 positive scaled levels P[j] = bf16(L[8 + j] * ap):
// lo = low bytes of P[0..7], hi = high bytes, 8 bytes each (two registers).
struct Lut4 {
  uint32_t lo_a, lo_b, hi_a, hi_b;
};

__device__ __forceinline__ Lut4 make_lut4(const Levels& lv, float ap) {
  const uint32_t p01 = cvt_pk_bf16(lv.v[8] * ap, lv.v[9] * ap);
  const uint32_t p23 = cvt_pk_bf16(lv.v[10] * ap, lv.v[11] * ap);
  const uint32_t p45 = cvt_pk_bf16(lv.v[12] * ap, lv.v[13] * ap);
  const uint32_t p67 = cvt_pk_bf16(lv.v[14] * ap, lv.v[15] * ap);
  return {perm(p23, p01, 0x06040200u), perm(p67, p45, 0x06040200u),
          perm(p23, p01, 0x07050301u), perm(p67, p45, 0x07050301u)};
}

// Eight 4-bit codes (LSB first) -> four bf16 pairs in code order.  Code c maps
// to P[c - 8] for c >= 8 and to -P[7 - c] for c < 8: the index is c ^ 7 when
// bit 3 is clear, and the sign is bit 3 clear, set into bit 15 of the bf16.
__device__ __forceinline__ void lut4_word(uint32_t w, const Lut4& t, uint32_t* o) {
  const uint32_t neg = ~w & 0x88888888u;  // bit 3 of every negative code
  const uint32_t m = neg >> 3;
  const uint32_t idx = w ^ ((m << 3) - m);  // low 3 bits of each nibble: level index
  const uint32_t se = idx & 0x07070707u, so = (idx >> 4) & 0x07070707u;  // even / odd codes
  const uint32_t loe = perm(t.lo_b, t.lo_a, se), loo = perm(t.lo_b, t.lo_a, so);
  const uint32_t hie = perm(t.hi_b, t.hi_a, se) | ((neg << 4) & 0x80808080u);
  const uint32_t hio = perm(t.hi_b, t.hi_a, so) | (neg & 0x80808080u);
  const uint32_t l03 = perm(loo, loe, 0x05010400u), h03 = perm(hio, hie, 0x05010400u);
  const uint32_t l47 = perm(loo, loe, 0x07030602u), h47 = perm(hio, hie, 0x07030602u);
  o[0] = perm(h03, l03, 0x05010400u);
  o[1] = perm(h03, l03, 0x07030602u);
  o[2] = perm(h47, l47, 0x05010400u);
  o[3] = perm(h47, l47, 0x07030602u);
}

// Pairs [J0, J1) of the 16 bf16 pairs of one thread's 32 codes, for widths
// other than 4 (float32 levels from a lane-private LDS table; tp = this lane's
// copy): o[j] = bf16 pair of codes 2j, 2j+1.
template <int BITS, int J0, int J1>
__device__ __forceinline__ void dequant_pairs(const Codes32<BITS>& c, float ap, uint32_t tp, uint32_t (&o)[16]) {
#pragma unroll
  for (int j = J0; j < J1; ++j) {
    if constexpr (BITS == 8) {
      // one float32 level per code; 16 lane copies, entry e of copy l at e*64 + 4l
      const uint32_t w = c.w[j >> 1] >> (16 * (j & 1));
      o[j] = cvt_pk_bf16(lds_f32(tp + ((w & 255u) << 6)) * ap, lds_f32(tp + (((w >> 8) & 255u) << 6)) * ap);
    } else {
      // float32 level pairs of two neighbouring codes; 32 lane copies, entry e at e*256 + 8l
      uint32_t e;
      if constexpr (BITS == 2) {
        e = (c.w[j >> 3] >> (4 * (j & 7))) & 15u;
      } else {
        const int bit = 6 * j, wd = bit >> 5, sh = bit & 31;
        uint32_t v = c.w[wd] >> sh;
        if (sh + 6 > 32) v |= c.w[wd + 1] << (32 - sh);
        e = v & 63u;
      }
      const float2 p = lds_pair(tp + (e << 8));
      o[j] = cvt_pk_bf16(p.x * ap, p.y * ap);
    }
  }
}

// XOR swizzle of the 16-byte chunks of LDS tile row r (see the header).
__device__ __forceinline__ uint32_t swz(uint32_t r) {
  return (r ^ ((r >> 2) & 1u) ^ ((r >> 3) & 1u)) & 7u;
}
// Physical 16-byte chunk of logical chunk c (0..15) of row R of the transposed
// GEMM's weight tile: c ^ (0, 6, 10, 12)[R mod 4] ^ bit 3 of c.
__device__ __forceinline__ uint32_t tr_chunk(uint32_t c, uint32_t R) {
  return c ^ ((0xCA60u >> (4u * (R & 3u))) & 15u) ^ ((c >> 3) & 1u);
}

// Level table in LDS for widths other than 4 (built once per workgroup).
template <int BITS>
__device__ __forceinline__ void build_gemm_table(const float* sL, int tid) {
  if constexpr (BITS == 8) {
    for (int idx = tid; idx < 256 * 16; idx += 256) {
      *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)(kTOff + 4 * idx)) = sL[idx >> 4];
    }
  } else if constexpr (BITS != 4) {
    constexpr int NL = 1 << BITS;
    constexpr int E = PairTableF32<BITS>::kEntries;
    for (int idx = tid; idx < E * 32; idx += 256) {
      const int e = idx >> 5;
      *reinterpret_cast<__attribute__((address_space(3))) f32x2_t*>((uintptr_t)(kTOff + 8 * idx)) =
          f32x2_t{sL[e & (NL - 1)], sL[e >> BITS]};
    }
  }
}

// One launch covers up to kGroupMax independent linears of one code width and
// one M (a mixed stack is launched as groups; a single linear is a group of
// one).  Tiles are numbered layer by layer, row tiles outer; the per-layer
// fields are read from the kernel arguments with scalar loads.
constexpr int kGroupMax = 16;
struct GemmLayer {
  const void* x;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* cst;
  const float* t;   // splits x M x r partial sums of x A^T (r > 0)
  const void* B;    // N x r
  void* y;
  const float* addend;  // M x N float32 or null (forward only; with the side channel: its other tiles)
  const int32_t* sp_rp;  // forward: CSR side channel added to the weight tiles that hold it (or null)
  const int32_t* sp_col;
  const float* sp_val;
  int64_t sp_nnz;
  int64_t N, K;
  int32_t r, t_splits;
  float scale;
  int32_t ntiles;   // column tiles (BN rows of W each)
  int64_t tile0;    // first tile of this layer in the launch
};
struct GemmParams {
  int64_t M;               // rows of x and y of every layer
  int64_t m_begin, m_end;  // rows [m_begin, m_end) in this launch
  int64_t mtiles, per_xcd, ntotal;
  int32_t nl;
  GemmLayer L[kGroupMax];
};

// ADP: the call has an adapter branch (r > 0).  Calls without one run a separate
// instantiation (no adapter tail), which also gives it its own kernel name.
//
// TR: the input gradient of the backward, dx = dy W' + scale u A with
// u = dy B (float32 partials in t), contracting over W's rows instead of its
// columns.  The x operand is dy (M x N), the output dx (M x K), the adapter
// operand A (r x K).  Per 64-row step the producers dequantize a 64 x 128
// slice of W' (two blocks of each of 64 rows; four lanes read a row's codes
// together) into a row-major LDS tile of 256-byte rows whose 16-byte chunks are
// XOR-swizzled (tr_chunk).  The consumers read the B fragments (8 consecutive
// rows of one column per lane) with the LDS transpose read, two 4-row reads per
// fragment.  The swizzle keeps both access streams free of bank conflicts
// whether the LDS serves 128 or 256 bytes per cycle: the producers' 16-byte
// stores (8 lanes = 2 rows x 4 chunks c, c + 4, c + 8, c + 12 per cycle, or 16
// lanes = 4 rows), and the transposed 8-byte reads (16 lanes = 4 rows x 2
// chunks x 2 halves per cycle, or 32 lanes).  Chunks c and c + 8 of a row share
// a 128-byte bank window, which the XOR with bit 3 of c pulls apart.
template <int BITS, int YDT, bool ADP, bool TR, bool SPF>
__global__ __launch_bounds__(512, 1) void k_gemm(GemmParams P, Levels lv) {
  static_assert(BITS != 16 || (!ADP && !TR && !SPF), "dense weights: forward without adapter or side channel");
  extern __shared__ uint32_t smem[];
  // XCD-aware tile order: workgroup b runs on XCD b % 8
  const int64_t xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int64_t tile = xcd * P.per_xcd + local;
  if (local >= P.per_xcd || tile >= P.ntotal) return;  // whole workgroup exits
  int li = 0;
  while (li + 1 < P.nl && tile >= P.L[li + 1].tile0) ++li;
  const GemmLayer& Lr = P.L[li];
  LinearArgs a;
  a.x = Lr.x;
  a.M = P.M;
  a.N = Lr.N;
  a.K = Lr.K;
  a.codes = Lr.codes;
  a.q8 = Lr.q8;
  a.cst = Lr.cst;
  a.t = Lr.t;
  a.t_splits = Lr.t_splits;
  a.B = Lr.B;
  a.r = Lr.r;
  a.scale = Lr.scale;
  a.y = Lr.y;
  a.addend = Lr.addend;
  const int64_t N = a.N, K = a.K;
  const int64_t KC = TR ? N : K;  // contraction length (a multiple of 64)
  const int64_t NO = TR ? K : N;  // output columns
  const int64_t nb = KC >> 6;
  // ADP: the adapter branch runs as nbt - nb extra K blocks of 32 adapter columns each
  const int64_t nbt = nb + (ADP ? (a.r + 31) / 32 : 0);
  const int64_t M = P.m_end;
  const int64_t lt = tile - Lr.tile0;
  // layer tiles row-major (one XCD keeps one x slab in its L2); with dense
  // weights column-major (one XCD reads its range of bf16 weight rows once)
  const int64_t mt = BITS == 16 ? lt % P.mtiles : lt / Lr.ntiles;
  const int64_t nt = BITS == 16 ? lt / P.mtiles : lt % Lr.ntiles;
  const int64_t m0 = P.m_begin + mt * BM, n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, h = lane >> 5;
  const int64_t kbl = nb - 1;

  if constexpr (BITS != 4 && BITS != 16) {
    float* sL = reinterpret_cast<float*>(smem) + kXOff / 4;
    stage_levels<1 << BITS>(lv, sL);
    __syncthreads();
    build_gemm_table<BITS>(sL, tid);
  }
  __syncthreads();

  // Outlier side channel (forward, SPF instantiations only): when the entries of the tile's weight rows
  // n0 .. n0 + 127 fit in LDS, the consumers stage them while the producers'
  // first loads are in flight, and each producer thread adds its row's entries
  // to the bf16 weights it has just dequantized (then rounded again to bf16);
  // otherwise the tile adds the float32 addend, which holds its rows.  The
  // offsets are clamped exactly as the addend kernel clamps them, so both agree
  // on which tiles are whose.
  constexpr int kSpCap = (TR || !SPF) ? 0 : gemm_sp_cap<BITS>();
  constexpr uint32_t kSpRo = gemm_sp_off<BITS>(), kSpCol = kSpRo + 528u, kSpVal = kSpCol + 4u * (uint32_t)kSpCap;
  bool spf = false;
  int64_t sp_e0 = 0, sp_cnt = 0;
  if (kSpCap > 0 && Lr.sp_rp != nullptr) {
    const int64_t nnz = Lr.sp_nnz;
    const int64_t e0 = min<int64_t>(max<int64_t>(Lr.sp_rp[n0], 0), nnz);
    const int64_t e1 = max<int64_t>(e0, min<int64_t>(Lr.sp_rp[min(n0 + BN, N)], nnz));
    sp_e0 = e0;
    sp_cnt = e1 - e0;
    spf = sp_cnt <= kSpCap;
  }
  typedef __attribute__((address_space(3))) int lds_int_t;
  auto lds_i32 = [](uint32_t addr) { return *reinterpret_cast<const lds_int_t*>((uintptr_t)addr); };

  if (wave >= 4) {
    // =================== producers: x staging and dequantization ===================
    const int pt = tid - 256;  // 0..255
    const int pw = wave - 4;
    // x of this launch as a buffer resource: reads past its last row return zero
    const uint16_t* xs_base = reinterpret_cast<const uint16_t*>(a.x) + P.m_begin * KC;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(xs_base), (short)0, (int)((P.m_end - P.m_begin) * KC * 2), 0x00020000);
    // load j (0..7) of wave pw: tile rows 64 pw + 8 j + t (t = lane / 8)
    const uint32_t t8 = (uint32_t)(lane >> 3);
    const uint32_t xg_row8 = (uint32_t)(8 * KC * 2);
    // x goes to LDS by direct loads: load j of a wave fills rows 64 pw + 8 j ..
    // + 7 (1 KB, lane L at byte 16 L: row 64 pw + 8 j + L / 8, slot L % 8), so
    // lane L reads the global chunk that the swizzle puts at its slot; the
    // swizzle depends on j only through j & 1
    uint32_t xgd[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      xgd[p] = (uint32_t)(((m0 - P.m_begin) + 64 * pw + t8) * KC + 8 * (((uint32_t)lane & 7u) ^ swz(t8 + 8u * p))) * 2u;
    typedef __attribute__((address_space(3))) char lds_char;
    lds_char* const xlds = (lds_char*)smem + kXOff + pw * 8192;
    if constexpr (BITS == 16) {
      // Dense bf16 weight (a.codes: N x K row-major, N K 2 < 2^31 bytes): the
      // weight tile goes to LDS by direct loads exactly as x does.  Load j (0..3)
      // of wave pw fills tile rows 32 pw + 8 j .. + 7, lane L reading the chunk
      // that the swizzle puts at its slot; rows past N read zero.  Step k issues
      // block k+2 (x and weight: 12 loads per wave) and waits for block k+1.
      const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.codes), (short)0, (int)(N * K * 2), 0x00020000);
      uint32_t wgd[2];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        wgd[p] = (uint32_t)((n0 + 32 * pw + t8) * K + 8 * (((uint32_t)lane & 7u) ^ swz(t8 + 8u * p))) * 2u;
      const uint32_t wg_row8 = (uint32_t)(8 * K * 2);
      lds_char* const wlds = (lds_char*)smem + kWOff + pw * 4096;
      auto load_xw = [&](int64_t kb, int buf) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (void __attribute__((address_space(3)))*)(
                                                           xlds + buf * kXTile + 1024 * j),
                                                   16, xgd[j & 1] + j * xg_row8, (int)(kb * 128), 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (void __attribute__((address_space(3)))*)(
                                                           wlds + buf * kWTile + 1024 * j),
                                                   16, wgd[j & 1] + j * wg_row8, (int)(kb * 128), 0, 0);
      };
      load_xw(0, 0);
      load_xw(min<int64_t>(1, kbl), 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // blocks 0 and 1 in LDS
      __syncthreads();
      // one step (and barrier) per consumer block; the last two load unused copies.
      // The barrier's fence waits for all of the step's direct loads: the
      // consumers read the first fragments of block k+2 before the next barrier.
      for (int64_t k = 0; k < nb; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        load_xw(min(k + 2, kbl), (int)((k + 2) % 3));
        asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        __syncthreads();
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      __syncthreads();
    } else {
      // Forward: weight row n0 + rr (rr = pt / 2), codes [32 dh, 32 dh + 32) of
      // block kb.  TR: weight row 64 kb + rr (rr = pt / 4), codes [32 dh, 32 dh +
      // 32) of block column n0 / 64 + bq.
      const int rr = TR ? (pt >> 2) : (pt >> 1), dh = pt & 1, bq = TR ? ((pt >> 1) & 1) : 0;
      bool wv;
      int64_t wblk, wstep;
      if constexpr (TR) {
        const int64_t nbK = K >> 6, wcol = (n0 >> 6) + bq;
        wv = wcol < nbK;
        wblk = (int64_t)rr * nbK + (wv ? wcol : nbK - 1);
        wstep = 64 * nbK;
      } else {
        const int64_t wn = n0 + rr;
        wv = wn < N;
        wblk = (wv ? wn : N - 1) * nb;
        wstep = 1;
      }
      uint32_t wst[4];  // LDS slot of the thread's chunk q of row rr
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (TR)
          wst[q] = kWOff + (uint32_t)(rr * 256) + (tr_chunk((uint32_t)(8 * bq + 4 * dh + q), (uint32_t)rr) << 4);
        else
          wst[q] = kWOff + (uint32_t)(rr * 128) + ((((uint32_t)(4 * dh + q)) ^ swz((uint32_t)rr & 15u)) << 4);
      }
      const uint32_t tp = kTOff + (BITS == 8 ? 4u * (lane & 15) : 8u * fr);

      struct CS { Codes32<BITS> c; uint32_t q8; float sc; };
      // block kb's x rows into buffer buf (in flight until a vmcnt wait)
      auto load_x_lds = [&](int64_t kb, int buf) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (void __attribute__((address_space(3)))*)(
                                                           xlds + buf * kXTile + 1024 * j),
                                                   16, xgd[j & 1] + j * xg_row8, (int)(kb * 128), 0, 0);
      };
      auto load_c = [&](CS& st, int64_t kb) {
        const int64_t blk = wblk + kb * wstep;
        st.c = load_codes32<BITS>(a.codes + blk * (8 * BITS) + dh * (4 * BITS));
        st.q8 = a.q8[blk];
        st.sc = a.cst[blk >> 8];
      };
      // Dequantization of block kb's codes (pinned first: an empty register-only
      // asm makes them opaque, so instruction selection cannot start their
      // arithmetic right after the load, which would wait for codes in flight).
      struct DQ { Codes32<BITS> c; float ap; Lut4 t; };
      auto dq_begin = [&](const CS& cs) {
        DQ d;
        d.c = cs.c;
        uint32_t q8 = cs.q8;
        float sc = cs.sc;
#pragma unroll
        for (int i = 0; i < BITS; ++i) asm volatile("" : "+v"(d.c.w[i]));
        asm volatile("" : "+v"(q8), "+v"(sc));
        d.ap = wv ? (float)q8 * sc : 0.0f;
        if constexpr (BITS == 4) d.t = make_lut4(lv, d.ap);
        return d;
      };
      // pairs [4 i, 4 i + 4) of the 16 output pairs (for 4-bit: code word i); the
      // results are pinned so that they are computed here, not next to the stores
      auto dq_part = [&](const DQ& d, auto part, uint32_t (&o)[16]) {
        constexpr int I = decltype(part)::value;
        if constexpr (BITS == 4) lut4_word(d.c.w[I], d.t, o + 4 * I);
        else dequant_pairs<BITS, 4 * I, 4 * I + 4>(d.c, d.ap, tp, o);
#pragma unroll
        for (int j = 4 * I; j < 4 * I + 4; ++j) asm volatile("" : "+v"(o[j]));
      };
      auto store_w = [&](const uint32_t (&o)[16], int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          lds_store_u32x4(wst[q] + buf * kWTile, u32x4_t{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]});
      };
      // (side channel) the thread's cursor over its row's entries: index of the
      // next one, the end, and the next two entries' columns (INT_MAX past the end)
      // and values in registers, so the test of a block never waits for LDS
      int sp_e = 0, sp_end = 0, sp_nc = INT_MAX, sp_nc2 = INT_MAX;
      float sp_nv = 0.0f, sp_nv2 = 0.0f;
      auto sp_load = [&](int e, int& c, float& v) {
        const uint32_t ec = (uint32_t)min(e, kSpCap - 1);  // read in range; past the end the entry is dropped
        const int cc = lds_i32(kSpCol + 4u * ec);
        v = lds_f32(kSpVal + 4u * ec);
        c = e < sp_end ? cc : INT_MAX;
      };
      // after block kbk's weights are in buffer buf: add the entries of columns
      // [64 kbk + 32 dh, + 32) to them, one packed bf16 LDS atomic add each (the
      // residual rounded to bf16, the sum rounded to nearest even)
      auto sp_patch = [&](int64_t kbk, int buf) {
        if constexpr (kSpCap > 0) {
          const int lo = (int)(64 * kbk) + 32 * dh, hi = lo + 32;
          while (sp_nc < hi) {
            if (sp_nc >= lo) {
              const uint32_t idx = (uint32_t)(sp_nc - lo);
              const uint32_t ad = kWOff + (uint32_t)buf * kWTile + (uint32_t)(rr * 128) +
                                  (((4u * (uint32_t)dh + (idx >> 3)) ^ swz((uint32_t)rr & 15u)) << 4) + 4u * ((idx & 7u) >> 1);
              const __bf16 hv = (__bf16)sp_nv, zv = (__bf16)0.0f;
              const bf16x2_t add = (idx & 1u) ? bf16x2_t{zv, hv} : bf16x2_t{hv, zv};
              __builtin_amdgcn_ds_atomic_fadd_v2bf16(
                  reinterpret_cast<__attribute__((address_space(3))) bf16x2_t*>((uintptr_t)ad), add);
            }
            ++sp_e;
            sp_nc = sp_nc2;
            sp_nv = sp_nv2;
            sp_load(sp_e + 1, sp_nc2, sp_nv2);
          }
        }
      };
      auto dequant_store = [&](const CS& cs, int buf, int64_t kbk) {
        const DQ d = dq_begin(cs);
        uint32_t o[16];
        dq_part(d, std::integral_constant<int, 0>{}, o);
        dq_part(d, std::integral_constant<int, 1>{}, o);
        dq_part(d, std::integral_constant<int, 2>{}, o);
        dq_part(d, std::integral_constant<int, 3>{}, o);
        store_w(o, buf);
        sp_patch(kbk, buf);
      };

      // Block k+2 is written while the consumers multiply block k.  x(j) and
      // codes(j) live in register set j % 3 and are loaded two blocks before they
      // are written (a set is free again once its block is in LDS).
      CS c0, c1, c2;
      load_x_lds(0, 0);
      load_c(c0, 0);
      if (!(ADP && nb == 1)) load_x_lds(min<int64_t>(1, kbl), 1);
      load_c(c1, min<int64_t>(1, kbl));
      load_c(c2, min<int64_t>(2, kbl));
      if (spf) {
        __syncthreads();  // the consumers have staged the tile's side channel
        sp_e = lds_i32(kSpRo + 4u * (uint32_t)rr);
        sp_end = lds_i32(kSpRo + 4u * (uint32_t)(rr + 1));
        sp_load(sp_e, sp_nc, sp_nv);
        sp_load(sp_e + 1, sp_nc2, sp_nv2);
      }
      dequant_store(c0, 0, 0);
      load_c(c0, min<int64_t>(3, kbl));
      // ADP: adapter block j >= nb (a = j - nb, adapter columns [32 a, 32 a + 32))
      // into buffer j % 3.  x side (thread = tile row): [hi(s t) | lo(s t)], t the
      // float32 adapter product of that row, split into bf16 hi = bf16(s t) and
      // lo = bf16(s t - hi).  Weight side: forward, row n of the tile holds
      // [B[n][32 a ..] | the same]; TR, rows 0..31 and 32..63 both hold A[32 a + row % 32]
      // over the tile's columns.  Runs in steps where the producers would otherwise
      // idle; its operands are mostly L2-resident (shared by the tile's neighbours).
      auto adapter_write = [&](int64_t j) {
        if constexpr (ADP) {
          const int aa = (int)(j - nb), r = a.r;
          const uint32_t bw = (uint32_t)(j % 3);
          const uint16_t* Bl = reinterpret_cast<const uint16_t*>(a.B);
          const u32x4_t zero4 = {0u, 0u, 0u, 0u};
          u32x4_t wv[4];
          if constexpr (TR) {
            const int jj = 32 * aa + (rr & 31);
            const uint16_t* ap = Bl + (int64_t)min(jj, r - 1) * K;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t c = n0 + 64 * bq + 32 * dh + 8 * q;
              const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ap + min(c, K - 8));
              wv[q] = (jj < r && c < K) ? v : zero4;
            }
          } else {
            const int64_t n = n0 + rr;
            const bool nv = n < N;
            const uint16_t* bp = Bl + (nv ? n : N - 1) * (int64_t)r;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int jq = 32 * aa + 8 * q;
              if (r % 8 == 0) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(bp + min(jq, r - 8));
                wv[q] = (nv && jq < r) ? v : zero4;
              } else {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                  const uint32_t lo = (nv && jq + 2 * e2 < r) ? bp[jq + 2 * e2] : 0u;
                  const uint32_t hi = (nv && jq + 2 * e2 + 1 < r) ? bp[jq + 2 * e2 + 1] : 0u;
                  wv[q][e2] = lo | (hi << 16);
                }
              }
            }
          }
          // x side: row pt of the tile
          const int64_t m = m0 + pt;
          const bool mv = m < M;
          float tv[32];
#pragma unroll
          for (int i = 0; i < 32; ++i) tv[i] = 0.0f;
          if (r % 4 == 0) {
            // per split, all eight 16-byte loads in flight at once (clamped
            // addresses, zeroed at use); splits added in order
            for (int sp = 0; sp < a.t_splits; ++sp) {
              const float* tq = a.t + ((int64_t)sp * a.M + (mv ? m : M - 1)) * r;
              f32x4_t v[8];
#pragma unroll
              for (int q4 = 0; q4 < 8; ++q4) v[q4] = *reinterpret_cast<const f32x4_t*>(tq + min(32 * aa + 4 * q4, r - 4));
#pragma unroll
              for (int q4 = 0; q4 < 8; ++q4)
#pragma unroll
                for (int e = 0; e < 4; ++e) tv[4 * q4 + e] += (32 * aa + 4 * q4 < r) ? v[q4][e] : 0.0f;
            }
          } else {
            for (int sp = 0; sp < a.t_splits; ++sp) {
              const float* tq = a.t + ((int64_t)sp * a.M + (mv ? m : M - 1)) * r;
#pragma unroll
              for (int i = 0; i < 32; ++i)
                if (32 * aa + i < r) tv[i] += tq[32 * aa + i];
            }
          }
          const uint32_t xrow = kXOff + bw * kXTile + (uint32_t)pt * 128u;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4_t hv, lv;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              const float u0 = mv ? a.scale * tv[8 * c + 2 * e2] : 0.0f;
              const float u1 = mv ? a.scale * tv[8 * c + 2 * e2 + 1] : 0.0f;
              const uint32_t hb0 = f32_to_bf16_bits(u0), hb1 = f32_to_bf16_bits(u1);
              hv[e2] = hb0 | (hb1 << 16);
              lv[e2] = pack_bf16x2(u0 - bf16_bits_to_f32(hb0), u1 - bf16_bits_to_f32(hb1));
            }
            lds_store_u32x4(xrow + ((((uint32_t)c) ^ swz((uint32_t)pt & 15u)) << 4), hv);
            lds_store_u32x4(xrow + ((((uint32_t)(4 + c)) ^ swz((uint32_t)pt & 15u)) << 4), lv);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) lds_store_u32x4(wst[q] + bw * kWTile, wv[q]);
        }
      };

      if (ADP && nb == 1) {
        adapter_write(1);
      } else {
        dequant_store(c1, 1, min<int64_t>(1, kbl));
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // x of blocks 0 and 1 in LDS
      __syncthreads();
      // Step k: x(k+2) by direct loads into buffer (k+2) % 3 (freed by the last
      // barrier), codes(k+4) into set (k+1) % 3, and the dequantized block k+2
      // into buffer (k+2) % 3.  x(k+2) must be in LDS at the step's barrier:
      // after it the consumers finish block k+1 and, two MFMA steps ahead,
      // already read the first fragments of block k+2.  The fence of
      // __syncthreads() waits for that (for every direct load into LDS in
      // flight; only the step's newest code loads stay outstanding), the
      // explicit wait before it for everything older than the step's 8 newest
      // loads.  So every step holds one round trip of its x loads; issuing x a
      // step earlier would take a fourth buffer.  The step runs in pinned
      // chunks, each a code word's arithmetic, so the wave keeps computing
      // while loads drain.
      auto pstep = [&](CS& cl, const CS& cw, int64_t k, int bw) {
        __builtin_amdgcn_sched_barrier(0);
        load_x_lds(min(k + 2, kbl), bw);
        __builtin_amdgcn_sched_barrier(0);
        load_c(cl, min(k + 4, kbl));
        const DQ d = dq_begin(cw);
        uint32_t o[16];
        dq_part(d, std::integral_constant<int, 0>{}, o);
        __builtin_amdgcn_sched_barrier(0);
        dq_part(d, std::integral_constant<int, 1>{}, o);
        __builtin_amdgcn_sched_barrier(0);
        dq_part(d, std::integral_constant<int, 2>{}, o);
        __builtin_amdgcn_sched_barrier(0);
        dq_part(d, std::integral_constant<int, 3>{}, o);
        store_w(o, bw);
        __builtin_amdgcn_sched_barrier(0);
        sp_patch(min(k + 2, kbl), bw);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      };
      // regular steps write blocks 2 .. nb - 1 (without an adapter, two more steps
      // write unused copies: every step ends with the barrier of one consumer block)
      const int64_t nreg = ADP ? (nb > 2 ? nb - 2 : 0) : nb;
      const int64_t nr3 = nreg - nreg % 3;
      int64_t kb = 0;
      for (; kb < nr3; kb += 3) {
        pstep(c1, c2, kb, 2);
        pstep(c2, c0, kb + 1, 0);
        pstep(c0, c1, kb + 2, 1);
      }
      if (kb < nreg) pstep(c1, c2, kb, 2);
      if (kb + 1 < nreg) pstep(c2, c0, kb + 1, 0);
      // every direct load in LDS before the adapter steps and the epilogue reuse it
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (ADP) {
        // steps nreg .. nbt - 1 write the adapter blocks (j = k + 2 >= nb)
        for (int64_t k = nreg; k < nbt; ++k) {
          if (k + 2 < nbt) adapter_write(k + 2);
          __syncthreads();
        }
      }
      // the consumers' two epilogue barriers: tiles free, then the output staged
      __syncthreads();
      __syncthreads();
    }
  } else {
    // =================== consumers: MFMA on 128 x 64 of the tile ===================
    const int mh = wave & 1, nh = wave >> 1;
    // fragment of step s (0..3): row fr (+32 i or +32 c), chunk 2 s + h.  One LDS
    // base address per step and operand (a second one for the third x buffer,
    // whose offset would pass 64 KB), pinned so that the compiler cannot see
    // their low bits: then every fragment read is base + a constant that fits the
    // instruction's 16-bit offset, instead of a precomputed address register each.
    uint32_t fo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) fo[s] = (uint32_t)(fr * 128) + ((((uint32_t)(2 * s + h)) ^ swz((uint32_t)fr & 15u)) << 4);
    const uint32_t xrow0 = (uint32_t)(128 * mh * 128);
    const uint32_t wrow0 = (uint32_t)(64 * nh * 128);
    uint32_t xb[4], xb2[4], wb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      xb[s] = kXOff + xrow0 + fo[s];
      xb2[s] = xb[s] + 2 * kXTile;
      wb[s] = kWOff + wrow0 + fo[s];
      asm volatile("" : "+v"(xb[s]), "+v"(xb2[s]), "+v"(wb[s]));
    }
    // TR: transpose-read address of 16-lane group g, lane sp, for column tile c
    // (rows 8 h + sp / 4 of the 16-row slice, four columns from 16 (g & 1) + 4 (sp & 3)).
    uint32_t tbo[2];
    if constexpr (TR) {
      const uint32_t g = (uint32_t)lane >> 4, sp = (uint32_t)lane & 15u;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t chunk = 8u * nh + 4u * c + 2u * (g & 1u) + ((sp >> 1) & 1u);
        tbo[c] = (8u * h + (sp >> 2)) * 256u + (tr_chunk(chunk, sp >> 2) << 4) + 8u * (sp & 1u);
      }
    }

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][c][v] = 0.0f;

    if (spf) {
      // the tile's row offsets (relative to its first entry, clamped into [0, count];
      // rows past N get count) and entries (columns clamped into the row), for the producers
      typedef __attribute__((address_space(3))) float lds_float_t;
      for (int i = tid; i <= BN; i += 256) {
        const int64_t v = min<int64_t>(max<int64_t>(Lr.sp_rp[min(n0 + i, N)], sp_e0), sp_e0 + sp_cnt) - sp_e0;
        *reinterpret_cast<lds_int_t*>((uintptr_t)(kSpRo + 4u * (uint32_t)i)) = (int)v;
      }
      for (int64_t j = tid; j < sp_cnt; j += 256) {
        *reinterpret_cast<lds_int_t*>((uintptr_t)(kSpCol + 4u * (uint32_t)j)) =
            min<int32_t>(max<int32_t>(Lr.sp_col[sp_e0 + j], 0), (int32_t)(K - 1));
        *reinterpret_cast<lds_float_t*>((uintptr_t)(kSpVal + 4u * (uint32_t)j)) = Lr.sp_val[sp_e0 + j];
      }
      __syncthreads();  // matches the producers' side-channel barrier
    }
    __syncthreads();  // producers: blocks 0 and 1 written
    // fragments of three MFMA steps in registers: step g (of 12 in the 3-block
    // unrolled loop) uses slot g % 3 while the reads of step g + 2 are in flight
    u32x4_t fa[3][4], fb[3][2];
    auto read_frags = [&](int buf, int s, int slot) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[slot][i] = lds_u32x4(buf == 2 ? xb2[s] + 4096u * i : xb[s] + (uint32_t)buf * kXTile + 4096u * i);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if constexpr (TR) {
          // rows 16 s + 8 h + {0..3} and {4..7} of the lane's column
          const uint32_t ad = kWOff + buf * kWTile + tbo[c] + 4096u * s;
          const u16x4_t lo = lds_tr16(ad), hi = lds_tr16(ad + 1024u);
          fb[slot][c] = u32x4_t{__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y};
        } else {
          fb[slot][c] = lds_u32x4(wb[s] + (uint32_t)buf * kWTile + 4096u * c);
        }
      }
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[i][c] = mfma32x32x16(as_bf16x8(fa[slot][i]), as_bf16x8(fb[slot][c]), acc[i][c]);
    };
    read_frags(0, 0, 0);
    read_frags(0, 1, 1);
    // block k at position J of the unrolled loop: four MFMA steps, each first
    // reading the fragments two steps ahead (steps 2 and 3 of block k, then
    // steps 0 and 1 of block k+1, buffer bn, written one block earlier)
    auto cstep = [&](auto jpos, int bc, int bn) {
      constexpr int J = decltype(jpos)::value;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int g = 4 * J + s;
        __builtin_amdgcn_sched_barrier(0);
        if (s < 2) read_frags(bc, s + 2, (g + 2) % 3);
        else read_frags(bn, s - 2, (g + 2) % 3);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(g % 3);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };
    // the regular blocks, then (ADP) the adapter blocks nb .. nbt - 1 that the
    // producers append: the same MFMA steps over [hi | lo] x [B | B] tiles
    const int64_t nb3 = nbt - nbt % 3;
    int64_t kb = 0;
    for (; kb < nb3; kb += 3) {
      cstep(std::integral_constant<int, 0>{}, 0, 1);
      cstep(std::integral_constant<int, 1>{}, 1, 2);
      cstep(std::integral_constant<int, 2>{}, 2, 0);
    }
    if (kb < nbt) cstep(std::integral_constant<int, 0>{}, 0, 1);
    if (kb + 1 < nbt) cstep(std::integral_constant<int, 1>{}, 1, 2);

    __syncthreads();  // every wave is past its last tile read: the staging area is free

    // ---- row-major staging of the 256 x 128 output tile in LDS:
    // lane (fr, h), register v of tile (i, c) -> row 32 i + 8 (v / 4) + 4 h + v % 4, column 32 c + fr
    constexpr int ES = (YDT == DT_F32) ? 4 : 2;
    constexpr uint32_t RS = 128 * ES + 16;  // padded row stride (bytes)
    // with an addend (forward only) the tile is staged in float32 whatever the
    // output type: the addend is added, and the sum rounded, by the store pass
    const bool stage32 = !TR && a.addend != nullptr && !spf;
    if (stage32) {
      constexpr uint32_t RS4 = 128 * 4 + 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t row = 128 * mh + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
            const uint32_t addr = row * RS4 + (uint32_t)(64 * nh + 32 * c + fr) * 4u;
            *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)addr) = acc[i][c][v];
          }
    } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t row = 128 * mh + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          const uint32_t addr = row * RS + (uint32_t)(64 * nh + 32 * c + fr) * ES;
          if constexpr (YDT == DT_F32)
            *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)addr) = acc[i][c][v];
          else
            *reinterpret_cast<__attribute__((address_space(3))) uint16_t*>((uintptr_t)addr) =
                (uint16_t)f32_to_bf16_bits(acc[i][c][v]);
        }
    }
    __syncthreads();  // staging written
  }
  // ---- coalesced global stores of the staged tile by all 512 threads
  if (!TR && a.addend != nullptr && !spf) {
    // float32 staging: 16-byte chunk idx = tid + 512 q holds columns 4 (idx % 32) ..
    // + 3 of row idx / 32; all 16 addend chunks of a thread are loaded first
    // (clamped addresses, 16-byte loads when the rows are 16-byte aligned)
    constexpr uint32_t RS4 = 128 * 4 + 16;
    const bool vec = (NO % 4) == 0;
    const float* ad = a.addend;
    f32x4_t av[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 512 * q;
      const int64_t gr = min(m0 + (idx >> 5), M - 1), gc = n0 + 4 * (idx & 31);
      if (vec) av[q] = *reinterpret_cast<const f32x4_t*>(ad + gr * NO + min(gc, NO - 4));
    }
    char* y = reinterpret_cast<char*>(a.y);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 512 * q;
      const int row = idx >> 5, ch = idx & 31;
      const int64_t gr = m0 + row, gc = n0 + 4 * ch;
      f32x4_t v = lds_f32x4((uint32_t)row * RS4 + (uint32_t)ch * 16u);
      if (gr < M && gc < NO) {
        if (vec) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = v[e] + av[q][e];
          if constexpr (YDT == DT_F32) {
            *reinterpret_cast<f32x4_t*>(y + (gr * NO + gc) * 4) = v;
          } else {
            *reinterpret_cast<uint2*>(y + (gr * NO + gc) * 2) =
                uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ve = v[e];
            if (gc + e < NO) {
              const float o = ve + ad[gr * NO + gc + e];
              if constexpr (YDT == DT_F32) reinterpret_cast<float*>(y)[gr * NO + gc + e] = o;
              else reinterpret_cast<uint16_t*>(y)[gr * NO + gc + e] = (uint16_t)f32_to_bf16_bits(o);
            }
          }
        }
      }
    }
  } else {
    constexpr int ES = (YDT == DT_F32) ? 4 : 2;
    constexpr uint32_t RS = 128 * ES + 16;
    constexpr int CPR = 128 * ES / 16;  // 16-byte chunks per row
    const bool vec_store = ((NO * ES) % 16) == 0;
    char* y = reinterpret_cast<char*>(a.y);
#pragma unroll 4
    for (int idx = tid; idx < 256 * CPR; idx += 512) {
      const int row = idx / CPR, ch = idx % CPR;
      const int64_t gr = m0 + row;
      const int64_t gc = n0 + ch * (16 / ES);
      const u32x4_t v = lds_u32x4((uint32_t)row * RS + (uint32_t)ch * 16);
      if (gr < M && gc < NO) {
        char* dst = y + (gr * NO + gc) * ES;
        if (vec_store && gc + 16 / ES <= NO) {
          *reinterpret_cast<u32x4_t*>(dst) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 16 / ES; ++e) {
            // (copy the element out first: bit-casting a vector-element lvalue
            // directly reads element 0)
            const uint32_t ve = v[e];
            if (gc + e < NO) {
              if constexpr (YDT == DT_F32) reinterpret_cast<float*>(dst)[e] = __uint_as_float(ve);
              else reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    }
  }
}

// x is read through a buffer resource with 32-bit offsets: one launch covers at
// most 2^31 bytes of x per layer (whole 256-row tiles).
int64_t gemm_max_rows(int64_t K) {
  const int64_t row_bytes = K * 2;
  if (row_bytes * (BM + 8) >= (int64_t(1) << 31)) return 0;
  return std::max<int64_t>(BM, ((int64_t(1) << 31) - 1) / row_bytes / BM * BM);
}

template <int BITS, int YDT, bool ADP, bool TR, bool SPF = false>
hipError_t launch_gemm_t(const LinearArgs* ls, int n, const Levels& lv, hipStream_t s) {
  // SPF (the outlier side channel added to the weight tiles): its staging takes the rest of LDS
  const size_t shmem = SPF ? kLdsAll : gemm_lds_bytes<BITS>();
  auto kern = k_gemm<BITS, YDT, ADP, TR, SPF>;
  static bool attr = false;
  if (!attr) {
    // the kernel addresses LDS from 0: it must not have static LDS
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsAll);
    if (e != hipSuccess) return e;
    attr = true;
  }
  if (n <= 0 || n > kGroupMax) return hipErrorInvalidValue;
  const int64_t M = ls[0].M;
  int64_t max_rows = INT64_MAX;
  for (int i = 0; i < n; ++i) {
    const int64_t mr = gemm_max_rows(TR ? ls[i].N : ls[i].K);
    if (mr == 0 || ls[i].M != M) return hipErrorInvalidValue;
    if (TR && (ls[i].N % 64 != 0 || ls[i].K % 64 != 0)) return hipErrorInvalidValue;
    max_rows = std::min(max_rows, mr);
  }
  for (int64_t mb = 0; mb < M; mb += max_rows) {
    GemmParams P;
    P.M = M;
    P.m_begin = mb;
    P.m_end = std::min(M, mb + max_rows);
    P.mtiles = (P.m_end - mb + BM - 1) / BM;
    P.nl = n;
    int64_t t0 = 0;
    for (int i = 0; i < n; ++i) {
      const LinearArgs& a = ls[i];
      GemmLayer& L = P.L[i];
      L.x = a.x;
      L.codes = a.codes;
      L.q8 = a.q8;
      L.cst = a.cst;
      L.t = a.t;
      L.B = a.B;
      L.y = a.y;
      L.addend = a.addend;
      L.sp_rp = SPF ? a.sp_row_ptr : nullptr;
      L.sp_col = a.sp_col;
      L.sp_val = a.sp_val;
      L.sp_nnz = a.sp_nnz;
      L.N = a.N;
      L.K = a.K;
      L.r = a.r;
      L.t_splits = a.t_splits;
      L.scale = a.scale;
      L.ntiles = (int32_t)(((TR ? a.K : a.N) + BN - 1) / BN);
      L.tile0 = t0;
      t0 += P.mtiles * L.ntiles;
    }
    P.ntotal = t0;
    P.per_xcd = (P.ntotal + 7) / 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * P.per_xcd)), dim3(512), shmem, s, P, lv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, bool TR>
hipError_t launch_gemm_b(const LinearArgs* ls, int n, const Levels& lv, hipStream_t s) {
  bool adp = false;
  for (int i = 0; i < n; ++i) adp = adp || ls[i].r > 0;
  if constexpr (!TR && (BITS == 2 || BITS == 4)) {
    // one linear whose outlier side channel goes into its weight tiles
    if (n == 1 && ls[0].sp_gemm && ls[0].sp_row_ptr != nullptr) {
      if (adp) {
        if (ls[0].ydt == DT_F32) return launch_gemm_t<BITS, DT_F32, true, false, true>(ls, n, lv, s);
        return launch_gemm_t<BITS, DT_BF16, true, false, true>(ls, n, lv, s);
      }
      if (ls[0].ydt == DT_F32) return launch_gemm_t<BITS, DT_F32, false, false, true>(ls, n, lv, s);
      return launch_gemm_t<BITS, DT_BF16, false, false, true>(ls, n, lv, s);
    }
  }
  if (adp) {
    if (ls[0].ydt == DT_F32) return launch_gemm_t<BITS, DT_F32, true, TR>(ls, n, lv, s);
    return launch_gemm_t<BITS, DT_BF16, true, TR>(ls, n, lv, s);
  }
  if (ls[0].ydt == DT_F32) return launch_gemm_t<BITS, DT_F32, false, TR>(ls, n, lv, s);
  return launch_gemm_t<BITS, DT_BF16, false, TR>(ls, n, lv, s);
}

}  // namespace

hipError_t launch_gemm(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  return launch_gemm_group(&a, 1, lv, s);
}

hipError_t launch_gemm_dense(const LinearArgs& a, hipStream_t s) {
  if (a.r != 0 || a.N <= 0 || a.K % 64 != 0 || a.N * a.K * 2 > INT_MAX || a.sp_row_ptr != nullptr)
    return hipErrorInvalidValue;
  static const Levels none{};
  if (a.ydt == DT_F32) return launch_gemm_t<16, DT_F32, false, false>(&a, 1, none, s);
  return launch_gemm_t<16, DT_BF16, false, false>(&a, 1, none, s);
}

int gemm_group_max() { return kGroupMax; }

int64_t gemm_max_rows_of(int64_t KC) { return gemm_max_rows(KC); }

int64_t gemm_sparse_cap(int bits) {
  switch (bits) {
    case 2: return gemm_sp_cap<2>();
    case 4: return gemm_sp_cap<4>();
    default: return 0;
  }
}

hipError_t launch_gemm_group(const LinearArgs* ls, int n, const Levels& lv, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  for (int i = 1; i < n; ++i)
    if (ls[i].bits != ls[0].bits || ls[i].ydt != ls[0].ydt) return hipErrorInvalidValue;
  switch (ls[0].bits) {
    case 2: return launch_gemm_b<2, false>(ls, n, lv, s);
    case 3: return launch_gemm_b<3, false>(ls, n, lv, s);
    case 4: return launch_gemm_b<4, false>(ls, n, lv, s);
    default: return launch_gemm_b<8, false>(ls, n, lv, s);
  }
}

hipError_t launch_gemm_dx(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_gemm_b<2, true>(&a, 1, lv, s);
    case 3: return launch_gemm_b<3, true>(&a, 1, lv, s);
    case 4: return launch_gemm_b<4, true>(&a, 1, lv, s);
    default: return launch_gemm_b<8, true>(&a, 1, lv, s);
  }
}

}  // namespace qlr

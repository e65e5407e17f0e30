// Adapter product t = x A^T, and the float32 forward path.
//
// The forward is y = x W'^T + scale * (x A^T) B^T with the adapter kept as a
// separate, unmerged branch (LoRDBA page, "adapter mode"; QLoRA page,
// memory-decomposition equation: frozen quantized base, bf16 adapters).
#include <algorithm>

#include "qlr_internal.h"

namespace qlr {

namespace {

// ---------------------------------------------------------------- t = x A^T

// float32 arithmetic for any dtypes: one wave per (m, j), lanes split K.
template <int XDT, int ADT>
__global__ __launch_bounds__(256) void k_lora_t_valu(const void* __restrict__ x, int64_t M,
                                                     int64_t K, const void* __restrict__ A, int r,
                                                     float* __restrict__ t) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= M * r) return;
  const int64_t m = item / r;
  const int j = (int)(item % r);
  float acc = 0.0f;
  for (int64_t k = lane; k < K; k += 64)
    acc = fmaf(load_elem<XDT>(x, m * K + k), load_elem<ADT>(A, (int64_t)j * K + k), acc);
  acc = wave_sum(acc);
  if (lane == 0) t[m * r + j] = acc;
}

// bf16 x and A, M > 16: t[m][j] in one pass (no K split).  A workgroup takes
// a tile of mt x rows (16, or 8 when 16-row tiles would leave CUs idle: the
// MFMA's other 8 rows then read zero) and 16 adapter rows.  Its 8 waves split
// K in 64-element blocks.  A wave loads its x and A pieces coalesced (16-byte pieces, 8 lanes
// per 128-byte row segment, through buffer resources: rows past M or r and
// blocks past the wave's range read zero, so every load is unconditional),
// keeps the next block in flight in registers, stages the current one in its
// own LDS slice (a wave's LDS accesses run in order, so no barrier) and reads it
// back in the 16x16x32 bf16 MFMA layout (x rows as the A operand, adapter rows
// as B; rows 144 bytes apart, conflict-free for those reads).  The waves' 16x16
// sums are added through LDS in wave order.
constexpr uint32_t kTRow = 144;                 // LDS row stride (128 bytes + 16)
constexpr uint32_t kTSlice = 2 * 16 * kTRow;     // one wave: x rows, then A rows
// LDS transpose read of 16-bit elements (ds_read_b64_tr_b16): within each group
// of 16 lanes, lane i receives element i % 4 of the 8-byte reads of lanes
// i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12, in that order.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4_t lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(const_cast<char*>(p)));
}
// Byte offset of row k (0..63) of a 64 x 16 bf16 block stored with 32-byte rows;
// rows 8..15 of every 16 swap their 128-byte halves, so the transpose reads of
// rows {q..q+3} and {q+8..q+11} by one half-wave hit distinct banks.
__device__ __forceinline__ uint32_t bt_row(uint32_t k) { return (k * 32u) ^ (((k >> 3) & 1u) << 7); }
__device__ __forceinline__ uint32_t t_off(bool ok, uint32_t off) {
  asm volatile("" : "+v"(off));  // keep the select a select (no branch around the load)
  return ok ? off : 0xFFFFFFF0u;
}
// One launch covers up to kTGroupMax independent products of one M (a mixed
// stack's adapters in groups; a single product is a group of one).  Tiles are
// numbered layer by layer, x-row tiles outer, adapter-row tiles inner, and
// dealt to the XCDs in contiguous ranges (workgroup b runs on XCD b % 8 and
// takes tile (b % 8) per_xcd + b / 8), so the adapter-row tiles of one x-row
// tile share an XCD and its L2 reads those x rows from HBM once.
constexpr int kTGroupMax = 16;
struct TLayer {
  const uint16_t* x;
  const uint16_t* A;  // r x K, or (bt) K x r
  float* t;
  int64_t K;
  int32_t r, jtiles, bt;
  int64_t tile0;
};
constexpr int kTtWaves = 8;
struct TGroup {
  int64_t M;
  int32_t mt;       // x rows per tile (16 or 8)
  int64_t ntiles;   // tiles of all layers
  int64_t per_xcd;  // tiles per XCD: the grid is 8 per_xcd workgroups
  int32_t nl;
  TLayer L[kTGroupMax];
};
__global__ __launch_bounds__(kTtWaves * 64) void k_lora_t_tile(TGroup G) {
  __shared__ __attribute__((aligned(16))) char lds[kTtWaves * kTSlice];
  __shared__ float red[kTtWaves][256];
  const int64_t tile = (int64_t)(blockIdx.x & 7) * G.per_xcd + (blockIdx.x >> 3);
  if (tile >= G.ntiles) return;  // whole workgroup, before any barrier
  int li = 0;
  while (li + 1 < G.nl && tile >= G.L[li + 1].tile0) ++li;
  const TLayer& Ly = G.L[li];
  const uint16_t* __restrict__ x = Ly.x;
  const uint16_t* __restrict__ A = Ly.A;
  float* __restrict__ t = Ly.t;
  const int64_t M = G.M, K = Ly.K;
  const int r = Ly.r;
  const int64_t lt = tile - Ly.tile0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (lt / Ly.jtiles) * G.mt, j0 = (lt % Ly.jtiles) * 16;
  const int64_t nb = K / 64;
  const int64_t kb0 = nb * wave / kTtWaves, kb1 = nb * (wave + 1) / kTtWaves;
  const int64_t mrows = std::min<int64_t>(G.mt, M - m0), jrows = std::min<int64_t>(16, (int64_t)r - j0);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + m0 * K), (short)0, (int)(mrows * K * 2), 0x00020000);
  // bt: the adapter operand is given as K x r (the backward's B, for u = dy B);
  // its 64 x 16 block (rows k, 16 adapter columns from j0) is read as 128
  // 16-byte pieces: piece q = row q / 2, columns 8 (q % 2) .. + 8
  const bool bt = Ly.bt != 0;
  const __amdgpu_buffer_rsrc_t ar = bt ? __builtin_amdgcn_make_buffer_rsrc(
                                             const_cast<uint16_t*>(A + j0), (short)0, (int)((K * r - j0) * 2), 0x00020000)
                                       : __builtin_amdgcn_make_buffer_rsrc(
                                             const_cast<uint16_t*>(A + j0 * K), (short)0, (int)(jrows * K * 2), 0x00020000);
  struct Blk { u32x4_t xa[2], aa[2]; };
  auto load = [&](int64_t kb, Blk& b) {
    const bool kv = kb < kb1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = i * 64 + lane;
      const uint32_t off = t_off(kv, (uint32_t)(((q >> 3) * K + kb * 64 + (q & 7) * 8) * 2));
      b.xa[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      // bt: columns past r are zeroed (a piece is 8 columns; r % 8 == 0)
      const uint32_t boff = t_off(kv && 8 * (q & 1) < jrows, (uint32_t)(((kb * 64 + (q >> 1)) * r + 8 * (q & 1)) * 2));
      uint32_t ao = bt ? boff : off;
      asm volatile("" : "+v"(ao));  // keep the select a select (no branch around the load)
      b.aa[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, ao, 0, 0));
    }
  };
  char* slice = lds + wave * kTSlice;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Blk& b) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = i * 64 + lane;
      const uint32_t o = (uint32_t)(q >> 3) * kTRow + (uint32_t)(q & 7) * 16;
      *reinterpret_cast<u32x4_t*>(slice + o) = b.xa[i];
      if (bt) *reinterpret_cast<u32x4_t*>(slice + 16 * kTRow + bt_row(q >> 1) + 16u * (q & 1)) = b.aa[i];
      else *reinterpret_cast<u32x4_t*>(slice + 16 * kTRow + o) = b.aa[i];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t o = (uint32_t)(lane & 15) * kTRow + (uint32_t)(4 * ks + (lane >> 4)) * 16;
      const u32x4_t xf = *reinterpret_cast<const u32x4_t*>(slice + o);
      u32x4_t af;
      if (bt) {
        // rows 32 ks + 8 g + {0..3} and {4..7} (g = lane / 16) of adapter column lane % 16
        const uint32_t g = (uint32_t)lane >> 4, sp = (uint32_t)lane & 15u;
        const char* base = slice + 16 * kTRow + 8u * (sp & 3u);
        const uint32_t row = 32u * ks + 8u * g + (sp >> 2);
        const s16x4_t lo = lds_tr16(base + bt_row(row)), hi = lds_tr16(base + bt_row(row + 4));
        af = u32x4_t{__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                     __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y};
      } else {
        af = *reinterpret_cast<const u32x4_t*>(slice + 16 * kTRow + o);
      }
      acc = mfma16x16x32(as_bf16x8(xf), as_bf16x8(af), acc);
    }
  };
  Blk b0, b1;
  load(kb0, b0);
  load(kb0 + 1, b1);
  for (int64_t kb = kb0; kb < kb1; kb += 2) {
    compute(b0);
    load(kb + 2, b0);
    if (kb + 1 < kb1) compute(b1);
    load(kb + 3, b1);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][lane * 4 + v] = acc[v];
  __syncthreads();
  const int e = threadIdx.x;
  if (e < 256) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kTtWaves; ++w) sum += red[w][e];  // wave order
    const int l = e >> 2, v = e & 3;
    const int mi = 4 * (l >> 4) + v;        // MFMA output row
    const int64_t m = m0 + mi;
    const int64_t j = j0 + (l & 15);        // MFMA output column
    if (mi < G.mt && m < M && j < r) t[m * r + j] = sum;
  }
}

// bf16 x and A, M <= 16 (one 16-row MFMA tile): K-split partial sums
// p[s][m][j] of t = x A^T.  Workgroup (16 adapter rows j0 .. j0 + 15, split s)
// of 16 waves: wave w takes the 32-column steps c0 + w, c0 + w + 16, ... of the
// split, issues the loads of up to kLtSteps of them before any product (the
// split count keeps a split within one such round for the decode shapes), and
// multiplies on 16x16x32 bf16 MFMA (x rows as the A operand, adapter rows as
// B).  A step's loads give each quad of lanes one row's 64 bytes (lane l: row
// l / 4, 8 columns from 8 (l % 4)), the rate the address unit sustains, and a
// lane permute per word puts row n's piece g in lane 16 g + n, the fragment
// layout.  The 16 waves' sums are added through LDS in wave order.
constexpr int kLtWaves = 16, kLtSteps = 8;
__device__ __forceinline__ void lora_t_small_body(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                  const uint16_t* __restrict__ A, int r, float* __restrict__ p,
                                                  int j0, int S, int sidx, float (*red)[256]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane >> 2, g = lane & 3;  // the lane's loads
  const bool xv = row < M, av = j0 + row < r;
  const uint16_t* xp = x + (int64_t)(xv ? row : 0) * K + g * 8;
  const uint16_t* ap = A + (int64_t)(av ? j0 + row : 0) * K + g * 8;
  const int src = (4 * (lane & 15) + (lane >> 4)) << 2;  // lane 16 g + n <- lane 4 n + g
  const int64_t nsteps = K / 32;
  const int64_t c0 = nsteps * sidx / S, c1 = nsteps * (sidx + 1) / S;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int64_t base = c0 + wave; base < c1; base += kLtWaves * kLtSteps) {
    u32x4_t xa[kLtSteps], ab[kLtSteps];
#pragma unroll
    for (int i = 0; i < kLtSteps; ++i) {
      const int64_t st = base + (int64_t)i * kLtWaves;
      const bool sv = st < c1;
      const int64_t k = (sv ? st : c0) * 32;
      xa[i] = (xv && sv) ? *reinterpret_cast<const u32x4_t*>(xp + k) : zero;
      ab[i] = (av && sv) ? *reinterpret_cast<const u32x4_t*>(ap + k) : zero;
    }
#pragma unroll
    for (int i = 0; i < kLtSteps; ++i) {
      if (base + (int64_t)i * kLtWaves >= c1) break;  // uniform: the split's last steps
      u32x4_t xf, af;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xf[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)xa[i][j]);
        af[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)ab[i][j]);
      }
      acc = mfma16x16x32(as_bf16x8(xf), as_bf16x8(af), acc);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][lane * 4 + v] = acc[v];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int e = threadIdx.x;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kLtWaves; ++w) sum += red[w][e];
    const int l = e >> 2, v = e & 3;
    const int m = 4 * (l >> 4) + v;  // MFMA output row (x row)
    const int j = j0 + (l & 15);     // MFMA output column (adapter row)
    if (m < M && j < r) p[((int64_t)sidx * M + m) * r + j] = sum;
  }
}

__global__ __launch_bounds__(kLtWaves * 64) void k_lora_t_small(const uint16_t* __restrict__ x, int64_t M,
                                                               int64_t K, const uint16_t* __restrict__ A, int r,
                                                               float* __restrict__ p) {
  __shared__ float red[kLtWaves][256];
  lora_t_small_body(x, M, K, A, r, p, blockIdx.x * 16, gridDim.y, blockIdx.y, red);
}

// Several products of one M <= 16 in one launch (a mixed stack's decode):
// workgroup w belongs to the item whose range [wg0, wg0 + jtiles x splits)
// holds it, and takes (16 adapter rows, split) of that item as k_lora_t_small.
constexpr int kLtsGroupMax = 32;
struct LtsItem {
  const uint16_t* x;
  const uint16_t* A;
  float* t;
  int64_t K;
  int32_t r, splits, jtiles, wg0;
};
struct LtsGroup {
  int64_t M;
  int32_t n;
  LtsItem L[kLtsGroupMax];
};
__global__ __launch_bounds__(kLtWaves * 64) void k_lora_t_small_group(LtsGroup G) {
  __shared__ float red[kLtWaves][256];
  int li = 0;
  while (li + 1 < G.n && (int32_t)blockIdx.x >= G.L[li + 1].wg0) ++li;
  const LtsItem& it = G.L[li];
  const int local = (int)blockIdx.x - it.wg0;
  lora_t_small_body(it.x, G.M, it.K, it.A, it.r, it.t, (local % it.jtiles) * 16, it.splits, local / it.jtiles, red);
}

// ---------------------------------------------------------------- float32 forward

// One wave per output row n; lanes take the 64 elements of each block; x rows in
// chunks of 8.  w' is formed exactly as dequantization defines it.
template <int BITS, int XDT, int BDT, int YDT>
__global__ __launch_bounds__(256) void k_linear_f32(LinearArgs a, Levels lv) {
  constexpr int NL = 1 << BITS;
  __shared__ float sL[NL];
  stage_levels<NL>(lv, sL);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.N) return;
  const int64_t nb = a.K / 64;
  const int bit0 = BITS * lane, byte0 = bit0 >> 3, sh = bit0 & 7;
  for (int64_t m0 = 0; m0 < a.M; m0 += 8) {
    float acc[8] = {};
    for (int64_t kb = 0; kb < nb; ++kb) {
      const int64_t blk = n * nb + kb;
      const uint8_t* cb = a.codes + blk * (8 * BITS);
      uint32_t two = cb[byte0];
      if (byte0 + 1 < 8 * BITS) two |= (uint32_t)cb[byte0 + 1] << 8;
      const int c = (int)((two >> sh) & (NL - 1));
      const float ap = (float)a.q8[blk] * a.cst[blk >> 8];
      const float w = sL[c] * ap;
      const int64_t k = kb * 64 + lane;
#pragma unroll
      for (int mm = 0; mm < 8; ++mm)
        if (m0 + mm < a.M) acc[mm] = fmaf(load_elem<XDT>(a.x, (m0 + mm) * a.K + k), w, acc[mm]);
    }
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      const int64_t m = m0 + mm;
      if (m >= a.M) break;
      float base = wave_sum(acc[mm]);
      float lo = 0.0f;
      for (int j = lane; j < a.r; j += 64) {
        float tj = 0.0f;
        for (int sp = 0; sp < a.t_splits; ++sp) tj += a.t[((int64_t)sp * a.M + m) * a.r + j];
        lo = fmaf(tj, load_elem<BDT>(a.B, n * a.r + j), lo);
      }
      lo = wave_sum(lo);
      float out = fmaf(a.scale, lo, base);
      if (a.addend) out += a.addend[m * a.N + n];
      if (lane == 0) {
        if constexpr (YDT == DT_F32) reinterpret_cast<float*>(a.y)[m * a.N + n] = out;
        else reinterpret_cast<uint16_t*>(a.y)[m * a.N + n] = (uint16_t)f32_to_bf16_bits(out);
      }
    }
  }
}

template <int BITS, int XDT, int BDT>
hipError_t launch_f32_b3(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
  if (a.ydt == DT_F32) hipLaunchKernelGGL((k_linear_f32<BITS, XDT, BDT, DT_F32>), grid, block, 0, s, a, lv);
  else hipLaunchKernelGGL((k_linear_f32<BITS, XDT, BDT, DT_BF16>), grid, block, 0, s, a, lv);
  return hipGetLastError();
}

template <int BITS, int XDT>
hipError_t launch_f32_b2(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.abdt == DT_F32) return launch_f32_b3<BITS, XDT, DT_F32>(a, lv, s);
  return launch_f32_b3<BITS, XDT, DT_BF16>(a, lv, s);
}

template <int BITS>
hipError_t launch_f32_b1(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.xdt == DT_F32) return launch_f32_b2<BITS, DT_F32>(a, lv, s);
  return launch_f32_b2<BITS, DT_BF16>(a, lv, s);
}

}  // namespace

int lora_t_splits(int64_t M, int64_t K, int r, int xdt, int abdt) {
  if (!(xdt == DT_BF16 && abdt == DT_BF16) || M > 16 || K % 64 != 0) return 1;
  // enough splits to spread A over the chip, few enough that a decode
  // workgroup prefetches all partial sums in one round (kTPartsMax floats)
  const int64_t steps = K / 32;
  int64_t s = std::min<int64_t>(steps / 4, 64);
  s = std::min<int64_t>(s, std::max<int64_t>(1, kTPartsMax / (M * std::max(r, 1))));
  return (int)std::max<int64_t>(s, 1);
}

hipError_t launch_lora_t(const void* x, int xdt, int64_t M, int64_t K, const void* A, int abdt,
                         int r, float* t, int splits, hipStream_t s) {
  if (M == 0 || r == 0) return hipSuccess;
  const bool mfma = xdt == DT_BF16 && abdt == DT_BF16 && K % 64 == 0;
  if (mfma && M > 16) {
    if (splits != 1) return hipErrorInvalidValue;
    const LoraTItem it{x, A, t, K, r};
    return launch_lora_t_group(&it, 1, M, s);
  }
  if (mfma) {
    if (M > 16 || splits < 1 || splits > 65535) return hipErrorInvalidValue;
    dim3 grid((unsigned)((r + 15) / 16), (unsigned)splits);
    hipLaunchKernelGGL(k_lora_t_small, grid, dim3(kLtWaves * 64), 0, s, reinterpret_cast<const uint16_t*>(x), M,
                       K, reinterpret_cast<const uint16_t*>(A), r, t);
    return hipGetLastError();
  }
  const int64_t items = M * r;
  dim3 grid((unsigned)((items + 3) / 4)), block(256);
  if (xdt == DT_F32 && abdt == DT_F32)
    hipLaunchKernelGGL((k_lora_t_valu<DT_F32, DT_F32>), grid, block, 0, s, x, M, K, A, r, t);
  else if (xdt == DT_F32)
    hipLaunchKernelGGL((k_lora_t_valu<DT_F32, DT_BF16>), grid, block, 0, s, x, M, K, A, r, t);
  else if (abdt == DT_F32)
    hipLaunchKernelGGL((k_lora_t_valu<DT_BF16, DT_F32>), grid, block, 0, s, x, M, K, A, r, t);
  else
    hipLaunchKernelGGL((k_lora_t_valu<DT_BF16, DT_BF16>), grid, block, 0, s, x, M, K, A, r, t);
  return hipGetLastError();
}

hipError_t launch_linear_f32(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_f32_b1<2>(a, lv, s);
    case 3: return launch_f32_b1<3>(a, lv, s);
    case 4: return launch_f32_b1<4>(a, lv, s);
    default: return launch_f32_b1<8>(a, lv, s);
  }
}

int lora_t_group_max() { return kTGroupMax; }

int lora_t_small_group_max() { return kLtsGroupMax; }

hipError_t launch_lora_t_small_group(const LoraTItem* items, int n, int64_t M, hipStream_t s) {
  if (n <= 0 || M <= 0) return hipSuccess;
  if (n > kLtsGroupMax || M > 16) return hipErrorInvalidValue;
  LtsGroup G;
  G.M = M;
  G.n = 0;
  int32_t wg = 0;
  for (int i = 0; i < n; ++i) {
    const LoraTItem& it = items[i];
    if (it.r <= 0) continue;
    if (it.bt || it.K % 64 != 0) return hipErrorInvalidValue;
    LtsItem& L = G.L[G.n++];
    L.x = reinterpret_cast<const uint16_t*>(it.x);
    L.A = reinterpret_cast<const uint16_t*>(it.A);
    L.t = it.t;
    L.K = it.K;
    L.r = it.r;
    L.splits = lora_t_splits(M, it.K, it.r, DT_BF16, DT_BF16);
    L.jtiles = (it.r + 15) / 16;
    L.wg0 = wg;
    wg += L.jtiles * L.splits;
  }
  if (G.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lora_t_small_group, dim3((unsigned)wg), dim3(kLtWaves * 64), 0, s, G);
  return hipGetLastError();
}

hipError_t launch_lora_t_group(const LoraTItem* items, int n, int64_t M, hipStream_t s) {
  if (n <= 0 || M <= 0) return hipSuccess;
  if (n > kTGroupMax || M <= 16) return hipErrorInvalidValue;
  TGroup G;
  G.M = M;
  G.nl = 0;
  int64_t jt = 0;
  for (int i = 0; i < n; ++i)
    if (items[i].r > 0) jt += (items[i].r + 15) / 16;
  // 8-row tiles when 16-row ones would give fewer workgroups than CUs
  G.mt = ((M + 15) / 16) * jt < 256 ? 8 : 16;
  int64_t t0 = 0;
  const int64_t mtiles = (M + G.mt - 1) / G.mt;
  for (int i = 0; i < n; ++i) {
    const LoraTItem& it = items[i];
    if (it.r <= 0) continue;
    // 16 rows of x or A are addressed with 32-bit buffer offsets
    if (16 * it.K * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    TLayer& L = G.L[G.nl++];
    L.x = reinterpret_cast<const uint16_t*>(it.x);
    L.A = reinterpret_cast<const uint16_t*>(it.A);
    L.t = it.t;
    L.K = it.K;
    L.r = it.r;
    L.jtiles = (it.r + 15) / 16;
    L.bt = it.bt ? 1 : 0;
    if (it.bt && it.r % 8 != 0) return hipErrorInvalidValue;
    L.tile0 = t0;
    t0 += mtiles * L.jtiles;
  }
  if (G.nl == 0) return hipSuccess;
  G.ntiles = t0;
  G.per_xcd = (t0 + 7) / 8;
  hipLaunchKernelGGL(k_lora_t_tile, dim3((unsigned)(8 * G.per_xcd)), dim3(kTtWaves * 64), 0, s, G);
  return hipGetLastError();
}

}  // namespace qlr

// Decode path (M <= 16, bf16 x): the dequantizing GEMV of the frozen base with
// the unmerged adapter added in the epilogue.
//
// The frozen base is read once, as packed k-bit codes (QLoRA page,
// memory-decomposition equation: the 4-bit base takes about half a byte per
// weight), so the kernel is bound by HBM bandwidth; the dequantization the
// QLoRA page's limitations section mentions is fused into the load path.
//
// Layout on the 16x16x32 bf16 MFMA (A = x rows, B = unscaled levels):
//   lane l: x row / weight row (l & 15), lane group g = l >> 4 owns the 16
//   consecutive elements [16g, 16g+16) of each 64-element block; the first
//   MFMA takes elements [16g, 16g+8), the second [16g+8, 16g+16).  Both MFMAs
//   of a block therefore stay inside one block, so the block's dequantized
//   absmax multiplies the 16x16 product afterwards (one FMA per output and
//   block) instead of every weight.
// Levels are looked up in a lane-private LDS table indexed by the packed code
// bits of two neighbouring weights (entry e of lane L at byte e*256 + 4L), so
// 64 lanes never collide on a bank; one table read yields a bf16 pair.
#include "qlr_internal.h"

namespace qlr {

namespace {

template <int BITS>
struct PairTable {
  // entries per lane copy: 2 codes per entry, except 8-bit (one code, bf16 in the low half)
  static constexpr int kEntries = (BITS == 8) ? 256 : (1 << (2 * BITS));
  static constexpr int kBytes = kEntries * 256;
};

template <int BITS>
__device__ __forceinline__ void build_table(uint32_t* tbl, const Levels& lv, int tid, int nthreads) {
  constexpr int NL = 1 << BITS;
  constexpr int E = PairTable<BITS>::kEntries;
  for (int idx = tid; idx < E * 64; idx += nthreads) {
    const int e = idx >> 6;
    uint32_t v;
    if constexpr (BITS == 8) v = f32_to_bf16_bits(lv.v[e]);
    else v = pack_bf16x2(lv.v[e & (NL - 1)], lv.v[e >> BITS]);
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

template <int BITS, int YDT, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(LinearArgs a, Levels lv) {
  extern __shared__ uint32_t smem[];
  uint32_t* tbl = smem;
  float* sRed = reinterpret_cast<float*>(smem + PairTable<BITS>::kBytes / 4);

  const int tid = threadIdx.x;
  build_table<BITS>(tbl, lv, tid, WAVES * 64);

  const int lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int64_t N = a.N, K = a.K, nb = K >> 6;
  const int M = (int)a.M;
  const int64_t n = (int64_t)blockIdx.x * 16 + nl;
  const bool nvalid = n < N;
  const int64_t nrow = nvalid ? n : N - 1;
  const int64_t blk_row = nrow * nb;
  const uint8_t* crow = a.codes + blk_row * (8 * BITS);
  const uint8_t* qrow = a.q8 + blk_row;
  const bool xvalid = nl < M;
  const uint16_t* xrow = reinterpret_cast<const uint16_t*>(a.x) + (int64_t)(xvalid ? nl : 0) * K + 16 * g;
  const int64_t kb0 = nb * wave / WAVES, kb1 = nb * (wave + 1) / WAVES;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  auto body = [&](const Raw<BITS>& raw, float ap, const u32x4_t& x0, const u32x4_t& x1) {
    u32x4_t b0, b1;
    decode16<BITS>(raw, tbl, lane4, b0, b1);
    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
    d = mfma16x16x32(as_bf16x8(x0), as_bf16x8(b0), d);
    d = mfma16x16x32(as_bf16x8(x1), as_bf16x8(b1), d);
    acc[0] = fmaf(ap, d[0], acc[0]);
    acc[1] = fmaf(ap, d[1], acc[1]);
    acc[2] = fmaf(ap, d[2], acc[2]);
    acc[3] = fmaf(ap, d[3], acc[3]);
  };

  int64_t kb = kb0;
  for (; kb + U <= kb1; kb += U) {
    Raw<BITS> raw[U];
    float ap[U];
    u32x4_t x0[U], x1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      raw[u] = load_raw<BITS>(crow + (kb + u) * (8 * BITS), g);
      const float sc = a.cst[(blk_row + kb + u) >> 8];
      ap[u] = nvalid ? (float)qrow[kb + u] * sc : 0.0f;
      if (xvalid) {
        x0[u] = *reinterpret_cast<const u32x4_t*>(xrow + (kb + u) * 64);
        x1[u] = *reinterpret_cast<const u32x4_t*>(xrow + (kb + u) * 64 + 8);
      } else {
        x0[u] = zero;
        x1[u] = zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) body(raw[u], ap[u], x0[u], x1[u]);
  }
  for (; kb < kb1; ++kb) {
    const Raw<BITS> raw = load_raw<BITS>(crow + kb * (8 * BITS), g);
    const float sc = a.cst[(blk_row + kb) >> 8];
    const float ap = nvalid ? (float)qrow[kb] * sc : 0.0f;
    u32x4_t x0 = zero, x1 = zero;
    if (xvalid) {
      x0 = *reinterpret_cast<const u32x4_t*>(xrow + kb * 64);
      x1 = *reinterpret_cast<const u32x4_t*>(xrow + kb * 64 + 8);
    }
    body(raw, ap, x0, x1);
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) sRed[wave * 256 + lane * 4 + v] = acc[v];
  __syncthreads();
  if (tid < 256) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += sRed[w * 256 + tid];
    const int l = tid >> 2, v = tid & 3;
    const int m = 4 * (l >> 4) + v;  // MFMA output row (x row)
    const int64_t nn = (int64_t)blockIdx.x * 16 + (l & 15);
    if (m < M && nn < N) {
      float lo = 0.0f;
      if (a.r > 0) {
        const float* tr = a.t + (int64_t)m * a.r;
        const uint16_t* br = reinterpret_cast<const uint16_t*>(a.B) + nn * a.r;
        for (int j = 0; j < a.r; ++j) lo = fmaf(tr[j], bf16_bits_to_f32(br[j]), lo);
      }
      const float out = fmaf(a.scale, lo, s);
      if constexpr (YDT == DT_F32) reinterpret_cast<float*>(a.y)[(int64_t)m * N + nn] = out;
      else reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * N + nn] = (uint16_t)f32_to_bf16_bits(out);
    }
  }
}

template <int BITS, int YDT>
hipError_t launch_gemv_b(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  constexpr int WAVES = 4, U = 4;
  const size_t shmem = PairTable<BITS>::kBytes + (size_t)WAVES * 256 * sizeof(float);
  auto kern = k_gemv<BITS, YDT, WAVES, U>;
  static bool attr_set = false;  // idempotent; set once per instantiation
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)((a.N + 15) / 16)), block(WAVES * 64);
  hipLaunchKernelGGL(kern, grid, block, shmem, s, a, lv);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_gemv_y(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.ydt == DT_F32) return launch_gemv_b<BITS, DT_F32>(a, lv, s);
  return launch_gemv_b<BITS, DT_BF16>(a, lv, s);
}

}  // namespace

hipError_t launch_gemv(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_gemv_y<2>(a, lv, s);
    case 3: return launch_gemv_y<3>(a, lv, s);
    case 4: return launch_gemv_y<4>(a, lv, s);
    default: return launch_gemv_y<8>(a, lv, s);
  }
}

}  // namespace qlr

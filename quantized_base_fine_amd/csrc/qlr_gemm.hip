// Prefill path (bf16 x, any M): the frozen base dequantized into LDS-staged
// bf16 tiles feeding 32x32x16 bf16 MFMA with float32 accumulation, and the
// unmerged adapter branch added as extra K steps.
//
// QLoRA page, section "Limitations": the quantized base is dequantized every
// time it is used; here that happens once per 128x64 weight tile and
// workgroup, straight into LDS.  LoRDBA page, "adapter mode": the adapter is a
// separate branch, y = x W'^T + scale (x A^T) B^T; with t = x A^T precomputed,
// the branch is the product [hi(s t) | lo(s t)] [B | B]^T, where hi/lo split
// s*t into two bf16 terms so the adapter product keeps about 16 bits.
#include "qlr_internal.h"

namespace qlr {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;  // LDS row stride (bf16): 144 bytes

template <int BITS>
__device__ __forceinline__ void load_codes32(const uint8_t* p, uint32_t (&c)[BITS]) {
  // the 32 codes of half a block: 4*BITS bytes at p (4-byte aligned for BITS != 3)
  if constexpr (BITS == 3) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int i = 0; i < 3; ++i) c[i] = (uint32_t)h[2 * i] | ((uint32_t)h[2 * i + 1] << 16);
  } else if constexpr (BITS == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    c[0] = u.x; c[1] = u.y;
  } else if constexpr (BITS == 4) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    c[0] = u.x; c[1] = u.y; c[2] = u.z; c[3] = u.w;
  } else {
    const uint4 u0 = *reinterpret_cast<const uint4*>(p);
    const uint4 u1 = *reinterpret_cast<const uint4*>(p + 16);
    c[0] = u0.x; c[1] = u0.y; c[2] = u0.z; c[3] = u0.w;
    c[4] = u1.x; c[5] = u1.y; c[6] = u1.z; c[7] = u1.w;
  }
}

template <int BITS>
__device__ __forceinline__ int code_at(const uint32_t (&c)[BITS], int e) {
  const int bit = BITS * e, w = bit >> 5, sh = bit & 31;
  uint32_t v = c[w] >> sh;
  if (sh + BITS > 32) v |= c[w + 1] << (32 - sh);
  return (int)(v & ((1u << BITS) - 1));
}

template <int BITS, int YDT>
__global__ __launch_bounds__(256) void k_gemm(LinearArgs a, Levels lv) {
  constexpr int NL = 1 << BITS;
  __shared__ __attribute__((aligned(16))) uint16_t sX[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sW[BN * LDK];
  __shared__ float sL[NL];

  const int tid = threadIdx.x;
  stage_levels<NL>(lv, sL);

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t M = a.M, N = a.N, K = a.K, nb = K >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);

  // loader mapping: row (tid >> 1), half block (tid & 1): 32 elements each
  const int lrow = tid >> 1, lhalf = tid & 1;
  const int64_t xm = m0 + lrow, wn_row = n0 + lrow;
  const bool xv = xm < M, wv = wn_row < N;
  const uint16_t* xsrc = x + (xv ? xm : 0) * K + lhalf * 32;
  const int64_t wblk_row = (wv ? wn_row : 0) * nb;
  uint16_t* xdst = sX + lrow * LDK + lhalf * 32;
  uint16_t* wdst = sW + lrow * LDK + lhalf * 32;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fk = (lane >> 5) * 8;
  auto mma_tile = [&]() {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const u32x4_t*>(sX + (wm * 64 + i * 32 + fr) * LDK + ks * 16 + fk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const u32x4_t*>(sW + (wn * 64 + j * 32 + fr) * LDK + ks * 16 + fk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(as_bf16x8(af[i]), as_bf16x8(bfr[j]), acc[i][j]);
    }
  };

  __syncthreads();
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll 1
  for (int64_t kb = 0; kb < nb; ++kb) {
    uint4 xr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = xv ? *reinterpret_cast<const uint4*>(xsrc + kb * 64 + i * 8) : z4;
    uint32_t c[BITS];
    float ap = 0.0f;
    if (wv) {
      const int64_t blk = wblk_row + kb;
      load_codes32<BITS>(a.codes + blk * (8 * BITS) + lhalf * (4 * BITS), c);
      ap = (float)a.q8[blk] * a.cst[blk >> 8];
    } else {
#pragma unroll
      for (int i = 0; i < BITS; ++i) c[i] = 0u;
    }
    uint32_t wp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      wp[i] = pack_bf16x2(sL[code_at<BITS>(c, 2 * i)] * ap, sL[code_at<BITS>(c, 2 * i + 1)] * ap);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(xdst + i * 8) = xr[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(wdst + i * 8) = make_uint4(wp[4 * i], wp[4 * i + 1], wp[4 * i + 2], wp[4 * i + 3]);
    __syncthreads();
    mma_tile();
    __syncthreads();
  }

  // adapter branch as extra K: columns [0, rp) hold hi(s t), [rp, 2rp) lo(s t)
  if (a.r > 0) {
    const int r = a.r, rp = (r + 15) & ~15, ke = 2 * rp;
    const uint16_t* Bl = reinterpret_cast<const uint16_t*>(a.B);
#pragma unroll 1
    for (int kc = 0; kc < ke; kc += BK) {
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int kk = kc + lhalf * 32 + i;
        uint16_t xv16 = 0, wv16 = 0;
        if (kk < ke) {
          const int j = kk < rp ? kk : kk - rp;
          if (j < r) {
            if (xv) {
              float tj = 0.0f;
              for (int sp = 0; sp < a.t_splits; ++sp) tj += a.t[((int64_t)sp * M + xm) * r + j];
              const float st = a.scale * tj;
              const uint32_t hi = f32_to_bf16_bits(st);
              xv16 = (uint16_t)(kk < rp ? hi : f32_to_bf16_bits(st - bf16_bits_to_f32(hi)));
            }
            if (wv) wv16 = Bl[wn_row * r + j];
          }
        }
        xdst[i] = xv16;
        wdst[i] = wv16;
      }
      __syncthreads();
      mma_tile();
      __syncthreads();
    }
  }

  // store: 32x32 output layout, lane l / register v -> row 8(v/4) + 4(l/32) + v%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < M && col < N) {
          if constexpr (YDT == DT_F32) reinterpret_cast<float*>(a.y)[row * N + col] = acc[i][j][v];
          else reinterpret_cast<uint16_t*>(a.y)[row * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][v]);
        }
      }
}

template <int BITS>
hipError_t launch_gemm_b(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM)), block(256);
  if (a.ydt == DT_F32) hipLaunchKernelGGL((k_gemm<BITS, DT_F32>), grid, block, 0, s, a, lv);
  else hipLaunchKernelGGL((k_gemm<BITS, DT_BF16>), grid, block, 0, s, a, lv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_gemm_b<2>(a, lv, s);
    case 3: return launch_gemm_b<3>(a, lv, s);
    case 4: return launch_gemm_b<4>(a, lv, s);
    default: return launch_gemm_b<8>(a, lv, s);
  }
}

}  // namespace qlr

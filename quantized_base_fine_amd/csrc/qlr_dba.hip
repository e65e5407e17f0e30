// Double-binary adapter branch (LoRDBA page, section 2 "Core architecture"):
//     dW = sum_i diag(alpha_i) B1 diag(beta_i) B2 diag(gamma_i),
// B1 (N x R) and B2 (R x K) in {-1, +1} stored one bit per entry, alpha_i,
// beta_i, gamma_i fp16 channel scales, served unmerged beside the quantized
// base ("adapter mode", sections 1-2):
//     y = x W'^T + sum_i alpha_i * ((x * gamma_i) B2^T * beta_i) B1^T.
//
// The branch is carried as an exact rank-2lR branch of the form the fused
// forward kernels already take (y += t2 Beff^T with scale 1):
//   t2   (M x 2lR, float32) = [t' | t'],  t'[m][iR + j] = beta_i[j] sum_k sign(B2[j][k]) x[m][k] gamma_i[k]
//   Beff (N x 2lR, bf16)    = [hi(alpha_i[n]) sign(B1[n][j]) | lo(alpha_i[n]) sign(B1[n][j])]
// An fp16 value splits exactly into two bf16 values (hi = nearest bf16, lo =
// the remainder, at most 4 significant bits), so Beff holds alpha exactly and
// t2 Beff^T = sum t' (hi + lo) sign = sum t' alpha sign.
#include <algorithm>

#include "qlr_internal.h"

namespace qlr {

namespace {

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// (hi, lo) bf16 bits of an fp16 value v: hi = round-to-nearest-even bf16(v), lo = bf16(v - hi) (exact)
__device__ __forceinline__ void split_f16(float v, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

// Beff[n][jj] for jj < lR: hi(alpha_i[n]) sign(B1[n][j]), jj = iR + j; Beff[n][lR + jj]: the lo part.
__global__ __launch_bounds__(256) void k_dba_beff(DbaArgs d, int64_t N, uint16_t* __restrict__ beff) {
  const int lr = d.ell * d.R;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= N * lr) return;
  const int64_t n = idx / lr;
  const int jj = (int)(idx % lr), i = jj / d.R, j = jj % d.R;
  const int w1 = (d.R + 31) / 32;
  const uint32_t bit = (d.b1[n * w1 + (j >> 5)] >> (j & 31)) & 1u;
  uint32_t hi, lo;
  split_f16(half_bits_to_f32(d.alpha[(int64_t)i * N + n]), hi, lo);
  const uint32_t flip = bit ? 0u : 0x8000u;
  beff[n * 2 * lr + jj] = (uint16_t)(hi ^ flip);
  beff[n * 2 * lr + lr + jj] = (uint16_t)(lo ^ flip);
}

// t' for bf16 x on 16x16x32 bf16 MFMA, float32 accumulation.  blockIdx.x: 16
// rows of x; blockIdx.y: (i, 16 adapter rows j); blockIdx.z: K split.  The 4
// waves share the split's 32-wide K steps and are added through LDS.  Per step
// a lane reads 8 elements of its x row (A operand) and builds its B operand,
// sign(B2[j][k]) gamma_i[k] for 8 k, as two exact bf16 halves (the sign applied
// by flipping sign bits), multiplied in two MFMAs into one accumulator.
__global__ __launch_bounds__(256) void k_dba_t_mfma(DbaArgs d, const uint16_t* __restrict__ x, int64_t M,
                                                    int64_t K, float* __restrict__ t2) {
  __shared__ float sRed[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, g = lane >> 4;
  const int rch = (d.R + 15) / 16;
  const int i = blockIdx.y / rch, j0 = 16 * (blockIdx.y % rch);
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int S = gridDim.z, sidx = blockIdx.z;
  const bool xv = m0 + row < M;
  const uint16_t* xp = x + (xv ? m0 + row : 0) * K + 8 * g;
  const int j = j0 + row;
  const bool jv = j < d.R;
  const int64_t w2 = (K + 31) / 32;
  const uint32_t* bp = d.b2 + (int64_t)(jv ? j : 0) * w2;
  const uint16_t* gp = d.gamma + (int64_t)i * K + 8 * g;
  const int64_t nsteps = K / 32;
  const int64_t c0 = nsteps * sidx / S, c1 = nsteps * (sidx + 1) / S;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll 2
  for (int64_t st = c0 + wave; st < c1; st += 4) {
    const int64_t k = st * 32;
    const u32x4_t xa = xv ? *reinterpret_cast<const u32x4_t*>(xp + k) : zero;
    const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(gp + k);
    const uint32_t bits = (bp[(k + 8 * g) >> 5] >> ((k + 8 * g) & 31)) & 0xFFu;
    u32x4_t bh, bl;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t h0, l0, h1, l1;
      split_f16(half_bits_to_f32(gv[e2] & 0xFFFFu), h0, l0);
      split_f16(half_bits_to_f32(gv[e2] >> 16), h1, l1);
      const uint32_t f0 = ((bits >> (2 * e2)) & 1u) ? 0u : 0x8000u;
      const uint32_t f1 = ((bits >> (2 * e2 + 1)) & 1u) ? 0u : 0x8000u;
      bh[e2] = jv ? ((h0 ^ f0) | ((h1 ^ f1) << 16)) : 0u;
      bl[e2] = jv ? ((l0 ^ f0) | ((l1 ^ f1) << 16)) : 0u;
    }
    acc = mfma16x16x32(as_bf16x8(xa), as_bf16x8(bh), acc);
    acc = mfma16x16x32(as_bf16x8(xa), as_bf16x8(bl), acc);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) sRed[wave][lane * 4 + v] = acc[v];
  __syncthreads();
  const int e = threadIdx.x;
  const float sum = (sRed[0][e] + sRed[1][e]) + (sRed[2][e] + sRed[3][e]);
  const int l = e >> 2, v = e & 3;
  const int64_t m = m0 + 4 * (l >> 4) + v;  // MFMA output row
  const int jo = j0 + (l & 15);             // MFMA output column
  if (m < M && jo < d.R) {
    const int lr = d.ell * d.R;
    const float val = half_bits_to_f32(d.beta[(int64_t)i * d.R + jo]) * sum;
    float* tr = t2 + ((int64_t)sidx * M + m) * 2 * lr;
    tr[i * d.R + jo] = val;
    tr[lr + i * d.R + jo] = val;
  }
}

// t' for float32 x (float32 arithmetic): one wave per (m, i, j), lanes split K.
__global__ __launch_bounds__(256) void k_dba_t_valu(DbaArgs d, const float* __restrict__ x, int64_t M, int64_t K,
                                                    float* __restrict__ t2) {
  const int lane = threadIdx.x & 63;
  const int lr = d.ell * d.R;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= M * lr) return;
  const int64_t m = item / lr;
  const int jj = (int)(item % lr), i = jj / d.R, j = jj % d.R;
  const int64_t w2 = (K + 31) / 32;
  float acc = 0.0f;
  for (int64_t k = lane; k < K; k += 64) {
    const float xg = x[m * K + k] * half_bits_to_f32(d.gamma[(int64_t)i * K + k]);
    acc += ((d.b2[(int64_t)j * w2 + (k >> 5)] >> (k & 31)) & 1u) ? xg : -xg;
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    const float val = half_bits_to_f32(d.beta[(int64_t)i * d.R + j]) * acc;
    t2[m * 2 * lr + jj] = val;
    t2[m * 2 * lr + lr + jj] = val;
  }
}

}  // namespace

int dba_t_splits(int64_t M, int64_t K, int xdt, int R, int ell) {
  // one pass for M > 16 (the prefill kernels read t2 once per tile row; split
  // partials there would be re-added per tile)
  if (xdt != DT_BF16 || M > 16) return 1;
  const int64_t steps = K / 32, mtiles = (M + 15) / 16, ych = (int64_t)ell * ((R + 15) / 16);
  int64_t s = std::min<int64_t>(steps / 4, (256 + mtiles * ych - 1) / (mtiles * ych));
  s = std::min<int64_t>(s, 64);
  return (int)std::max<int64_t>(s, 1);
}

hipError_t launch_dba_prep(const DbaArgs& d, const void* x, int xdt, int64_t M, int64_t N, int64_t K, float* t2,
                           int splits, uint16_t* beff, hipStream_t s) {
  const int64_t lr = (int64_t)d.ell * d.R;
  hipLaunchKernelGGL(k_dba_beff, dim3((unsigned)((N * lr + 255) / 256)), dim3(256), 0, s, d, N, beff);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || M == 0) return e;
  if (xdt == DT_BF16) {
    dim3 grid((unsigned)((M + 15) / 16), (unsigned)(d.ell * ((d.R + 15) / 16)), (unsigned)splits);
    hipLaunchKernelGGL(k_dba_t_mfma, grid, dim3(256), 0, s, d, reinterpret_cast<const uint16_t*>(x), M, K, t2);
  } else {
    if (splits != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_dba_t_valu, dim3((unsigned)((M * lr + 3) / 4)), dim3(256), 0, s, d,
                       reinterpret_cast<const float*>(x), M, K, t2);
  }
  return hipGetLastError();
}

}  // namespace qlr

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
__device__ __forceinline__ void dba_beff_item(const DbaArgs& d, int64_t N, uint16_t* __restrict__ beff, int64_t idx) {
  const int lr = d.ell * d.R;
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

// One launch: workgroups [0, tblocks) compute t' for bf16 x on 16x16x32 bf16
// MFMA (float32 accumulation), the rest expand Beff (one item per thread).
// A t' workgroup owns 16 rows of x, 16 adapter rows j of one term i and one K
// split.  It first splits gamma_i over its K range into bf16 hi and lo halves
// in LDS (once, shared by all its rows and adapter rows); its 16 waves then
// take every 16th 32-wide K step, all of a wave's steps loaded before any is
// multiplied (kDbaSteps at a time), and are added through LDS.  Per step a
// lane takes 8 elements of its x row (A operand; loaded coalesced and moved
// into place by a lane permute) and 8 hi and 8 lo halves of gamma, flips the
// sign bits where B2[j][k] is -1 (B operand) and multiplies both halves into
// one accumulator.
constexpr int kDbaWaves = 16, kDbaSteps = 4;
struct DbaGrid {
  int64_t mtiles, tblocks;
  int rch, splits;
  int64_t kspan;  // largest K range of a split (elements), for the LDS halves
};
__global__ __launch_bounds__(1024) void k_dba_prep(DbaArgs d, DbaGrid gd, const uint16_t* __restrict__ x, int64_t M,
                                                   int64_t N, int64_t K, float* __restrict__ t2,
                                                   uint16_t* __restrict__ beff) {
  __shared__ float sRed[kDbaWaves][256];
  extern __shared__ __attribute__((aligned(16))) char sG[];  // hi halves, then lo halves (kspan each)
  if ((int64_t)blockIdx.x >= gd.tblocks) {
    dba_beff_item(d, N, beff, ((int64_t)blockIdx.x - gd.tblocks) * 1024 + threadIdx.x);
    return;
  }
  const int64_t bid = blockIdx.x;
  const int64_t mt = bid % gd.mtiles, rest = bid / gd.mtiles;
  const int yc = (int)(rest % ((int64_t)d.ell * gd.rch)), sidx = (int)(rest / ((int64_t)d.ell * gd.rch));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, g = lane >> 4;
  const int i = yc / gd.rch, j0 = 16 * (yc % gd.rch);
  const int64_t m0 = mt * 16;
  const int S = gd.splits;
  const bool xv = m0 + row < M;
  // x loads: each quad of lanes one row's 64 bytes of a step (lane l: row l / 4,
  // 8 columns from 8 (l % 4)); a lane permute per word moves row n's piece g to
  // lane 16 g + n, the fragment layout
  const int xrow = lane >> 2;
  const uint16_t* xp = x + (m0 + xrow < M ? m0 + xrow : 0) * K + 8 * (lane & 3);
  const int xsrc = (4 * row + g) << 2;
  const int j = j0 + row;
  const bool jv = j < d.R;
  const int64_t w2 = (K + 31) / 32;
  const uint32_t* bp = d.b2 + (int64_t)(jv ? j : 0) * w2;
  const int64_t nsteps = K / 32;
  const int64_t c0 = nsteps * sidx / S, c1 = nsteps * (sidx + 1) / S;
  const int64_t kb = c0 * 32;
  uint16_t* sGh = reinterpret_cast<uint16_t*>(sG);
  uint16_t* sGl = sGh + gd.kspan;

  u32x4_t xa[kDbaSteps];
  uint32_t bw[kDbaSteps];
  auto load = [&](int64_t sb) {
#pragma unroll
    for (int q = 0; q < kDbaSteps; ++q) {
      const int64_t st = min(sb + (int64_t)q * kDbaWaves, c1 - 1);  // clamped: a valid step
      const int64_t k = st * 32;
      xa[q] = *reinterpret_cast<const u32x4_t*>(xp + k);
      bw[q] = bp[(k + 8 * g) >> 5];
    }
  };
  const int64_t sb0 = c0 + wave;
  if (sb0 < c1) load(sb0);
  // gamma_i over [kb, 32 c1) split into exact bf16 halves, once
  for (int64_t k = kb + threadIdx.x; k < c1 * 32; k += 1024) {
    uint32_t hi, lo;
    split_f16(half_bits_to_f32(d.gamma[(int64_t)i * K + k]), hi, lo);
    sGh[k - kb] = (uint16_t)hi;
    sGl[k - kb] = (uint16_t)lo;
  }
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int64_t sb = sb0; sb < c1; sb += kDbaWaves * kDbaSteps) {
    if (sb != sb0) load(sb);
#pragma unroll
    for (int q = 0; q < kDbaSteps; ++q) {
      const int64_t st = sb + (int64_t)q * kDbaWaves;
      const bool sv = st < c1 && xv;  // wave-uniform st; rows past M add zero
      const int64_t ko = min(st, c1 - 1) * 32 + 8 * g - kb;  // this lane's 8 gamma halves
      const u32x4_t gh = *reinterpret_cast<const u32x4_t*>(sGh + ko);
      const u32x4_t gl = *reinterpret_cast<const u32x4_t*>(sGl + ko);
      // sign masks: bit e of the byte clear -> flip the sign of element e
      const uint32_t nb = ~(bw[q] >> ((st * 32 + 8 * g) & 31));
      u32x4_t bh, bl;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t f = (((nb >> (2 * e2)) & 1u) << 15) | (((nb >> (2 * e2 + 1)) & 1u) << 31);
        bh[e2] = jv ? (gh[e2] ^ f) : 0u;
        bl[e2] = jv ? (gl[e2] ^ f) : 0u;
      }
      u32x4_t xf;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) xf[e2] = (uint32_t)__builtin_amdgcn_ds_bpermute(xsrc, (int)xa[q][e2]);
      const u32x4_t xq = sv ? xf : zero;
      acc = mfma16x16x32(as_bf16x8(xq), as_bf16x8(bh), acc);
      acc = mfma16x16x32(as_bf16x8(xq), as_bf16x8(bl), acc);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) sRed[wave][lane * 4 + v] = acc[v];
  __syncthreads();
  if (threadIdx.x >= 256) return;
  const int e = threadIdx.x;
  float sum = 0.0f;
#pragma unroll
  for (int w = 0; w < kDbaWaves; ++w) sum += sRed[w][e];
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

__global__ __launch_bounds__(256) void k_dba_beff(DbaArgs d, int64_t N, uint16_t* __restrict__ beff) {
  dba_beff_item(d, N, beff, (int64_t)blockIdx.x * 256 + threadIdx.x);
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
  // enough workgroups for the chip; at M > 16 at most 4 splits (the prefill
  // kernels re-add the split partials of every tile row they read)
  if (xdt != DT_BF16) return 1;
  const int64_t steps = K / 32, mtiles = (M + 15) / 16, ych = (int64_t)ell * ((R + 15) / 16);
  int64_t s = std::min<int64_t>(steps / kDbaWaves, (256 + mtiles * ych - 1) / (mtiles * ych));
  s = std::min<int64_t>(s, M > 16 ? 4 : 64);
  return (int)std::max<int64_t>(s, 1);
}

hipError_t launch_dba_prep(const DbaArgs& d, const void* x, int xdt, int64_t M, int64_t N, int64_t K, float* t2,
                           int splits, uint16_t* beff, hipStream_t s) {
  const int64_t lr = (int64_t)d.ell * d.R;
  if (xdt == DT_BF16 && M > 0) {
    DbaGrid gd;
    gd.mtiles = (M + 15) / 16;
    gd.rch = (d.R + 15) / 16;
    gd.splits = splits;
    gd.tblocks = gd.mtiles * d.ell * gd.rch * splits;
    const int64_t nsteps = K / 32;
    gd.kspan = 32 * ((nsteps + splits - 1) / splits + 1);
    const size_t shmem = (size_t)gd.kspan * 4;
    if (shmem > 96 * 1024) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_dba_prep),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
      if (e != hipSuccess) return e;
      attr = true;
    }
    const int64_t eblocks = (N * lr + 1023) / 1024;
    hipLaunchKernelGGL(k_dba_prep, dim3((unsigned)(gd.tblocks + eblocks)), dim3(1024), shmem, s, d, gd,
                       reinterpret_cast<const uint16_t*>(x), M, N, K, t2, beff);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_dba_beff, dim3((unsigned)((N * lr + 255) / 256)), dim3(256), 0, s, d, N, beff);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || M == 0) return e;
  if (splits != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dba_t_valu, dim3((unsigned)((M * lr + 3) / 4)), dim3(256), 0, s, d,
                     reinterpret_cast<const float*>(x), M, K, t2);
  return hipGetLastError();
}

}  // namespace qlr

// Backward of the layer for adapter training: the input gradient through the
// frozen quantized base, and the gradients of the adapter.
//
// QLoRA page, memory-decomposition equation: the 4-bit base stays frozen while
// the bf16 adapters are trained; AutoQRA page, "1. Problem statement": the
// quantized backbone is frozen and lightweight adapters are fine-tuned.  For
// y = x W'^T + s (x A^T) B^T and an upstream gradient dy (M x N), with
// u = dy B and t = x A^T (M x r each):
//     dx = dy W' + s u A     (M x K)
//     dA = s u^T x           (r x K)
//     dB = s dy^T t          (N x r)
// This file holds the helpers of that backward; the bf16 input gradient runs on
// the transposed dequantizing GEMM (k_gemm with TR), u and t on the
// adapter-product kernels.
#include <algorithm>

#include "qlr_internal.h"

namespace qlr {

namespace {

// Bt[j][n] = B[n][j]: B (N x r) as r x N, so that u = dy B is the adapter
// product dy Bt^T.  Writes are coalesced along n.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_nr(const T* __restrict__ B, int64_t N, int r,
                                                      T* __restrict__ Bt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N * r) return;
  const int64_t j = i / N, n = i % N;
  Bt[i] = B[n * r + j];
}

// ---------------------------------------------------------------- dA and dB
//
// Both are rank-r contractions over the M rows: out[j][c] = s sum_m P[m][j] Q[m][c]
// with (P, Q, C) = (u, x, K) for dA (stored r x K) and (t, dy, N) for dB (stored
// N x r, "column-major" in this indexing).  float32 arithmetic.
//
// A workgroup owns 256 columns (4 per lane, one 8- or 16-byte load per row) x
// 16 adapter rows x one range of M.  Its P rows (sum of the partial splits) are
// staged in LDS and read as broadcasts; each wave takes a quarter of the rows in
// batches of 8 (8 loads in flight per lane) and the 4 waves are added through
// LDS in wave order.  With several M ranges the range sums go to float32
// partials that a second kernel adds in range order; the result does not depend
// on timing.
constexpr int kGradBatch = 8;
struct GradJob {
  const float* P;  // p_splits x M x r float32 partials (u or t)
  const void* Q;   // M x C (x or dy)
  float* part;     // msplit x r x C (msplit > 1)
  float* out;      // r x C, or C x r when cols_major
  int64_t C;
  int32_t p_splits, cols_major, ctiles;
  int64_t tile0;
};
struct GradParams {
  int64_t M, rows;  // rows of one M range (a multiple of 32)
  int32_t r, jchunks, msplit, nj;
  float scale;
  GradJob J[2];
};

template <int QDT>
__global__ __launch_bounds__(256) void k_lora_grad(GradParams G) {
  __shared__ float red[3 * 64 * 64];
  extern __shared__ f32x4_t sP[];  // rows x 4 (16 adapter rows per staged row)
  const int ji = (G.nj > 1 && (int64_t)blockIdx.x >= G.J[1].tile0) ? 1 : 0;
  const GradJob& J = G.J[ji];
  const int64_t lt = (int64_t)blockIdx.x - J.tile0;
  const int64_t ct = lt % J.ctiles, rest = lt / J.ctiles;
  const int jc = (int)(rest % G.jchunks), z = (int)(rest / G.jchunks);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t M = G.M, C = J.C;
  const int r = G.r, j0 = 16 * jc;
  const int64_t mb = (int64_t)z * G.rows, me = min(M, mb + G.rows);
  const int64_t c0 = ct * 256 + 4 * lane;

  // stage P rows [mb, me), adapter rows [j0, j0 + 16), zero past r
  for (int64_t idx = threadIdx.x; idx < (me - mb) * 16; idx += 256) {
    const int64_t m = mb + idx / 16;
    const int j = j0 + (int)(idx % 16);
    float v = 0.0f;
    if (j < r)
      for (int sp = 0; sp < J.p_splits; ++sp) v += J.P[((int64_t)sp * M + m) * r + j];
    reinterpret_cast<float*>(sP)[idx] = v;
  }
  __syncthreads();

  float acc[16][4];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[jj][e] = 0.0f;

  const bool vec = (C % 4) == 0 && c0 + 4 <= C;
  const int64_t rw = G.rows / 4;  // rows of one wave (a multiple of 8)
  const int64_t wb = mb + w * rw, we = min(me, wb + rw);
  for (int64_t m = wb; m < we; m += kGradBatch) {
    float q[kGradBatch][4];
#pragma unroll
    for (int b = 0; b < kGradBatch; ++b) {
      const int64_t mm = m + b;
      const bool mv = mm < we;
      const int64_t base = (mv ? mm : wb) * C + c0;
      if (vec) {
        if constexpr (QDT == DT_F32) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(J.Q) + base);
#pragma unroll
          for (int e = 0; e < 4; ++e) q[b][e] = mv ? v[e] : 0.0f;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(J.Q) + base);
          q[b][0] = mv ? bf16_bits_to_f32(v.x & 0xFFFFu) : 0.0f;
          q[b][1] = mv ? bf16_bits_to_f32(v.x >> 16) : 0.0f;
          q[b][2] = mv ? bf16_bits_to_f32(v.y & 0xFFFFu) : 0.0f;
          q[b][3] = mv ? bf16_bits_to_f32(v.y >> 16) : 0.0f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) q[b][e] = (mv && c0 + e < C) ? load_elem<QDT>(J.Q, base + e) : 0.0f;
      }
    }
#pragma unroll
    for (int b = 0; b < kGradBatch; ++b) {
      const int64_t row = min(m + b, we - 1) - mb;  // rows past we carry q = 0
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4_t p = sP[row * 4 + j4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * j4 + jj][e] = fmaf(p[jj], q[b][e], acc[4 * j4 + jj][e]);
      }
    }
  }

  // add the waves in order 0, 1, 2, 3
  if (w > 0) {
#pragma unroll
    for (int v = 0; v < 64; ++v) red[((w - 1) * 64 + v) * 64 + lane] = acc[v >> 2][v & 3];
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    float s = acc[v >> 2][v & 3];
    s += red[(0 * 64 + v) * 64 + lane];
    s += red[(1 * 64 + v) * 64 + lane];
    s += red[(2 * 64 + v) * 64 + lane];
    acc[v >> 2][v & 3] = s;
  }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = j0 + jj;
    if (j >= r) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = c0 + e;
      if (c >= C) break;
      if (G.msplit > 1) J.part[((int64_t)z * r + j) * C + c] = acc[jj][e];
      else if (J.cols_major) J.out[c * r + j] = G.scale * acc[jj][e];
      else J.out[(int64_t)j * C + c] = G.scale * acc[jj][e];
    }
  }
}

// out = s * (sum over the M ranges, in range order) of the partials.
__global__ __launch_bounds__(256) void k_lora_grad_reduce(GradParams G) {
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n0 = (int64_t)G.r * G.J[0].C;
  const int ji = (G.nj > 1 && i0 >= n0) ? 1 : 0;
  const GradJob& J = G.J[ji];
  const int64_t i = ji ? i0 - n0 : i0;
  if (i >= (int64_t)G.r * J.C) return;
  const int64_t j = i / J.C, c = i % J.C;
  float s = 0.0f;
  for (int z = 0; z < G.msplit; ++z) s += J.part[((int64_t)z * G.r + j) * J.C + c];
  if (J.cols_major) J.out[c * G.r + j] = G.scale * s;
  else J.out[j * J.C + c] = G.scale * s;
}

__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ---------------------------------------------------------------- float32 dx
//
// dx[m][k] = sum_n dy[m][n] w'[n][k] + s sum_j u[m][j] A[j][k], float32 FMA in
// n order, w' formed exactly as dequantization defines it.  One thread per
// column k, 8 rows of dy per workgroup (dy and u are read with uniform loads).
template <int BITS, int GDT, int ADT, int ODT>
__global__ __launch_bounds__(256) void k_bwd_dx_f32(LinearArgs a, Levels lv) {
  constexpr int NL = 1 << BITS;
  __shared__ float sL[NL];
  stage_levels<NL>(lv, sL);
  __syncthreads();
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= a.K) return;
  const int64_t N = a.N, K = a.K, M = a.M, nbK = K / 64, kb = k >> 6;
  const int e = (int)(k & 63);
  const int bit0 = BITS * e, byte0 = bit0 >> 3, sh = bit0 & 7;
  const int64_t m0 = (int64_t)blockIdx.y * 8;
  float acc[8] = {};
  for (int64_t n = 0; n < N; ++n) {
    const int64_t blk = n * nbK + kb;
    const uint8_t* cb = a.codes + blk * (8 * BITS);
    uint32_t two = cb[byte0];
    if (byte0 + 1 < 8 * BITS) two |= (uint32_t)cb[byte0 + 1] << 8;
    const int c = (int)((two >> sh) & (NL - 1));
    const float ap = (float)a.q8[blk] * a.cst[blk >> 8];
    const float w = sL[c] * ap;
#pragma unroll
    for (int mm = 0; mm < 8; ++mm)
      if (m0 + mm < M) acc[mm] = fmaf(load_elem<GDT>(a.x, (m0 + mm) * N + n), w, acc[mm]);
  }
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const int64_t m = m0 + mm;
    if (m >= M) break;
    float lo = 0.0f;
    for (int j = 0; j < a.r; ++j) {
      float uj = 0.0f;
      for (int sp = 0; sp < a.t_splits; ++sp) uj += a.t[((int64_t)sp * M + m) * a.r + j];
      lo = fmaf(uj, load_elem<ADT>(a.B, (int64_t)j * K + k), lo);
    }
    const float out = fmaf(a.scale, lo, acc[mm]);
    if constexpr (ODT == DT_F32) reinterpret_cast<float*>(a.y)[m * K + k] = out;
    else reinterpret_cast<uint16_t*>(a.y)[m * K + k] = (uint16_t)f32_to_bf16_bits(out);
  }
}

template <int BITS, int GDT, int ADT>
hipError_t launch_dx_f32_3(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  dim3 grid((unsigned)((a.K + 255) / 256), (unsigned)((a.M + 7) / 8)), block(256);
  if (a.ydt == DT_F32) hipLaunchKernelGGL((k_bwd_dx_f32<BITS, GDT, ADT, DT_F32>), grid, block, 0, s, a, lv);
  else hipLaunchKernelGGL((k_bwd_dx_f32<BITS, GDT, ADT, DT_BF16>), grid, block, 0, s, a, lv);
  return hipGetLastError();
}
template <int BITS, int GDT>
hipError_t launch_dx_f32_2(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.abdt == DT_F32) return launch_dx_f32_3<BITS, GDT, DT_F32>(a, lv, s);
  return launch_dx_f32_3<BITS, GDT, DT_BF16>(a, lv, s);
}
template <int BITS>
hipError_t launch_dx_f32_1(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.xdt == DT_F32) return launch_dx_f32_2<BITS, DT_F32>(a, lv, s);
  return launch_dx_f32_2<BITS, DT_BF16>(a, lv, s);
}

}  // namespace

hipError_t launch_transpose_nr(const void* B, int dt, int64_t N, int r, void* Bt, hipStream_t s) {
  const int64_t n = N * r;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dt == DT_F32)
    hipLaunchKernelGGL(k_transpose_nr<float>, grid, dim3(256), 0, s, reinterpret_cast<const float*>(B), N, r,
                       reinterpret_cast<float*>(Bt));
  else
    hipLaunchKernelGGL(k_transpose_nr<uint16_t>, grid, dim3(256), 0, s, reinterpret_cast<const uint16_t*>(B), N,
                       r, reinterpret_cast<uint16_t*>(Bt));
  return hipGetLastError();
}

hipError_t launch_dx_f32(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  switch (a.bits) {
    case 2: return launch_dx_f32_1<2>(a, lv, s);
    case 3: return launch_dx_f32_1<3>(a, lv, s);
    case 4: return launch_dx_f32_1<4>(a, lv, s);
    default: return launch_dx_f32_1<8>(a, lv, s);
  }
}

// M ranges of the adapter-gradient kernel: enough workgroups to fill the chip,
// ranges of whole 32-row multiples, at most kGradRowsMax rows (their staged P
// rows take 64 bytes each of LDS).
constexpr int64_t kGradRowsMax = 1024;
void grad_split(int64_t M, int64_t N, int64_t K, int r, int* msplit, int64_t* rows) {
  const int64_t tiles = ((K + 255) / 256 + (N + 255) / 256) * ((r + 15) / 16);
  const int64_t max_split = std::max<int64_t>(1, (M + 127) / 128);
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(max_split, (512 + tiles - 1) / tiles));
  int64_t rw = (M + want - 1) / want;
  rw = std::max<int64_t>(32, (rw + 31) / 32 * 32);
  rw = std::min(rw, kGradRowsMax);
  *rows = rw;
  *msplit = (int)std::max<int64_t>(1, (M + rw - 1) / rw);
}

size_t grad_partial_floats(int64_t M, int64_t N, int64_t K, int r) {
  int ms;
  int64_t rows;
  grad_split(M, N, K, r, &ms, &rows);
  return ms > 1 ? (size_t)ms * (size_t)r * (size_t)(N + K) : 0;
}

hipError_t launch_lora_grads(const float* u, int u_splits, const float* t, int t_splits, const void* x,
                             const void* dy, int qdt, int64_t M, int64_t N, int64_t K, int r, float scale,
                             float* dA, float* dB, float* part, hipStream_t s) {
  if (r == 0) return hipSuccess;
  if (M == 0) {
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((r * K + 255) / 256)), dim3(256), 0, s, dA, (int64_t)r * K);
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((r * N + 255) / 256)), dim3(256), 0, s, dB, (int64_t)r * N);
    return hipGetLastError();
  }
  GradParams G;
  G.M = M;
  G.r = r;
  G.jchunks = (r + 15) / 16;
  grad_split(M, N, K, r, &G.msplit, &G.rows);
  G.scale = scale;
  G.nj = 2;
  GradJob& a = G.J[0];
  a.P = u;
  a.p_splits = u_splits;
  a.Q = x;
  a.C = K;
  a.part = part;
  a.out = dA;
  a.cols_major = 0;
  a.ctiles = (int32_t)((K + 255) / 256);
  a.tile0 = 0;
  GradJob& b = G.J[1];
  b.P = t;
  b.p_splits = t_splits;
  b.Q = dy;
  b.C = N;
  b.part = part + (G.msplit > 1 ? (size_t)G.msplit * r * K : 0);
  b.out = dB;
  b.cols_major = 1;
  b.ctiles = (int32_t)((N + 255) / 256);
  b.tile0 = (int64_t)a.ctiles * G.jchunks * G.msplit;
  const int64_t tiles = b.tile0 + (int64_t)b.ctiles * G.jchunks * G.msplit;
  const size_t shmem = (size_t)G.rows * 16 * sizeof(float);
  if (shmem > (size_t)kGradRowsMax * 64) return hipErrorInvalidValue;
  if (qdt == DT_F32) {
    static bool attr = false;
    if (!attr) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_lora_grad<DT_F32>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kGradRowsMax * 64));
      if (e != hipSuccess) return e;
      attr = true;
    }
    hipLaunchKernelGGL(k_lora_grad<DT_F32>, dim3((unsigned)tiles), dim3(256), shmem, s, G);
  } else {
    static bool attr = false;
    if (!attr) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_lora_grad<DT_BF16>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kGradRowsMax * 64));
      if (e != hipSuccess) return e;
      attr = true;
    }
    hipLaunchKernelGGL(k_lora_grad<DT_BF16>, dim3((unsigned)tiles), dim3(256), shmem, s, G);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || G.msplit == 1) return e;
  const int64_t outs = (int64_t)r * (K + N);
  hipLaunchKernelGGL(k_lora_grad_reduce, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, G);
  return hipGetLastError();
}

}  // namespace qlr

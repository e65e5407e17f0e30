// Walsh-Hadamard adapter branch (QWHA page, section 2.1 "Adapter design:
// Walsh-Hadamard adaptation"): dW = F H^-1 with H the +-1 Walsh-Hadamard matrix
// and F sparse (values c at an index list).  H is symmetric and H^-1 = H / P, so
// x dW^T = z F^T with z = x blockdiag(H_P) / P: a fast transform of each x row
// (additions and subtractions only) and a sparse product.
//
// One kernel forms C = z F^T (float32, M x N), which the forward kernels add to
// every output before rounding.  A workgroup stages MR rows of x in LDS as
// float32 column records (MR values of one column together), transforms them
// in place within blocks of P columns, and then walks the coefficients of a
// range of F's rows: G lanes per row, each taking every G-th coefficient in
// rounds of 8 (all loads of a round in flight together), summed over the G
// lanes in a fixed butterfly order.
#include <algorithm>

#include "qlr_internal.h"

namespace qlr {

namespace {

constexpr int64_t kWhaLds = 128 * 1024;     // the staged x records at most
constexpr int64_t kWhaLdsAll = 160 * 1024;  // records, the row order and the class counters

// LDS slot of column c's record: its low 3 bits XORed with bits 3..5, so the 8
// consecutive records a thread stages, and its neighbours', spread over the banks
__device__ __forceinline__ int64_t wslot(int64_t c) { return (c & ~int64_t(7)) | ((c & 7) ^ ((c >> 3) & 7)); }

template <int MR>
struct Rec {
  float v[MR];
};

template <int MR>
__device__ __forceinline__ Rec<MR> rec_load(const float* z, int64_t c) {
  Rec<MR> r;
  const float* p = z + wslot(c) * MR;
  if constexpr (MR % 4 == 0) {
#pragma unroll
    for (int q = 0; q < MR / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(p)[q];
      r.v[4 * q] = v.x;
      r.v[4 * q + 1] = v.y;
      r.v[4 * q + 2] = v.z;
      r.v[4 * q + 3] = v.w;
    }
  } else if constexpr (MR == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    r.v[0] = v.x;
    r.v[1] = v.y;
  } else {
    r.v[0] = *p;
  }
  return r;
}

template <int MR>
__device__ __forceinline__ void rec_store(float* z, int64_t c, const Rec<MR>& r) {
  float* p = z + wslot(c) * MR;
  if constexpr (MR % 4 == 0) {
#pragma unroll
    for (int q = 0; q < MR / 4; ++q)
      reinterpret_cast<float4*>(p)[q] = make_float4(r.v[4 * q], r.v[4 * q + 1], r.v[4 * q + 2], r.v[4 * q + 3]);
  } else if constexpr (MR == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(r.v[0], r.v[1]);
  } else {
    *p = r.v[0];
  }
}

// blockIdx.x: x rows [MR bx, MR bx + MR); blockIdx.y: F rows [nchunk by, ...).
// TB threads; G lanes per F row, lane g taking the row's coefficients
// g + G u (u < 8) of each round, so a round covers 8 G consecutive ones; each
// lane walks RB rows per pass, and the next pass's row offsets are loaded
// while the current pass's coefficients are in flight.
template <int XDT, int MR, int G, int RB, int TB>
__global__ __launch_bounds__(TB) void k_wha_addend(const void* __restrict__ x, int64_t M, int64_t K, int64_t N,
                                                    int lp, const int32_t* __restrict__ row_ptr,
                                                    const int32_t* __restrict__ col, const float* __restrict__ val,
                                                    int64_t nnz, float* __restrict__ C, int64_t nchunk) {
  extern __shared__ float4 wha_smem[];
  float* z = reinterpret_cast<float*>(wha_smem);
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * MR;

  // 1. stage: chunk q = columns 8 q .. 8 q + 7 of each of the MR rows (16-byte loads)
  for (int64_t q = tid; q < K / 8; q += TB) {
    float v[MR][8];
#pragma unroll
    for (int mm = 0; mm < MR; ++mm) {
      const bool mv = m0 + mm < M;
      const int64_t m = mv ? m0 + mm : M - 1;
      if constexpr (XDT == DT_F32) {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + m * K + 8 * q);
        const float4 a = p[0], b = p[1];
        const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[mm][i] = mv ? e[i] : 0.0f;
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + m * K + 8 * q);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[mm][i] = mv ? bf16_bits_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      Rec<MR> r;
#pragma unroll
      for (int mm = 0; mm < MR; ++mm) r.v[mm] = v[mm][i];
      rec_store<MR>(z, 8 * q + i, r);
    }
  }
  __syncthreads();

  // 2. the transform within blocks of 2^lp columns, up to 3 bits of the column
  // index per round: a task is the 8 (4, 2) columns that differ only in bits
  // b .. b + nbit - 1, loaded, combined by butterflies in registers, stored back
  for (int b = 0; b < lp; b += 3) {
    const int nbit = min(3, lp - b);
    const int R = 1 << nbit;
    const int64_t h = int64_t(1) << b;
    const int64_t tasks = K >> nbit;
    for (int64_t t = tid; t < tasks; t += TB) {
      const int64_t c0 = ((t >> b) << (b + nbit)) | (t & (h - 1));
      Rec<MR> r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < R) r[j] = rec_load<MR>(z, c0 + j * h);
#pragma unroll
      for (int s = 1; s < 8; s <<= 1) {
        if (s < R) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (j < R && !(j & s)) {
#pragma unroll
              for (int mm = 0; mm < MR; ++mm) {
                const float a = r[j].v[mm], c = r[j + s].v[mm];
                r[j].v[mm] = a + c;
                r[j + s].v[mm] = a - c;
              }
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < R) rec_store<MR>(z, c0 + j * h, r[j]);
    }
    __syncthreads();
  }

  // 3. the sparse product over the transformed rows
  const float inv_p = 1.0f / (float)(int64_t(1) << lp);  // exact: a power of two
  const int g = tid % G;
  constexpr int kE = 8;                       // coefficients per lane per round
  constexpr int kRowsPass = (TB / G) * RB;
  const int64_t nb = (int64_t)blockIdx.y * nchunk, ne = min(N, nb + nchunk), nrows = ne - nb;
  if (nrows <= 0) return;  // uniform
  // Rows are taken in order of their round count (a counting sort into perm,
  // after the records), so that a pass's rows need about as many rounds each
  // and no pass waits on one long row.  The order within a count class comes
  // from LDS atomics; it decides only which rows share a pass, not any sum.
  constexpr int kCls = 16;
  __shared__ uint32_t cls_n[kCls], cls_at[kCls];
  int32_t* perm = reinterpret_cast<int32_t*>(z + (size_t)MR * K);
  auto row_len = [&](int64_t q) {
    const int64_t a0 = min<int64_t>(max<int64_t>(row_ptr[nb + q], 0), nnz);
    return max<int64_t>(a0, min<int64_t>(row_ptr[nb + q + 1], nnz)) - a0;
  };
  auto cls_of = [&](int64_t len) { return (int)min<int64_t>(kCls - 1, (len + kE * G - 1) / (kE * G)); };
  if (tid < kCls) cls_n[tid] = 0;
  __syncthreads();
  for (int64_t q = tid; q < nrows; q += TB) atomicAdd(&cls_n[cls_of(row_len(q))], 1u);
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int c = 0; c < kCls; ++c) {
      cls_at[c] = acc;
      acc += cls_n[c];
    }
  }
  __syncthreads();
  for (int64_t q = tid; q < nrows; q += TB) perm[atomicAdd(&cls_at[cls_of(row_len(q))], 1u)] = (int32_t)q;
  __syncthreads();
  // row offsets of a pass (position i of perm), clamped into range: a malformed
  // CSR gives wrong sums, never a stray access
  auto row_at = [&](int64_t i) { return nb + perm[i < nrows ? i : nrows - 1]; };
  auto offsets = [&](int64_t base, int64_t (&q0)[RB], int64_t (&q1)[RB]) {
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int64_t i = base + tid / G + (TB / G) * u;
      const int64_t nc = row_at(i);
      q0[u] = i < nrows ? min<int64_t>(max<int64_t>(row_ptr[nc], 0), nnz) : 0;
      q1[u] = i < nrows ? max<int64_t>(q0[u], min<int64_t>(row_ptr[nc + 1], nnz)) : 0;
    }
  };
  int64_t p0[RB], p1[RB];
  offsets(0, p0, p1);
  for (int64_t base = 0; base < nrows; base += kRowsPass) {
    int64_t n0[RB], n1[RB];
    offsets(base + kRowsPass, n0, n1);  // the next pass's (past ne: empty)
    float acc[RB][MR];
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int mm = 0; mm < MR; ++mm) acc[u][mm] = 0.0f;
    for (int64_t e0 = 0;; e0 += kE * G) {
      bool more = false;
#pragma unroll
      for (int u = 0; u < RB; ++u) more |= p0[u] + e0 + g < p1[u];
      if (!more) break;
      int32_t cc[RB][kE];
      float vv[RB][kE];
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int64_t j = p0[u] + e0 + g + (int64_t)G * e;
          const int64_t jc = j < nnz ? j : nnz - 1;
          cc[u][e] = min<int32_t>(max<int32_t>(col[jc], 0), (int32_t)(K - 1));
          vv[u][e] = val[jc];
        }
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          if (p0[u] + e0 + g + (int64_t)G * e < p1[u]) {
            const Rec<MR> r = rec_load<MR>(z, cc[u][e]);
#pragma unroll
            for (int mm = 0; mm < MR; ++mm) acc[u][mm] = fmaf(vv[u][e], r.v[mm], acc[u][mm]);
          }
        }
    }
    // sum over the row's G lanes (adjacent lanes of one wave), fixed order
#pragma unroll
    for (int o = 1; o < G; o <<= 1)
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int mm = 0; mm < MR; ++mm) acc[u][mm] += __shfl_xor(acc[u][mm], o, 64);
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int64_t i = base + tid / G + (TB / G) * u;
      if (g == 0 && i < nrows) {
        const int64_t n = row_at(i);
#pragma unroll
        for (int mm = 0; mm < MR; ++mm)
          if (m0 + mm < M) C[(m0 + mm) * N + n] = acc[u][mm] * inv_p;
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      p0[u] = n0[u];
      p1[u] = n1[u];
    }
  }
}

template <int XDT, int MR, int G, int RB, int TB>
hipError_t wha_t(const void* x, int64_t M, int64_t K, int64_t N, int lp, const int32_t* row_ptr, const int32_t* col,
                 const float* val, int64_t nnz, float* C, hipStream_t s) {
  const int64_t xblocks = (M + MR - 1) / MR;
  constexpr int64_t kRowsPass = (TB / G) * RB;
  // enough workgroups to fill the chip (each stages and transforms its x rows
  // once), and row ranges short enough for their order (int32 each) beside the records
  const int64_t rec = (int64_t)MR * K * 4;
  const int64_t max_rows = (kWhaLdsAll - 256 - rec) / 4;
  int64_t nch = std::max<int64_t>(1, std::min<int64_t>((N + kRowsPass - 1) / kRowsPass, (256 + xblocks - 1) / xblocks));
  nch = std::max<int64_t>(nch, (N + max_rows - 1) / max_rows);
  const int64_t nchunk = (N + nch - 1) / nch;
  const size_t shmem = (size_t)rec + (size_t)nchunk * 4;
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_wha_addend<XDT, MR, G, RB, TB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kWhaLdsAll - 256));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_wha_addend<XDT, MR, G, RB, TB>), dim3((unsigned)xblocks, (unsigned)nch), dim3(TB), shmem, s, x,
                     M, K, N, lp, row_ptr, col, val, nnz, C, nchunk);
  return hipGetLastError();
}

template <int XDT>
hipError_t wha_x(const void* x, int64_t M, int64_t K, int64_t N, int lp, const int32_t* row_ptr, const int32_t* col,
                 const float* val, int64_t nnz, float* C, hipStream_t s) {
  if (M >= 8 && 8 * K * 4 <= kWhaLds) return wha_t<XDT, 8, 4, 1, 1024>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  if (M >= 4 && 4 * K * 4 <= kWhaLds) return wha_t<XDT, 4, 4, 1, 1024>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  if (M >= 2 && 2 * K * 4 <= kWhaLds) return wha_t<XDT, 2, 4, 1, 1024>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  return wha_t<XDT, 1, 4, 1, 1024>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
}

}  // namespace

int64_t wha_max_cols() { return kWhaLds / 4; }

hipError_t launch_wha_addend(const void* x, int xdt, int64_t M, int64_t K, int64_t N, int lp, const int32_t* row_ptr,
                             const int32_t* col, const float* val, int64_t nnz, float* C, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K > wha_max_cols() || K % 8 != 0) return hipErrorInvalidValue;
  if (xdt == DT_F32) return wha_x<DT_F32>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  return wha_x<DT_BF16>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
}

}  // namespace qlr

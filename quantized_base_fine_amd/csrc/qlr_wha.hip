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
// range of F's rows: G lanes per row, each taking 8 of every 8 G coefficients
// per round (all loads of a round in flight together), summed over the G lanes
// in a fixed butterfly order.
//
// For the prefill GEMM a second kernel forms instead the weight with the branch
// merged into it, Wd = bf16(W' + F blockdiag(H_P) / P) (bf16, N x K), which the
// dense-weight GEMM multiplies: row n of F H / P is the transform of F's row n
// (its coefficients scattered into a zero row), so the branch costs one pass
// over the weight instead of a gather per x row and coefficient.
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
// TB threads; G lanes per F row, and a round covers 8 G consecutive
// coefficients of the row.  VL: lane g takes 4 g + {0..3} and 4 (g + G) +
// {0..3}, two 16-byte loads each of col and val, so the G lanes of a row read
// 16 G contiguous bytes per load (needs 4 <= nnz < 2^29); otherwise lane g
// takes g + G u (u < 8), one 4-byte load each.  Each lane walks RB rows per
// pass, and the next pass's row offsets are loaded while the current pass's
// coefficients are in flight.
template <int XDT, int MR, int G, int RB, int TB, bool VL>
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
      // both loads unconditional (nc is in range) and their values used
      // unconditionally: a load behind a branch would make the compiler wait
      // for every load in flight.  Past the range the pass gets [lo, lo).
      const int64_t a0 = row_ptr[nc], a1 = row_ptr[nc + 1];
      const int64_t lo = a0 < 0 ? 0 : (a0 > nnz ? nnz : a0);
      const int64_t hi = a1 < lo ? lo : (a1 > nnz ? nnz : a1);
      q0[u] = lo;
      q1[u] = i < nrows ? hi : lo;
    }
  };
  // VL: col and val as buffer resources (loads past the end read zero)
  const int nbytes = VL ? (int)(nnz * 4) : 0;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(col), (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(val), (short)0, nbytes, 0x00020000);
  // One round of a lane: its kE coefficients of each of its RB rows from offset
  // e0 of rows [q, qe), and which of them exist (bit u kE + e).
  struct Round {
    int32_t cc[RB][kE];
    float vv[RB][kE];
    uint32_t ok;
  };
  auto first = [&](int64_t q, int64_t e0) { return VL ? q + e0 + 4 * g : q + e0 + g; };
  auto load_round = [&](const int64_t (&q)[RB], const int64_t (&qe)[RB], int64_t e0, Round& R) {
    R.ok = 0;
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if constexpr (VL) {
        // a load that would run past nnz starts at nnz - 4 instead; its element
        // t then sits at js + t, and those before j belong to another lane
#pragma unroll
        for (int hh = 0; hh < kE / 4; ++hh) {
          const int64_t j = q[u] + e0 + 4 * (g + G * hh);
          const int64_t js = j < nnz - 4 ? j : nnz - 4;
          const u32x4_t lc = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, (int)(js * 4), 0, 0));
          const u32x4_t lv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)(js * 4), 0, 0));
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            R.cc[u][4 * hh + t] = min<int32_t>(max<int32_t>((int32_t)lc[t], 0), (int32_t)(K - 1));
            R.vv[u][4 * hh + t] = __uint_as_float(lv[t]);
            R.ok |= (js + t >= j && js + t < qe[u]) ? 1u << (u * kE + 4 * hh + t) : 0u;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int64_t j = q[u] + e0 + g + (int64_t)G * e;
          const int64_t jc = j < nnz ? j : (nnz > 0 ? nnz - 1 : 0);
          R.cc[u][e] = nnz > 0 ? min<int32_t>(max<int32_t>(col[jc], 0), (int32_t)(K - 1)) : 0;
          R.vv[u][e] = nnz > 0 ? val[jc] : 0.0f;
          R.ok |= j < qe[u] ? 1u << (u * kE + e) : 0u;
        }
      }
    }
  };
  // Offsets run two passes ahead and coefficients one round ahead: while a
  // round is summed, the lane's next round of the pass is in flight, or after
  // its last round the first round of the next pass.
  int64_t p0[RB], p1[RB], n0[RB], n1[RB];
  offsets(0, p0, p1);
  offsets(kRowsPass, n0, n1);
  Round cur;
  load_round(p0, p1, 0, cur);
  for (int64_t base = 0; base < nrows; base += kRowsPass) {
    int64_t f0[RB], f1[RB];
    offsets(base + 2 * kRowsPass, f0, f1);  // past ne: empty
    float acc[RB][MR];
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int mm = 0; mm < MR; ++mm) acc[u][mm] = 0.0f;
    for (int64_t e0 = 0;; e0 += kE * G) {
      bool more = false;
#pragma unroll
      for (int u = 0; u < RB; ++u) more |= first(p0[u], e0 + kE * G) < p1[u];
      int64_t lq[RB], lqe[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        lq[u] = more ? p0[u] : n0[u];
        lqe[u] = more ? p1[u] : n1[u];
      }
      Round nxt;
      load_round(lq, lqe, more ? e0 + kE * G : 0, nxt);
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          if (cur.ok >> (u * kE + e) & 1u) {
            const Rec<MR> r = rec_load<MR>(z, cur.cc[u][e]);
#pragma unroll
            for (int mm = 0; mm < MR; ++mm) acc[u][mm] = fmaf(cur.vv[u][e], r.v[mm], acc[u][mm]);
          }
        }
      cur = nxt;
      if (!more) break;
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
      n0[u] = f0[u];
      n1[u] = f1[u];
    }
  }
}

template <int XDT, int MR, int G, int RB, int TB, bool VL>
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
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_wha_addend<XDT, MR, G, RB, TB, VL>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kWhaLdsAll - 256));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_wha_addend<XDT, MR, G, RB, TB, VL>), dim3((unsigned)xblocks, (unsigned)nch), dim3(TB), shmem, s, x,
                     M, K, N, lp, row_ptr, col, val, nnz, C, nchunk);
  return hipGetLastError();
}

template <int XDT, bool VL>
hipError_t wha_x(const void* x, int64_t M, int64_t K, int64_t N, int lp, const int32_t* row_ptr, const int32_t* col,
                 const float* val, int64_t nnz, float* C, hipStream_t s) {
  if (M >= 8 && 8 * K * 4 <= kWhaLds) return wha_t<XDT, 8, 4, 1, 1024, VL>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  if (M >= 4 && 4 * K * 4 <= kWhaLds) return wha_t<XDT, 4, 4, 1, 1024, VL>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  if (M >= 2 && 2 * K * 4 <= kWhaLds) return wha_t<XDT, 2, 4, 1, 1024, VL>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  return wha_t<XDT, 1, 4, 1, 1024, VL>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
}

// ---- the merged weight of the prefill path
//
// One workgroup of 256 threads per weight row n.  Its float32 row of F
// (coefficients added into a zeroed LDS row, columns clamped into the row) is
// transformed in place within blocks of P = 2^lp columns.  The butterfly
// stages of different column bits commute, so the bits from 10 up (blocks
// longer than 1024) go first, in LDS passes of up to four stages (each thread
// holds the 16 values of one group in registers); then, for each 4096 columns,
// thread t takes columns 16 t .. 16 t + 15: bits 0-3 are combined in its
// registers and bits 4-9 across the wave's lanes (DPP quad permutations for
// lane bits 0-1, swizzles for 2-3, half swaps for 4-5).  The thread then
// dequantizes its 16 weights, w' = fl32(L[c] fl32(m s)) as dequantization
// defines it, adds its transform values scaled by 2^-lp (exact) and stores
// bf16(w' + d) rounded to nearest even.  LDS slot of column i: bits 0..3 XORed
// with bits 6..9 and bits 4..5 with bits 8..9, so that the 64 lanes of every
// pass's 4-byte reads and writes, and of the threads' 16-column reads, hit 64
// distinct banks.  The first 4096 columns' codes and scales are loaded before
// the transform.
__device__ __forceinline__ uint32_t mslot(uint32_t i) { return i ^ ((i >> 6) & 15u) ^ (((i >> 8) & 3u) << 4); }

template <int B>
__device__ __forceinline__ void merge_pass(float* row, uint32_t K, int sh) {
  constexpr int E = 1 << B;
  const uint32_t ng = K >> B;
  for (uint32_t gi = threadIdx.x; gi < ng; gi += 256) {
    const uint32_t base = ((gi >> sh) << (sh + B)) | (gi & ((1u << sh) - 1u));
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = row[mslot(base + ((uint32_t)i << sh))];
#pragma unroll
    for (int st = 1; st < E; st <<= 1)
#pragma unroll
      for (int i = 0; i < E; ++i)
        if ((i & st) == 0) {
          const float a = v[i], c = v[i + st];
          v[i] = a + c;
          v[i + st] = a - c;
        }
#pragma unroll
    for (int i = 0; i < E; ++i) row[mslot(base + ((uint32_t)i << sh))] = v[i];
  }
}

// 16 codes of BITS bits (LSB first) starting at element 16 q of the flat codes
template <int BITS>
__device__ __forceinline__ void merge_codes16(const uint8_t* codes, int64_t q, uint32_t (&w)[(BITS + 1) / 2]) {
  const uint8_t* p = codes + q * (2 * BITS);
  if constexpr (BITS == 2) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (BITS == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    w[0] = u.x;
    w[1] = u.y;
  } else if constexpr (BITS == 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    w[0] = u.x;
    w[1] = u.y;
    w[2] = u.z;
    w[3] = u.w;
  } else {  // 6 bytes at a 2-byte boundary
    const uint16_t* h = reinterpret_cast<const uint16_t*>(p);
    w[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    w[1] = h[2];
  }
}
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[(BITS + 1) / 2], int i) {
  if constexpr (BITS == 3) {
    const uint64_t v = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
    return (uint32_t)(v >> (3 * i)) & 7u;
  } else {
    return (w[(BITS * i) >> 5] >> ((BITS * i) & 31)) & ((1u << BITS) - 1u);
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void k_wha_merge(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ q8,
                                                   const float* __restrict__ cst, Levels lv, int64_t K, int lp,
                                                   const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                                                   const float* __restrict__ val, int64_t nnz, uint16_t* __restrict__ out) {
  constexpr int NL = 1 << BITS, CW = (BITS + 1) / 2;
  extern __shared__ float msm[];
  float* sL = msm;
  float* row = msm + NL;
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t Ku = (uint32_t)K;
  const int64_t e0 = n * K;  // first flat element of the row
  // the first 4096 columns' codes and block scale (clamped reads; used only in range)
  uint32_t cw[CW];
  float ap0;
  {
    const int64_t c = e0 + min(16u * (uint32_t)tid, Ku - 16u);
    merge_codes16<BITS>(codes, c >> 4, cw);
    ap0 = (float)q8[c >> 6] * cst[c >> 14];
  }
  const int64_t c0 = min<int64_t>(max<int64_t>(row_ptr[n], 0), nnz);
  const int64_t c1 = max<int64_t>(c0, min<int64_t>(row_ptr[n + 1], nnz));
  stage_levels<NL>(lv, sL);
  for (uint32_t i = 4 * tid; i < Ku; i += 1024) *reinterpret_cast<float4*>(row + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();
  for (int64_t e = c0 + tid; e < c1; e += 256) {
    const uint32_t c = (uint32_t)min<int64_t>(max<int64_t>(col[e], 0), K - 1);
    atomicAdd(row + mslot(c), val[e]);  // (repeated columns of a row add up)
  }
  __syncthreads();
  for (int sh = 10; sh < lp; sh += 4) {
    switch (min(4, lp - sh)) {
      case 1: merge_pass<1>(row, Ku, sh); break;
      case 2: merge_pass<2>(row, Ku, sh); break;
      case 3: merge_pass<3>(row, Ku, sh); break;
      default: merge_pass<4>(row, Ku, sh); break;
    }
    __syncthreads();
  }
  const float inv_p = __builtin_bit_cast(float, (uint32_t)(127 - lp) << 23);  // 2^-lp
  for (uint32_t s0 = 0; s0 < Ku; s0 += 4096) {  // uniform: every lane takes part in the lane exchanges
    const uint32_t cb = s0 + 16u * (uint32_t)tid;
    const bool on = cb < Ku;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = on ? row[mslot(cb + (uint32_t)j)] : 0.0f;
#pragma unroll
    for (int st = 1; st < 16; st <<= 1)
      if ((1 << lp) > st) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (!(j & st)) {
            const float a = v[j], b = v[j + st];
            v[j] = a + b;
            v[j + st] = a - b;
          }
      }
    // lane bit sb pairs lane l (value a if bit sb of l is 0) with l ^ 2^sb
    // (value b): the pair becomes (a + b, a - b)
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
      if (lp > 4 + sb) {
        const bool up = (lane >> sb) & 1;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int vi = __float_as_int(v[j]);
          int oi;
          if (sb == 0) oi = __builtin_amdgcn_mov_dpp(vi, 0xB1, 0xF, 0xF, false);       // lane ^ 1
          else if (sb == 1) oi = __builtin_amdgcn_mov_dpp(vi, 0x4E, 0xF, 0xF, false);  // lane ^ 2
          else if (sb == 2) oi = __builtin_amdgcn_ds_swizzle(vi, (4 << 10) | 0x1F);    // lane ^ 4
          else oi = __builtin_amdgcn_ds_swizzle(vi, (8 << 10) | 0x1F);                 // lane ^ 8
          const float o = __int_as_float(oi);
          v[j] = up ? o - v[j] : v[j] + o;
        }
      }
    // lane bits 4 and 5: the half swaps hand both lanes of a pair (a, b)
    if (lp > 8) {
      const bool up = (lane >> 4) & 1;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
        const float a = __uint_as_float(sw[0]), b = __uint_as_float(sw[1]);
        v[j] = up ? a - b : a + b;
      }
    }
    if (lp > 9) {
      const bool up = (lane >> 5) & 1;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
        const float a = __uint_as_float(sw[0]), b = __uint_as_float(sw[1]);
        v[j] = up ? a - b : a + b;
      }
    }
    if (on) {
      uint32_t w[CW];
      float ap;
      if (s0 == 0) {
#pragma unroll
        for (int i = 0; i < CW; ++i) w[i] = cw[i];
        ap = ap0;
      } else {
        const int64_t c = e0 + cb;
        merge_codes16<BITS>(codes, c >> 4, w);
        ap = (float)q8[c >> 6] * cst[c >> 14];
      }
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float w0 = __fmul_rn(sL[code_at<BITS>(w, i)], ap) + v[i] * inv_p;
        const float w1 = __fmul_rn(sL[code_at<BITS>(w, i + 1)], ap) + v[i + 1] * inv_p;
        o[i / 2] = pack_bf16x2(w0, w1);
      }
      uint4* dst = reinterpret_cast<uint4*>(out + e0 + cb);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

template <int BITS>
hipError_t wha_merge_b(const uint8_t* codes, const uint8_t* q8, const float* cst, const Levels& lv, int64_t N,
                       int64_t K, int lp, const int32_t* row_ptr, const int32_t* col, const float* val, int64_t nnz,
                       uint16_t* out, hipStream_t s) {
  const size_t shmem = (size_t)((1 << BITS) + K) * 4;
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_wha_merge<BITS>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWhaLdsAll);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_wha_merge<BITS>), dim3((unsigned)N), dim3(256), shmem, s, codes, q8, cst, lv, K, lp,
                     row_ptr, col, val, nnz, out);
  return hipGetLastError();
}

}  // namespace

int64_t wha_max_cols() { return kWhaLds / 4; }

hipError_t launch_wha_merge(const uint8_t* codes, const uint8_t* q8, const float* cst, int bits, const Levels& lv,
                            int64_t N, int64_t K, int lp, const int32_t* row_ptr, const int32_t* col, const float* val,
                            int64_t nnz, uint16_t* out, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (K > wha_max_cols() || K % 64 != 0 || lp < 0 || (int64_t(1) << lp) > K) return hipErrorInvalidValue;
  switch (bits) {
    case 2: return wha_merge_b<2>(codes, q8, cst, lv, N, K, lp, row_ptr, col, val, nnz, out, s);
    case 3: return wha_merge_b<3>(codes, q8, cst, lv, N, K, lp, row_ptr, col, val, nnz, out, s);
    case 4: return wha_merge_b<4>(codes, q8, cst, lv, N, K, lp, row_ptr, col, val, nnz, out, s);
    default: return wha_merge_b<8>(codes, q8, cst, lv, N, K, lp, row_ptr, col, val, nnz, out, s);
  }
}

hipError_t launch_wha_addend(const void* x, int xdt, int64_t M, int64_t K, int64_t N, int lp, const int32_t* row_ptr,
                             const int32_t* col, const float* val, int64_t nnz, float* C, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K > wha_max_cols() || K % 8 != 0) return hipErrorInvalidValue;
  // 16-byte coefficient loads address col and val with 32-bit byte offsets
  const bool vl = nnz >= 4 && nnz < (int64_t(1) << 29);
  if (xdt == DT_F32)
    return vl ? wha_x<DT_F32, true>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s)
              : wha_x<DT_F32, false>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
  return vl ? wha_x<DT_BF16, true>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s)
            : wha_x<DT_BF16, false>(x, M, K, N, lp, row_ptr, col, val, nnz, C, s);
}

}  // namespace qlr

// Hybrid outlier split of a frozen weight (QFT page, section 2.2 "Hybrid
// feature quantizer"): the k entries of largest |w| are kept at full precision
// in a sparse side channel and the dense rest is quantized.  The dense rest
// uses the blockwise quantile format; the side channel holds, per outlier, the
// float32 residual w - w' against the dense part's dequantized value there (the
// codebook has no exact zero level), as CSR by weight row.
//
// Selection: the k largest keys |w| (float32 bits, monotone for |w| >= 0), ties
// to the lower flat index.  A radix select finds the k-th largest key T in
// three passes over 11, 11 and 9 key bits (per-workgroup LDS histograms merged
// with global atomics, one single-workgroup step per pass narrowing the prefix);
// then every key > T is taken and the keys == T in index order until k.
#include <algorithm>
#include <type_traits>

#include "qlr_internal.h"

namespace qlr {

namespace {

constexpr int kOlBins = 2048;
constexpr int kOlElems = 4096;  // elements per workgroup in the count / emit passes
constexpr int64_t kSparseLds = 64 * 1024;  // staged x rows of the sparse term (two workgroups per CU)

template <int WDT>
__device__ __forceinline__ uint32_t ol_key(const void* W, int64_t i, float* wv) {
  const float w = load_elem<WDT>(W, i);
  *wv = w;
  return __float_as_uint(w) & 0x7FFFFFFFu;
}

// state: [0] prefix, [1] mask, [2] k still to place below the prefix's bin, [3] keys > prefix counted so far,
// [4] non-finite flag
template <int WDT>
__global__ __launch_bounds__(256) void k_ol_hist(const void* W, int64_t n, int shift, int nbits,
                                                 uint32_t* __restrict__ state, uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kOlBins];
  for (int b = threadIdx.x; b < kOlBins; b += 256) h[b] = 0;
  __syncthreads();
  const uint32_t prefix = state[0], mask = state[1];
  const uint32_t bmask = (1u << nbits) - 1u;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float w;
    const uint32_t key = ol_key<WDT>(W, i, &w);
    bad |= !(fabsf(w) <= 3.402823466e38f);
    if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & bmask], 1u);
  }
  if (bad) state[4] = 1u;
  __syncthreads();
  for (int b = threadIdx.x; b <= (int)bmask; b += 256)
    if (h[b]) atomicAdd(&hist[b], h[b]);
}

// one workgroup: find the bin holding the k-th largest remaining key; clears hist
// for the next pass.  Thread t owns bins nb-1-2t and nb-2-2t; an inclusive scan of
// the pairs from the top gives, per bin, the count of keys in the bins above it,
// and the one bin with above < need <= above + count writes the state (bin 0
// when the counts fall short, as a sequential walk down the bins would end).
__global__ __launch_bounds__(1024) void k_ol_select(int shift, int nbits, uint32_t* __restrict__ state,
                                                    uint32_t* __restrict__ hist) {
  __shared__ uint32_t sc[1024];
  const int nb = 1 << nbits;
  const int t = threadIdx.x;
  const int b0 = nb - 1 - 2 * t, b1 = nb - 2 - 2 * t;
  uint32_t h0 = 0, h1 = 0;
  if (b0 >= 0) {
    h0 = hist[b0];
    hist[b0] = 0;
  }
  if (b1 >= 0) {
    h1 = hist[b1];
    hist[b1] = 0;
  }
  const uint32_t need = state[2];
  sc[t] = h0 + h1;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t v = t >= o ? sc[t - o] : 0u;
    __syncthreads();
    sc[t] += v;
    __syncthreads();
  }
  const uint32_t above0 = sc[t] - (h0 + h1), above1 = above0 + h0;
  const uint32_t total = sc[1023];
  int bin = -1;
  uint32_t above = 0;
  if (b0 >= 0 && above0 < need && need <= above0 + h0) {
    bin = b0;
    above = above0;
  } else if (b1 >= 0 && above1 < need && need <= above1 + h1) {
    bin = b1;
    above = above1;
  } else if (total < need && (b0 == 0 || b1 == 0)) {
    bin = 0;
    above = b0 == 0 ? above0 : above1;
  }
  if (bin >= 0) {
    state[0] |= (uint32_t)bin << shift;
    state[1] |= (uint32_t)(nb - 1) << shift;
    state[2] = need - above;
    state[3] += above;
  }
}

// per workgroup of kOlElems elements: counts of keys > T and == T
template <int WDT>
__global__ __launch_bounds__(256) void k_ol_count(const void* W, int64_t n, const uint32_t* __restrict__ state,
                                                  uint32_t* __restrict__ cnt) {
  __shared__ uint32_t sgt, seq;
  if (threadIdx.x == 0) sgt = seq = 0;
  __syncthreads();
  const uint32_t T = state[0];
  uint32_t gt = 0, eq = 0;
  const int64_t b0 = (int64_t)blockIdx.x * kOlElems;
  for (int t = threadIdx.x; t < kOlElems; t += 256) {
    const int64_t i = b0 + t;
    if (i >= n) break;
    float w;
    const uint32_t key = ol_key<WDT>(W, i, &w);
    gt += key > T;
    eq += key == T;
  }
  atomicAdd(&sgt, gt);
  atomicAdd(&seq, eq);
  __syncthreads();
  if (threadIdx.x == 0) {
    cnt[2 * blockIdx.x] = sgt;
    cnt[2 * blockIdx.x + 1] = seq;
  }
}

// one workgroup: per block, the number of ties it takes and its first output slot (in index order)
__global__ __launch_bounds__(1024) void k_ol_scan(int64_t nblocks, const uint32_t* __restrict__ state,
                                                  const uint32_t* __restrict__ cnt, uint32_t* __restrict__ plan) {
  __shared__ uint32_t seq[1024], ssel[1024];
  __shared__ uint32_t carry_eq, carry_sel;
  if (threadIdx.x == 0) carry_eq = carry_sel = 0;
  __syncthreads();
  const uint32_t need_eq = state[2];
  for (int64_t c0 = 0; c0 < nblocks; c0 += 1024) {
    const int64_t b = c0 + threadIdx.x;
    const uint32_t gt = b < nblocks ? cnt[2 * b] : 0u, eq = b < nblocks ? cnt[2 * b + 1] : 0u;
    seq[threadIdx.x] = eq;
    __syncthreads();
    // inclusive scan of eq (Hillis-Steele)
    for (int o = 1; o < 1024; o <<= 1) {
      const uint32_t v = threadIdx.x >= (unsigned)o ? seq[threadIdx.x - o] : 0u;
      __syncthreads();
      seq[threadIdx.x] += v;
      __syncthreads();
    }
    const uint32_t eq_before = carry_eq + seq[threadIdx.x] - eq;
    const uint32_t take = eq_before >= need_eq ? 0u : min(eq, need_eq - eq_before);
    const uint32_t sel = gt + take;
    ssel[threadIdx.x] = sel;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const uint32_t v = threadIdx.x >= (unsigned)o ? ssel[threadIdx.x - o] : 0u;
      __syncthreads();
      ssel[threadIdx.x] += v;
      __syncthreads();
    }
    if (b < nblocks) {
      plan[2 * b] = take;
      plan[2 * b + 1] = carry_sel + ssel[threadIdx.x] - sel;
    }
    __syncthreads();
    if (threadIdx.x == 1023) {
      carry_eq += seq[1023];
      carry_sel += ssel[1023];
    }
    __syncthreads();
  }
}

// per workgroup: mark, compact (flat index, w) in index order, write the dense copy
template <int WDT>
__global__ __launch_bounds__(256) void k_ol_emit(const void* W, int64_t n, const uint32_t* __restrict__ state,
                                                 const uint32_t* __restrict__ plan, void* __restrict__ dense,
                                                 int32_t* __restrict__ oidx, float* __restrict__ oval) {
  // thread t handles elements b0 + 16 t .. + 15 (contiguous, so local ranks follow index order)
  __shared__ uint32_t seq[256], ssel[256];
  const uint32_t T = state[0];
  const int64_t b0 = (int64_t)blockIdx.x * kOlElems + 16 * threadIdx.x;
  uint32_t keys[16];
  float ws[16];
  uint32_t rw[16];  // raw 16-bit words (16-bit weights)
  uint32_t neq = 0;
  const bool full = b0 + 16 <= n;
  if (full) {
    // the thread's 16 elements in 16-byte loads (W is 16-byte aligned)
    if constexpr (WDT == DT_F32) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + b0)[q];
        ws[4 * q] = v.x;
        ws[4 * q + 1] = v.y;
        ws[4 * q + 2] = v.z;
        ws[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 v = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(W) + b0)[q];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t h = (w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          rw[8 * q + e] = h;
          ws[8 * q + e] = WDT == DT_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      keys[e] = __float_as_uint(ws[e]) & 0x7FFFFFFFu;
      neq += keys[e] == T;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t i = b0 + e;
      keys[e] = i < n ? ol_key<WDT>(W, i, &ws[e]) : 0u;
      if (i >= n) ws[e] = 0.0f;
      rw[e] = (WDT != DT_F32 && i < n) ? (uint32_t)reinterpret_cast<const uint16_t*>(W)[i] : 0u;
      neq += (i < n && keys[e] == T);
    }
  }
  seq[threadIdx.x] = neq;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const uint32_t v = threadIdx.x >= (unsigned)o ? seq[threadIdx.x - o] : 0u;
    __syncthreads();
    seq[threadIdx.x] += v;
    __syncthreads();
  }
  const uint32_t take = plan[2 * blockIdx.x];
  uint32_t eq_rank = seq[threadIdx.x] - neq;
  bool sel[16];
  uint32_t nsel = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t i = b0 + e;
    const bool valid = i < n;
    const bool is_eq = valid && keys[e] == T;
    sel[e] = valid && (keys[e] > T || (is_eq && eq_rank < take));
    eq_rank += is_eq;
    nsel += sel[e];
  }
  ssel[threadIdx.x] = nsel;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const uint32_t v = threadIdx.x >= (unsigned)o ? ssel[threadIdx.x - o] : 0u;
    __syncthreads();
    ssel[threadIdx.x] += v;
    __syncthreads();
  }
  uint32_t pos = plan[2 * blockIdx.x + 1] + ssel[threadIdx.x] - nsel;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (sel[e]) {
      oidx[pos] = (int32_t)(b0 + e);
      oval[pos] = ws[e];
      ++pos;
    }
  }
  // the dense copy: the weight with the selected entries zeroed
  if (full) {
    if constexpr (WDT == DT_F32) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        reinterpret_cast<float4*>(reinterpret_cast<float*>(dense) + b0)[q] =
            make_float4(sel[4 * q] ? 0.0f : ws[4 * q], sel[4 * q + 1] ? 0.0f : ws[4 * q + 1],
                        sel[4 * q + 2] ? 0.0f : ws[4 * q + 2], sel[4 * q + 3] ? 0.0f : ws[4 * q + 3]);
    } else {
      uint32_t pk[8];
#pragma unroll
      for (int p = 0; p < 8; ++p)
        pk[p] = (sel[2 * p] ? 0u : rw[2 * p]) | ((sel[2 * p + 1] ? 0u : rw[2 * p + 1]) << 16);
#pragma unroll
      for (int q = 0; q < 2; ++q)
        reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(dense) + b0)[q] =
            make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t i = b0 + e;
      if (i >= n) break;
      if constexpr (WDT == DT_F32) reinterpret_cast<float*>(dense)[i] = sel[e] ? 0.0f : ws[e];
      else reinterpret_cast<uint16_t*>(dense)[i] = sel[e] ? (uint16_t)0 : (uint16_t)rw[e];
    }
  }
}

// per outlier: residual against the dense part's dequantized value, and its column
template <int BITS>
__global__ __launch_bounds__(256) void k_ol_finish(int64_t k, int64_t cols, const int32_t* __restrict__ oidx,
                                                   const float* __restrict__ oval, const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ q8, const float* __restrict__ cst,
                                                   Levels lv, int32_t* __restrict__ col, float* __restrict__ val) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  const int64_t flat = oidx[j];
  const int64_t blk = flat >> 6;
  const int e = (int)(flat & 63);
  const int bit0 = BITS * e;
  const uint8_t* cb = codes + blk * (8 * BITS);
  uint32_t two = cb[bit0 >> 3];
  if ((bit0 >> 3) + 1 < 8 * BITS) two |= (uint32_t)cb[(bit0 >> 3) + 1] << 8;
  const int c = (int)((two >> (bit0 & 7)) & ((1u << BITS) - 1u));
  {
    // two products and one difference, each rounded on its own: no fused multiply-add
#pragma clang fp contract(off)
    const float ap = (float)q8[blk] * cst[blk >> 8];
    const float wd = lv.v[c] * ap;
    val[j] = oval[j] - wd;
  }
  col[j] = (int32_t)(flat % cols);
}

// row_ptr[r] = number of outliers with flat index < r * cols (binary search over the ascending indices)
// Largest entry count over the row groups [128 g, 128 g + 128) of a CSR, by
// one workgroup: a strided max per thread, then over the wave's lanes and the
// waves (row offsets clamped into [0, k], as the forward kernels read them).
__global__ __launch_bounds__(1024) void k_ol_group_max(int64_t rows, int64_t k, const int32_t* __restrict__ row_ptr,
                                                       uint32_t* __restrict__ out) {
  __shared__ uint32_t red[16];
  const int64_t groups = (rows + 127) / 128;
  auto off = [&](int64_t r) { return min<int64_t>(max<int64_t>(row_ptr[r], 0), k); };
  uint32_t m = 0;
  for (int64_t g = threadIdx.x; g < groups; g += 1024) {
    const int64_t a = off(128 * g), b = off(min<int64_t>(rows, 128 * (g + 1)));
    m = max(m, (uint32_t)max<int64_t>(b - a, 0));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) r = max(r, red[w]);
    *out = r;
  }
}

__global__ __launch_bounds__(256) void k_ol_rowptr(int64_t rows, int64_t cols, int64_t k,
                                                   const int32_t* __restrict__ oidx, int32_t* __restrict__ row_ptr) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r > rows) return;
  const int64_t target = r * cols;
  int64_t lo = 0, hi = k;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)oidx[mid] < target) lo = mid + 1;
    else hi = mid;
  }
  row_ptr[r] = (int32_t)lo;
}

// C[m][n] = sum over row n's outliers j of val[j] x[m][col[j]] (float32, x widened
// exactly, outliers in CSR order).
//
// blockIdx.x: MR rows of x, staged in LDS transposed (sx[c][mm], MR values of
// one column contiguous, so one 16-byte read serves 8 bf16 rows); MR = 0 reads
// one x row from global memory (rows too long for LDS).  blockIdx.y: a range of
// weight rows, 1024 threads each taking one row per pass (see the loop).
template <int XDT, int MR, int TB>
__global__ __launch_bounds__(TB) void k_sparse_addend(const void* __restrict__ x, int64_t M, int64_t K, int64_t N,
                                                       const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col,
                                                       const float* __restrict__ val, int64_t nnz,
                                                       float* __restrict__ C, int64_t nchunk, int64_t cap) {
  using XT = std::conditional_t<XDT == DT_F32, float, uint16_t>;
  // cap >= 0: rows of kGemmTileRows-row groups with at most cap entries are the
  // prefill GEMM's own (it adds them to its weights) and are skipped; a
  // workgroup whose range holds none of the other rows ends here.  The clamps
  // are the GEMM's.
  const int64_t nb = (int64_t)blockIdx.y * nchunk, ne = min(N, nb + nchunk);
  auto group_count = [&](int64_t g) {
    const int64_t e0 = min<int64_t>(max<int64_t>(row_ptr[min(g * kGemmTileRows, N)], 0), nnz);
    return max<int64_t>(e0, min<int64_t>(row_ptr[min((g + 1) * kGemmTileRows, N)], nnz)) - e0;
  };
  if (cap >= 0) {
    const int64_t g0 = nb / kGemmTileRows, g1 = ne > nb ? (ne - 1) / kGemmTileRows + 1 : g0;
    bool any = false;
    for (int64_t g = g0 + threadIdx.x; g < g1; g += TB) any = any || group_count(g) > cap;
    if (!__syncthreads_or(any)) return;  // uniform
  }
  constexpr int R = MR > 0 ? MR : 1;
  constexpr int EPC = 16 / (int)sizeof(XT);  // elements per 16-byte chunk of an x row
  extern __shared__ uint4 smem_u4[];
  XT* sx = reinterpret_cast<XT*>(smem_u4);
  const XT* xg = reinterpret_cast<const XT*>(x);
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * R;
  // (bf16, 8 rows): column c's 8 values form one 16-byte record at slot
  // sl(c) = c with its low 3 bits XORed by bits 3..5, so the 8 records a thread
  // writes (columns 8 q .. 8 q + 7) and those of its neighbours fall in distinct banks
  constexpr bool kRec = XDT == DT_BF16 && MR == 8;
  auto sl = [](int64_t c) -> int64_t { return (c & ~int64_t(7)) | ((c & 7) ^ ((c >> 3) & 7)); };
  if constexpr (MR > 0) {
    // chunk q of the x rows: EPC consecutive columns of each of the MR rows
    for (int64_t q = tid; q < K / EPC; q += TB) {
      XT v[MR][EPC];
#pragma unroll
      for (int mm = 0; mm < MR; ++mm) {
        const int64_t m = m0 + mm < M ? m0 + mm : M - 1;
        const uint4 u = *reinterpret_cast<const uint4*>(xg + m * K + q * EPC);
        const XT* e = reinterpret_cast<const XT*>(&u);
#pragma unroll
        for (int i = 0; i < EPC; ++i) v[mm][i] = m0 + mm < M ? e[i] : (XT)0;
      }
      if constexpr (kRec) {
#pragma unroll
        for (int i = 0; i < EPC; ++i) {
          uint4 rec;
          rec.x = (uint32_t)v[0][i] | ((uint32_t)v[1][i] << 16);
          rec.y = (uint32_t)v[2][i] | ((uint32_t)v[3][i] << 16);
          rec.z = (uint32_t)v[4][i] | ((uint32_t)v[5][i] << 16);
          rec.w = (uint32_t)v[6][i] | ((uint32_t)v[7][i] << 16);
          smem_u4[sl(q * EPC + i)] = rec;
        }
      } else {
#pragma unroll
        for (int i = 0; i < EPC; ++i)
#pragma unroll
          for (int mm = 0; mm < MR; ++mm) sx[(q * EPC + i) * MR + mm] = v[mm][i];
      }
    }
    __syncthreads();
  }
  // the R x values of column c
  auto xcol = [&](int64_t c, float (&xv)[R]) {
    if constexpr (kRec) {
      const uint4 rec = smem_u4[sl(c)];
      const uint32_t w[4] = {rec.x, rec.y, rec.z, rec.w};
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) xv[mm] = bf16_bits_to_f32((w[mm >> 1] >> (16 * (mm & 1))) & 0xFFFFu);
    } else {
#pragma unroll
      for (int mm = 0; mm < R; ++mm) {
        if constexpr (MR > 0) {
          const XT e = sx[c * MR + mm];
          if constexpr (XDT == DT_F32) xv[mm] = e;
          else xv[mm] = bf16_bits_to_f32(e);
        } else {
          if constexpr (XDT == DT_F32) xv[mm] = xg[m0 * K + c];
          else xv[mm] = bf16_bits_to_f32(xg[m0 * K + c]);
        }
      }
    }
  };
  // One weight row per thread and pass, its outliers in rounds of 8.  Offsets
  // run two passes ahead and outliers one round ahead: while a round is summed,
  // the thread's next round, or after its last round the first round of its
  // next pass, is in flight.  Offsets and columns are clamped into range: a
  // malformed CSR gives wrong sums, never a stray access.
  constexpr int kE = 8;
  auto offsets = [&](int64_t base, int64_t& q0, int64_t& q1, bool& keep) {
    const int64_t n = base + tid;
    const int64_t nc = n < ne ? n : ne - 1;
    // both loads unconditional and their values used unconditionally (a load
    // behind a branch would make the compiler wait for every load in flight);
    // past the range, and for the GEMM's own rows, the pass gets [lo, lo)
    const int64_t a0 = row_ptr[nc], a1 = row_ptr[nc + 1];
    const int64_t lo = a0 < 0 ? 0 : (a0 > nnz ? nnz : a0);
    const int64_t hi = a1 < lo ? lo : (a1 > nnz ? nnz : a1);
    keep = n < ne && (cap < 0 || group_count(nc / kGemmTileRows) > cap);
    q0 = lo;
    q1 = keep ? hi : lo;
  };
  // VL (4 <= nnz < 2^29): two 16-byte loads each of col and val per round; a
  // load that would run past nnz starts at nnz - 4, its element t then at js + t
  const bool vl = nnz >= 4 && nnz < (int64_t(1) << 29);
  const int nbytes = vl ? (int)(nnz * 4) : 0;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(col), (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(val), (short)0, nbytes, 0x00020000);
  struct Round {
    int32_t cc[kE];
    float vv[kE];
    uint32_t ok;  // bit e: coefficient e exists
  };
  auto load_round = [&](int64_t q, int64_t qe, int64_t e0, Round& R) {
    R.ok = 0;
    if (vl) {  // uniform
#pragma unroll
      for (int hh = 0; hh < kE / 4; ++hh) {
        const int64_t j = q + e0 + 4 * hh;
        const int64_t js = j < nnz - 4 ? j : nnz - 4;
        const u32x4_t lc = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, (int)(js * 4), 0, 0));
        const u32x4_t lv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)(js * 4), 0, 0));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          R.cc[4 * hh + t] = min<int32_t>(max<int32_t>((int32_t)lc[t], 0), (int32_t)(K - 1));
          R.vv[4 * hh + t] = __uint_as_float(lv[t]);
          R.ok |= (js + t >= j && js + t < qe) ? 1u << (4 * hh + t) : 0u;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int64_t j = q + e0 + e;
        const int64_t jc = j < nnz ? j : (nnz > 0 ? nnz - 1 : 0);
        R.cc[e] = nnz > 0 ? min<int32_t>(max<int32_t>(col[jc], 0), (int32_t)(K - 1)) : 0;
        R.vv[e] = nnz > 0 ? val[jc] : 0.0f;
        R.ok |= j < qe ? 1u << e : 0u;
      }
    }
  };
  int64_t p0, p1, n0, n1;
  bool pk, nk;  // the pass's row is stored
  offsets(nb, p0, p1, pk);
  offsets(nb + TB, n0, n1, nk);
  Round cur;
  load_round(p0, p1, 0, cur);
  for (int64_t base = nb; base < ne; base += TB) {
    int64_t f0, f1;
    bool fk;
    offsets(base + 2 * TB, f0, f1, fk);
    float acc[R];
#pragma unroll
    for (int mm = 0; mm < R; ++mm) acc[mm] = 0.0f;
    for (int64_t e0 = 0;; e0 += kE) {
      const bool more = p0 + e0 + kE < p1;
      Round nxt;
      load_round(more ? p0 : n0, more ? p1 : n1, more ? e0 + kE : 0, nxt);
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        if (cur.ok >> e & 1u) {
          float xv[R];
          xcol(cur.cc[e], xv);
#pragma unroll
          for (int mm = 0; mm < R; ++mm) acc[mm] = fmaf(cur.vv[e], xv[mm], acc[mm]);
        }
      }
      cur = nxt;
      if (!more) break;
    }
    const int64_t n = base + tid;
    if (pk) {
#pragma unroll
      for (int mm = 0; mm < R; ++mm)
        if (m0 + mm < M) C[(m0 + mm) * N + n] = acc[mm];
    }
    p0 = n0;
    p1 = n1;
    pk = nk;
    n0 = f0;
    n1 = f1;
    nk = fk;
  }
}

template <int XDT, int MR>
hipError_t sparse_addend_t(int64_t cap, const void* x, int64_t M, int64_t K, int64_t N, const int32_t* row_ptr,
                           const int32_t* col, const float* val, int64_t nnz, float* C, hipStream_t s) {
  constexpr int R = MR > 0 ? MR : 1;
  constexpr int TB = 1024;
  const int64_t xblocks = (M + R - 1) / R;
  // enough workgroups to fill the chip (each stages its x rows once)
  const int64_t nch = std::max<int64_t>(1, std::min<int64_t>((N + TB - 1) / TB, (256 + xblocks - 1) / xblocks));
  const int64_t nchunk = (N + nch - 1) / nch;
  const size_t es = XDT == DT_F32 ? 4 : 2;
  const size_t shmem = MR > 0 ? (size_t)MR * K * es : 0;
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_sparse_addend<XDT, MR, TB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kSparseLds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_sparse_addend<XDT, MR, TB>), dim3((unsigned)xblocks, (unsigned)nch), dim3(TB), shmem, s, x, M,
                     K, N, row_ptr, col, val, nnz, C, nchunk, cap);
  return hipGetLastError();
}

template <int XDT>
hipError_t sparse_addend_x(int64_t cap, const void* x, int64_t M, int64_t K, int64_t N, const int32_t* row_ptr,
                           const int32_t* col, const float* val, int64_t nnz, float* C, hipStream_t s) {
  const int64_t row = K * (XDT == DT_F32 ? 4 : 2);  // LDS bytes of one staged x row
  if (M > 4 && 8 * row <= kSparseLds) return sparse_addend_t<XDT, 8>(cap, x, M, K, N, row_ptr, col, val, nnz, C, s);
  if (M > 2 && 4 * row <= kSparseLds) return sparse_addend_t<XDT, 4>(cap, x, M, K, N, row_ptr, col, val, nnz, C, s);
  if (M > 1 && 2 * row <= kSparseLds) return sparse_addend_t<XDT, 2>(cap, x, M, K, N, row_ptr, col, val, nnz, C, s);
  if (row <= kSparseLds) return sparse_addend_t<XDT, 1>(cap, x, M, K, N, row_ptr, col, val, nnz, C, s);
  return sparse_addend_t<XDT, 0>(cap, x, M, K, N, row_ptr, col, val, nnz, C, s);
}

template <int WDT>
hipError_t ol_select_emit(const void* W, int64_t n, int64_t k, uint32_t* state, uint32_t* hist, uint32_t* cnt,
                          uint32_t* plan, void* dense, int32_t* oidx, float* oval, hipStream_t s) {
  const int hgrid = (int)std::min<int64_t>(1024, (n + 255) / 256);
  const int shifts[3] = {20, 9, 0}, bits[3] = {11, 11, 9};
  for (int p = 0; p < 3; ++p) {
    hipLaunchKernelGGL((k_ol_hist<WDT>), dim3(hgrid), dim3(256), 0, s, W, n, shifts[p], bits[p], state, hist);
    hipLaunchKernelGGL(k_ol_select, dim3(1), dim3(1024), 0, s, shifts[p], bits[p], state, hist);
  }
  const int64_t nblocks = (n + kOlElems - 1) / kOlElems;
  hipLaunchKernelGGL((k_ol_count<WDT>), dim3((unsigned)nblocks), dim3(256), 0, s, W, n, state, cnt);
  hipLaunchKernelGGL(k_ol_scan, dim3(1), dim3(1024), 0, s, nblocks, state, cnt, plan);
  hipLaunchKernelGGL((k_ol_emit<WDT>), dim3((unsigned)nblocks), dim3(256), 0, s, W, n, state, plan, dense, oidx,
                     oval);
  return hipGetLastError();
}

template <int BITS>
hipError_t ol_finish_b(int64_t k, int64_t cols, const int32_t* oidx, const float* oval, const uint8_t* codes,
                       const uint8_t* q8, const float* cst, const Levels& lv, int32_t* col, float* val,
                       hipStream_t s) {
  hipLaunchKernelGGL((k_ol_finish<BITS>), dim3((unsigned)((k + 255) / 256)), dim3(256), 0, s, k, cols, oidx, oval,
                     codes, q8, cst, lv, col, val);
  return hipGetLastError();
}

}  // namespace

size_t outlier_ws_bytes(int64_t numel, int64_t k) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const int64_t nblocks = (numel + kOlElems - 1) / kOlElems;
  return up(64) + up(kOlBins * 4) + up((size_t)nblocks * 8) * 2 + up((size_t)k * 4) * 2 + up((size_t)numel * 4);
}

hipError_t launch_outlier_split(const void* W, int wdt, int64_t numel, int64_t k, void* ws, void** dense,
                                uint32_t** flag, int32_t** oidx, float** oval, hipStream_t s) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const int64_t nblocks = (numel + kOlElems - 1) / kOlElems;
  char* p = reinterpret_cast<char*>(ws);
  uint32_t* state = reinterpret_cast<uint32_t*>(p);
  p += up(64);
  uint32_t* hist = reinterpret_cast<uint32_t*>(p);
  p += up(kOlBins * 4);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(p);
  p += up((size_t)nblocks * 8);
  uint32_t* plan = reinterpret_cast<uint32_t*>(p);
  p += up((size_t)nblocks * 8);
  *oidx = reinterpret_cast<int32_t*>(p);
  p += up((size_t)k * 4);
  *oval = reinterpret_cast<float*>(p);
  p += up((size_t)k * 4);
  *dense = p;
  *flag = state + 4;
  // state = {prefix 0, mask 0, k, 0, flag 0}, histogram cleared (fill kernels: no memset nodes)
  hipError_t e = launch_fill_u32(state, 0u, 16, s);
  if (e != hipSuccess) return e;
  e = launch_fill_u32(state + 2, (uint32_t)k, 1, s);
  if (e != hipSuccess) return e;
  e = launch_fill_u32(hist, 0u, kOlBins, s);
  if (e != hipSuccess) return e;
  switch (wdt) {
    case DT_F32: return ol_select_emit<DT_F32>(W, numel, k, state, hist, cnt, plan, *dense, *oidx, *oval, s);
    case DT_F16: return ol_select_emit<DT_F16>(W, numel, k, state, hist, cnt, plan, *dense, *oidx, *oval, s);
    default: return ol_select_emit<DT_BF16>(W, numel, k, state, hist, cnt, plan, *dense, *oidx, *oval, s);
  }
}

hipError_t launch_sparse_addend(const void* x, int xdt, int64_t M, int64_t K, int64_t N, const int32_t* row_ptr,
                                const int32_t* col, const float* val, int64_t nnz, float* C, hipStream_t s,
                                int64_t cap) {
  if (M == 0 || N == 0) return hipSuccess;
  if (xdt == DT_F32) return sparse_addend_x<DT_F32>(cap, x, M, K, N, row_ptr, col, val, nnz, C, s);
  return sparse_addend_x<DT_BF16>(cap, x, M, K, N, row_ptr, col, val, nnz, C, s);
}

hipError_t launch_outlier_finish(int64_t rows, int64_t cols, int64_t k, int bits, const Levels& lv,
                                 const uint8_t* codes, const uint8_t* q8, const float* cst, const int32_t* oidx,
                                 const float* oval, int32_t* row_ptr, int32_t* col, float* val, hipStream_t s) {
  hipLaunchKernelGGL(k_ol_rowptr, dim3((unsigned)((rows + 1 + 255) / 256)), dim3(256), 0, s, rows, cols, k, oidx,
                     row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || k == 0) return e;
  switch (bits) {
    case 2: return ol_finish_b<2>(k, cols, oidx, oval, codes, q8, cst, lv, col, val, s);
    case 3: return ol_finish_b<3>(k, cols, oidx, oval, codes, q8, cst, lv, col, val, s);
    case 4: return ol_finish_b<4>(k, cols, oidx, oval, codes, q8, cst, lv, col, val, s);
    default: return ol_finish_b<8>(k, cols, oidx, oval, codes, q8, cst, lv, col, val, s);
  }
}

hipError_t launch_group_max(int64_t rows, int64_t k, const int32_t* row_ptr, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_ol_group_max, dim3(1), dim3(1024), 0, s, rows, k, row_ptr, out);
  return hipGetLastError();
}

}  // namespace qlr

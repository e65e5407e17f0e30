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
#include <type_traits>

#include "qlr_internal.h"

namespace qlr {

namespace {

// LDS transpose read of 16-bit elements (ds_read_b64_tr_b16): within each group
// of 16 lanes, lane i receives element i % 4 of the 8-byte reads of lanes
// i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12, in that order.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4_t lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(const_cast<char*>(p)));
}

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

// VEC: every row of Q is 4-element aligned (C % 4 == 0): one 8- or 16-byte load
// per lane and row; lanes past C read the last 4 columns and drop them.
template <int QDT, bool VEC>
__global__ __launch_bounds__(256, 2) void k_lora_grad(GradParams G) {
  __shared__ float red[3 * 64 * 64];
  extern __shared__ f32x4_t sP[];  // rows x 4 (16 adapter rows per staged row)
  const int ji = (G.nj > 1 && (int64_t)blockIdx.x >= G.J[1].tile0) ? 1 : 0;
  const float* __restrict__ P = G.J[ji].P;
  const char* __restrict__ Q = reinterpret_cast<const char*>(G.J[ji].Q);
  float* part = G.J[ji].part;
  float* out = G.J[ji].out;
  const int64_t C = G.J[ji].C;
  const int p_splits = G.J[ji].p_splits, cols_major = G.J[ji].cols_major, ctiles = G.J[ji].ctiles;
  const int64_t lt = (int64_t)blockIdx.x - G.J[ji].tile0;
  const int64_t ct = lt % ctiles, rest = lt / ctiles;
  const int jc = (int)(rest % G.jchunks), z = (int)(rest / G.jchunks);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t M = G.M;
  const int r = G.r, j0 = 16 * jc;
  const int64_t mb = (int64_t)z * G.rows, me = min(M, mb + G.rows);
  const int64_t c0 = ct * 256 + 4 * lane;
  float* sPf = reinterpret_cast<float*>(sP);

  constexpr int ES = QDT == DT_F32 ? 4 : 2;
  // columns read by this lane: clamped to valid addresses, dropped at use
  const int64_t cl = VEC ? min(c0, C - 4) : 0;
  bool cv[4];
  int64_t ce[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    cv[e] = c0 + e < C;
    ce[e] = min(c0 + e, C - 1);
  }
  const int64_t rw = G.rows / 4;  // rows of one wave (a multiple of 8)
  const int64_t wb = mb + w * rw, we = min(me, wb + rw);
  // One batch: 8 rows of Q, loaded from wave-uniform rows clamped into
  // [wb, we) (every address valid; rows past we are dropped at use).
  using Raw = typename std::conditional<QDT == DT_F32, f32x4_t, uint2>::type;
  struct Batch {
    Raw raw[kGradBatch];
    float q[kGradBatch][4];
  };
  auto load_batch = [&](int64_t m, Batch& bt) {
#pragma unroll
    for (int b = 0; b < kGradBatch; ++b) {
      const int64_t row = max(wb, min(m + b, we - 1));
      if constexpr (VEC) {
        bt.raw[b] = *reinterpret_cast<const Raw*>(Q + (row * C + cl) * ES);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) bt.q[b][e] = load_elem<QDT>(Q, row * C + ce[e]);
      }
    }
  };

  float acc[16][4];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[jj][e] = 0.0f;
  auto compute = [&](int64_t m, Batch& bt) {
#pragma unroll
    for (int b = 0; b < kGradBatch; ++b) {
      float q[4];
      if constexpr (VEC) {
        if constexpr (QDT == DT_F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = bt.raw[b][e];
        } else {
          q[0] = __uint_as_float(bt.raw[b].x << 16);
          q[1] = __uint_as_float(bt.raw[b].x & 0xFFFF0000u);
          q[2] = __uint_as_float(bt.raw[b].y << 16);
          q[3] = __uint_as_float(bt.raw[b].y & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = bt.q[b][e];
      }
      const bool rv = m + b < we;  // wave-uniform
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = (rv && cv[e]) ? q[e] : 0.0f;
      const int64_t srow = max(wb, min(m + b, we - 1)) - mb;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4_t p = sP[srow * 4 + j4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * j4 + jj][e] = fmaf(p[jj], q[e], acc[4 * j4 + jj][e]);
      }
    }
  };

  // the first batch is in flight while P is staged
  Batch ba, bb;
  if (wb < we) load_batch(wb, ba);

  // stage P rows [mb, me), adapter rows [j0, j0 + 16), zero past r
  const int nst = (int)(me - mb) * 16;
  if (p_splits == 1) {
#pragma unroll 4
    for (int idx = threadIdx.x; idx < nst; idx += 256) {
      const int j = j0 + (idx & 15);
      const float v = P[(mb + (idx >> 4)) * r + min(j, r - 1)];
      sPf[idx] = j < r ? v : 0.0f;
    }
  } else {
    for (int idx = threadIdx.x; idx < nst; idx += 256) {
      const int j = j0 + (idx & 15);
      float v = 0.0f;
      for (int sp = 0; sp < p_splits; ++sp) v += P[((int64_t)sp * M + mb + (idx >> 4)) * r + min(j, r - 1)];
      sPf[idx] = j < r ? v : 0.0f;
    }
  }
  __syncthreads();

  // two batches in flight: the next one loads while the current one is multiplied
  for (int64_t m = wb; m < we; m += 2 * kGradBatch) {
    load_batch(m + kGradBatch, bb);
    compute(m, ba);
    load_batch(m + 2 * kGradBatch, ba);
    compute(m + kGradBatch, bb);
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
  const float scale = G.scale;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = j0 + jj;
    if (j >= r) break;
    if (G.msplit > 1) {
      float* dst = part + ((int64_t)z * r + j) * C;
      if (VEC && c0 + 4 <= C) {
        *reinterpret_cast<f32x4_t*>(dst + c0) = f32x4_t{acc[jj][0], acc[jj][1], acc[jj][2], acc[jj][3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (cv[e]) dst[c0 + e] = acc[jj][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!cv[e]) continue;
        if (cols_major) out[(c0 + e) * r + j] = scale * acc[jj][e];
        else out[(int64_t)j * C + c0 + e] = scale * acc[jj][e];
      }
    }
  }
}

// The same contraction on bf16 MFMA (16x16x32, float32 accumulation) for bf16 Q,
// computed as out^T[c][j] = sum_m Q[m][c] P[m][j]: Q^T is the A operand (its
// fragments, 8 consecutive rows of one column, come from the LDS transpose
// read of a row-major Q tile) and P the B operand.  P (float32) is split into
// hi = bf16(P) and lo = bf16(P - hi), multiplied as two MFMAs, which keeps
// about 16 significant bits of P.
//
// A workgroup owns 128 columns x up to 64 adapter rows (blockIdx: job, column
// tile, group of 64 adapter rows, M range); wave w the columns [32 w, 32 w + 32)
// as two 16-column MFMA tiles against every 16-row adapter tile, so no sums
// cross waves.  Per 32-row step the workgroup stages Q (32 x 128 bf16, 16-byte
// chunks XOR-swizzled by 2 h(row), h = row mod 4 + 4 (row / 8 mod 2), so the
// transpose reads of rows {q..q+3, q+8..q+11} hit distinct banks) and P
// (float32, transposed to [j][m], 144-byte rows) in one of two LDS buffers.
// Three steps of global loads are in flight; one barrier per step.
constexpr int kGmRows = 32;                  // rows of one step
constexpr int kGmChunk = 8;                  // steps of one straight-line chunk
constexpr uint32_t kGmQ = kGmRows * 256;     // Q tile bytes (32 rows x 128 bf16)
constexpr uint32_t kGmPRow = 144;            // one adapter row: 32 float32 + 16 pad
constexpr uint32_t kGmP = 64 * kGmPRow;      // P tile bytes (64 adapter rows)
constexpr uint32_t kGmBuf = kGmQ + kGmP;     // one buffer

__device__ __forceinline__ uint32_t gm_chunk(uint32_t row, uint32_t chunk) {
  const uint32_t h = (row & 3u) | (((row >> 3) & 1u) << 2);
  return chunk ^ (h << 1);
}

// The M range of a workgroup is walked in chunks of kGmChunk steps written as
// straight-line code (loads three steps ahead, fixed at compile time; steps past
// the range load zeros), so that the compiler's wait counts stay exact: a loop
// back-edge or a branch around a load makes it wait for every load in flight.
// PF: P is one split and r % 4 == 0 (one unconditional 16-byte load per item).
// NPL: P loads per thread and step (1 for r <= 32, else 2).
template <bool PF, int NPL>
__global__ __launch_bounds__(256) void k_lora_grad_mfma(GradParams G) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kGmBuf];
  const int ji = (G.nj > 1 && (int64_t)blockIdx.x >= G.J[1].tile0) ? 1 : 0;
  const float* __restrict__ P = G.J[ji].P;
  const uint16_t* __restrict__ Q = reinterpret_cast<const uint16_t*>(G.J[ji].Q);
  float* part = G.J[ji].part;
  float* out = G.J[ji].out;
  const int64_t C = G.J[ji].C;
  const int p_splits = G.J[ji].p_splits, cols_major = G.J[ji].cols_major, ctiles = G.J[ji].ctiles;
  const int64_t lt = (int64_t)blockIdx.x - G.J[ji].tile0;
  const int64_t ct = lt % ctiles, rest = lt / ctiles;
  const int jg = (int)(rest % G.jchunks), z = (int)(rest / G.jchunks);  // jchunks: groups of 64 here
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t M = G.M;
  const int r = G.r, j0 = 64 * jg;
  const int jt = min(4, (r - j0 + 15) / 16);  // 16-row adapter tiles of this group
  const int nq = 4 * jt;                      // float4 quads of one staged P row
  const int64_t mb = (int64_t)z * G.rows, me = min(M, mb + G.rows);
  const int64_t cb = ct * 128;

  // Q rows [mb, me) as a buffer resource: rows past me read as zero
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Q + mb * C), (short)0, (int)((me - mb) * C * 2), 0x00020000);
  // Q staging: round i (0, 1) -> tile row (tid >> 4) + 16 i, chunk tid & 15 (8 columns)
  const uint32_t qrow = (uint32_t)(tid >> 4), qch = (uint32_t)(tid & 15);
  const int64_t qcol = min<int64_t>(cb + 8 * qch, C - 8);  // clamped (outputs past C are dropped)

  struct Stage {
    u32x4_t q[2];
    f32x4_t p[NPL];
  };
  // P staging: item idx = tid + 256 i (i = 0, 1) -> row idx / nq, adapter rows
  // j0 + 4 (idx % nq) .. + 4; items past 32 nq idle
  auto load = [&](int64_t m0, Stage& st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = m0 - mb + qrow + 16 * i;
      const uint32_t off = (uint32_t)((row * C + qcol) * 2);
      st.q[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int idx = min(tid + 256 * i, 32 * nq - 1);  // items past 32 nq repeat the last one
      const int64_t m = min(m0 + idx / nq, me - 1);
      const int jb = j0 + 4 * (idx % nq);
      if constexpr (PF) {
        st.p[i] = *reinterpret_cast<const f32x4_t*>(P + m * r + min(jb, r - 4));
      } else {
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < p_splits; ++sp) {
          const float* pr = P + ((int64_t)sp * M + m) * r;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += pr[min(jb + e, r - 1)];
        }
        st.p[i] = v;
      }
    }
  };
  auto store = [&](int64_t m0, const Stage& st, uint32_t buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t row = qrow + 16u * i;
      *reinterpret_cast<u32x4_t*>(lds + buf + row * 256u + (gm_chunk(row, qch) << 4)) = st.q[i];
    }
    // threads past the 32 nq items store the clamped last item again: the same
    // value to the same place (an unconditional store keeps its load unconditional)
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int idx = min(tid + 256 * i, 32 * nq - 1);
      const int prow = idx / nq, q4 = idx % nq;
      const bool mv = m0 + prow < me;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = mv && j0 + 4 * q4 + e < r;
        *reinterpret_cast<float*>(lds + buf + kGmQ + (uint32_t)(4 * q4 + e) * kGmPRow + 4u * prow) =
            ok ? st.p[i][e] : 0.0f;
      }
    }
  };

  // fragment addresses: A (Q^T) by transpose reads, lane group g = lane / 16 takes
  // rows 8 g .. 8 g + 7; B (P) the float32 row j = 16 t + lane % 16, rows 8 g .. + 8
  const uint32_t g = (uint32_t)lane >> 4, sp = (uint32_t)lane & 15u;
  uint32_t qa[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t row = 8u * g + 4u * hf + (sp >> 2);
      const uint32_t col = 32u * w + 16u * c + 4u * (sp & 3u);  // element within the 128 columns
      qa[c][hf] = row * 256u + (gm_chunk(row, col >> 3) << 4) + 2u * (col & 7u);
    }
  const uint32_t pb = kGmQ + sp * kGmPRow + 32u * g;

  f32x4_t acc[2][4];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[c][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // three steps of loads in flight: step s is stored from register stage s % 4
  // while step s + 3 loads into stage (s + 3) % 4 (loads past the range are
  // harmless: Q reads zero there and P is clamped, then zeroed at store)
  Stage st[4];
  uint32_t buf = 0;
  auto step = [&](int64_t m0, const Stage& cur, Stage* nxt) {
    store(m0, cur, buf);
    if (nxt) load(m0 + 3 * kGmRows, *nxt);
    __syncthreads();
    u32x4_t a[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const s16x4_t lo = lds_tr16(lds + buf + qa[c][0]), hi = lds_tr16(lds + buf + qa[c][1]);
      a[c] = u32x4_t{__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                     __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t >= jt) break;
      const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(lds + buf + pb + 16u * t * kGmPRow);
      const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(lds + buf + pb + 16u * t * kGmPRow + 16u);
      const float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      u32x4_t bh, bl;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t h0 = f32_to_bf16_bits(pv[2 * e2]), h1 = f32_to_bf16_bits(pv[2 * e2 + 1]);
        bh[e2] = h0 | (h1 << 16);
        bl[e2] = pack_bf16x2(pv[2 * e2] - bf16_bits_to_f32(h0), pv[2 * e2 + 1] - bf16_bits_to_f32(h1));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        acc[c][t] = mfma16x16x32(as_bf16x8(a[c]), as_bf16x8(bh), acc[c][t]);
        acc[c][t] = mfma16x16x32(as_bf16x8(a[c]), as_bf16x8(bl), acc[c][t]);
      }
    }
    buf ^= kGmBuf;
  };
  for (int64_t c0 = mb; c0 < me; c0 += kGmChunk * kGmRows) {
    load(c0, st[0]);
    load(c0 + kGmRows, st[1]);
    load(c0 + 2 * kGmRows, st[2]);
#pragma unroll
    for (int k = 0; k < kGmChunk; ++k)
      step(c0 + k * kGmRows, st[k & 3], k + 3 < kGmChunk ? &st[(k + 3) & 3] : nullptr);
  }

  // D[c][j]: lane l holds columns c = 4 (l / 16) + v (v = 0..3) of adapter row j = l % 16
  const float scale = G.scale;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t >= jt) break;
    const int j = j0 + 16 * t + (int)sp;
    if (j >= r) continue;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t c0 = cb + 32 * w + 16 * c + 4 * (int64_t)g;
      if (G.msplit > 1) {
        float* dst = part + ((int64_t)z * r + j) * C + c0;
        if (c0 + 4 <= C) {
          *reinterpret_cast<f32x4_t*>(dst) = acc[c][t];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (c0 + v < C) dst[v] = acc[c][t][v];
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (c0 + v >= C) continue;
          if (cols_major) out[(c0 + v) * r + j] = scale * acc[c][t][v];
          else out[(int64_t)j * C + c0 + v] = scale * acc[c][t][v];
        }
      }
    }
  }
}

// out = s * (sum over the M ranges, in range order) of the partials.  A thread
// owns 4 consecutive columns of one adapter row (16-byte loads; C % 4 == 0,
// else one column), and eight ranges' loads are in flight at once.
template <bool V4>
__global__ __launch_bounds__(256) void k_lora_grad_reduce(GradParams G) {
  constexpr int W = V4 ? 4 : 1;
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * W;
  const int64_t n0 = (int64_t)G.r * G.J[0].C;
  const int ji = (G.nj > 1 && i0 >= n0) ? 1 : 0;
  const float* __restrict__ part = G.J[ji].part;
  float* out = G.J[ji].out;
  const int64_t C = G.J[ji].C;
  const int r = G.r, ms = G.msplit;
  const int64_t i = ji ? i0 - n0 : i0;
  if (i >= (int64_t)r * C) return;
  const int64_t j = i / C, c = i % C;
  const int64_t stride = (int64_t)r * C;
  using V = typename std::conditional<V4, f32x4_t, float>::type;
  V s = {};
  for (int z0 = 0; z0 < ms; z0 += 8) {
    V v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) v[b] = *reinterpret_cast<const V*>(part + (int64_t)min(z0 + b, ms - 1) * stride + i);
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (z0 + b < ms) s += v[b];
  }
  if constexpr (V4) {
    if (G.J[ji].cols_major) {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(c + e) * r + j] = G.scale * s[e];
    } else {
      *reinterpret_cast<f32x4_t*>(out + i) = G.scale * s;
    }
  } else {
    if (G.J[ji].cols_major) out[c * r + j] = G.scale * s;
    else out[i] = G.scale * s;
  }
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

// M ranges of the adapter-gradient kernels: enough workgroups to fill the chip,
// ranges of whole 32-row multiples.  The float32 kernel stages its P rows in
// LDS (64 bytes each), so its ranges hold at most kGradRowsMax rows.
constexpr int64_t kGradRowsMax = 1024;
void grad_split(int64_t M, int64_t N, int64_t K, int r, bool mfma, int* msplit, int64_t* rows) {
  const int64_t tiles = mfma ? ((K + 127) / 128 + (N + 127) / 128) * ((r + 63) / 64)
                             : ((K + 255) / 256 + (N + 255) / 256) * ((r + 15) / 16);
  const int64_t max_split = std::max<int64_t>(1, (M + 127) / 128);
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(max_split, (512 + tiles - 1) / tiles));
  int64_t rw = (M + want - 1) / want;
  const int64_t unit = mfma ? 256 : 32;  // the MFMA kernel walks whole chunks of 256 rows
  rw = std::max<int64_t>(unit, (rw + unit - 1) / unit * unit);
  if (!mfma) rw = std::min(rw, kGradRowsMax);
  *rows = rw;
  *msplit = (int)std::max<int64_t>(1, (M + rw - 1) / rw);
}

size_t grad_partial_floats(int64_t M, int64_t N, int64_t K, int r) {
  size_t most = 0;
  for (int mf = 0; mf < 2; ++mf) {
    int ms;
    int64_t rows;
    grad_split(M, N, K, r, mf == 1, &ms, &rows);
    if (ms > 1) most = std::max(most, (size_t)ms * (size_t)r * (size_t)(N + K));
  }
  return most;
}

template <int QDT, bool VEC>
hipError_t launch_grad_k(const GradParams& G, int64_t tiles, size_t shmem, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_lora_grad<QDT, VEC>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kGradRowsMax * 64));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_lora_grad<QDT, VEC>), dim3((unsigned)tiles), dim3(256), shmem, s, G);
  return hipGetLastError();
}

hipError_t launch_lora_grads(const float* u, int u_splits, const float* t, int t_splits, const void* x,
                             const void* dy, int qdt, bool mfma, int64_t M, int64_t N, int64_t K, int r,
                             float scale, float* dA, float* dB, float* part, hipStream_t s) {
  if (r == 0) return hipSuccess;
  if (M == 0) {
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((r * K + 255) / 256)), dim3(256), 0, s, dA, (int64_t)r * K);
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((r * N + 255) / 256)), dim3(256), 0, s, dB, (int64_t)r * N);
    return hipGetLastError();
  }
  if (mfma && (qdt != DT_BF16 || K % 8 != 0 || N % 8 != 0)) return hipErrorInvalidValue;
  const int cw = mfma ? 128 : 256;  // columns per workgroup
  GradParams G;
  G.M = M;
  G.r = r;
  G.jchunks = mfma ? (r + 63) / 64 : (r + 15) / 16;
  grad_split(M, N, K, r, mfma, &G.msplit, &G.rows);
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
  a.ctiles = (int32_t)((K + cw - 1) / cw);
  a.tile0 = 0;
  GradJob& b = G.J[1];
  b.P = t;
  b.p_splits = t_splits;
  b.Q = dy;
  b.C = N;
  b.part = part + (G.msplit > 1 ? (size_t)G.msplit * r * K : 0);
  b.out = dB;
  b.cols_major = 1;
  b.ctiles = (int32_t)((N + cw - 1) / cw);
  b.tile0 = (int64_t)a.ctiles * G.jchunks * G.msplit;
  const int64_t tiles = b.tile0 + (int64_t)b.ctiles * G.jchunks * G.msplit;
  hipError_t e;
  if (mfma) {
    // Q rows of one range are addressed with 32-bit buffer offsets
    if ((G.rows + 4 * kGmRows) * std::max(K, N) * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const bool pf = u_splits == 1 && t_splits == 1 && r % 4 == 0;
    const bool two = std::min(r, 64) > 32;
    if (pf && !two) hipLaunchKernelGGL((k_lora_grad_mfma<true, 1>), dim3((unsigned)tiles), dim3(256), 0, s, G);
    else if (pf) hipLaunchKernelGGL((k_lora_grad_mfma<true, 2>), dim3((unsigned)tiles), dim3(256), 0, s, G);
    else if (!two) hipLaunchKernelGGL((k_lora_grad_mfma<false, 1>), dim3((unsigned)tiles), dim3(256), 0, s, G);
    else hipLaunchKernelGGL((k_lora_grad_mfma<false, 2>), dim3((unsigned)tiles), dim3(256), 0, s, G);
    e = hipGetLastError();
  } else {
    const size_t shmem = (size_t)G.rows * 16 * sizeof(float);
    if (shmem > (size_t)kGradRowsMax * 64) return hipErrorInvalidValue;
    const bool vec = (K % 4) == 0 && (N % 4) == 0;
    if (qdt == DT_F32) e = vec ? launch_grad_k<DT_F32, true>(G, tiles, shmem, s) : launch_grad_k<DT_F32, false>(G, tiles, shmem, s);
    else e = vec ? launch_grad_k<DT_BF16, true>(G, tiles, shmem, s) : launch_grad_k<DT_BF16, false>(G, tiles, shmem, s);
  }
  if (e != hipSuccess || G.msplit == 1) return e;
  const int64_t outs = (int64_t)r * (K + N);
  if (K % 4 == 0 && N % 4 == 0)
    hipLaunchKernelGGL(k_lora_grad_reduce<true>, dim3((unsigned)((outs / 4 + 255) / 256)), dim3(256), 0, s, G);
  else
    hipLaunchKernelGGL(k_lora_grad_reduce<false>, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, G);
  return hipGetLastError();
}

}  // namespace qlr

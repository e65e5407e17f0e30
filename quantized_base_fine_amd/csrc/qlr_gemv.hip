// Decode path (M <= 16, bf16 x): the dequantizing GEMV of the frozen base with
// the unmerged adapter added in the epilogue.
//
// The frozen base is read once, as packed k-bit codes (QLoRA page,
// memory-decomposition equation: the 4-bit base takes about half a byte per
// weight), so the kernel is bound by HBM bandwidth; the dequantization the
// QLoRA page's limitations section mentions is fused into the load path.
//
// Work decomposition: a persistent grid of 1024-thread workgroups (one per CU)
// walks 16-row tiles of W; inside a workgroup the 16 waves split K (whole
// 64-element blocks) and are reduced through LDS at the end of every tile.
// Each wave streams its code slice in chunks of up to CH blocks and keeps one
// chunk in flight ahead of the one it computes, across tile boundaries too, so
// HBM requests stay outstanding while the previous tile is reduced.
//
// Layout on the 16x16x32 bf16 MFMA (A = x rows, B = unscaled levels):
//   lane l: x row / weight row (l & 15), lane group g = l >> 4 owns the 16
//   consecutive elements [16g, 16g+16) of each 64-element block; the first
//   MFMA takes elements [16g, 16g+8), the second [16g+8, 16g+16).  Both MFMAs
//   of a block stay inside that block, so the block's dequantized absmax
//   multiplies the 16x16 product afterwards (one FMA per output and block)
//   instead of every weight.
// Levels are looked up in a lane-private LDS table indexed by the packed code
// bits of two neighbouring weights (entry e of lane L at byte e*256 + 4L), so
// 64 lanes never collide on a bank; one table read yields a bf16 pair.
#include <algorithm>

#include "qlr_internal.h"
#include "qlr_lut.h"

namespace qlr {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int CH = 8;  // blocks per chunk and wave

// One chunk of a wave's stream: up to CH blocks of one 16-row tile.  Only raw
// loaded values live here: nothing is computed from them until the chunk is
// used, so a prefetched chunk never forces a wait on its loads.
template <int BITS>
struct Chunk {
  Raw<BITS> raw[CH];
  uint32_t q8[CH];
  float sc[CH];
};

struct Params {
  LinearArgs a;
  int64_t ntiles;
  int tlds;     // summed adapter product staged in LDS (M x r float32)
  int nparts;   // adapter partial sums: producers (fused) or K splits of the separate kernel
  float* tpart; // fused: nparts x M x r partials in the workspace (else a.t)
};

constexpr int kMaxFusedParts = 32;
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FUSED: the first P.nparts workgroups also compute the adapter product x A^T
// over one K-chunk each and publish it; every workgroup waits for all of them
// before its first epilogue.  The grid never exceeds one workgroup per CU, so
// all workgroups are resident together and the wait ends; it is also bounded.
template <int BITS, int YDT, bool XLDS, bool FUSED>
__global__ __launch_bounds__(kThreads, 1) void k_gemv(Params P, Levels lv) {
  extern __shared__ uint32_t smem[];
  const LinearArgs& a = P.a;
  const int64_t N = a.N, K = a.K, nb = K >> 6;
  const int M = (int)a.M;
  const int r = a.r;
  const int mr = M * r;
  uint32_t* tbl = smem;
  float* sRed = reinterpret_cast<float*>(smem + PairTable<BITS>::kBytes / 4);
  float* sL = sRed + kWaves * 256;  // codebook levels (256 floats)
  float* sT = sL + 256;
  uint16_t* sX = reinterpret_cast<uint16_t*>(sT + (P.tlds ? ((mr + 3) & ~3) : 0));  // 16-byte aligned
  const int64_t xstride = K + 8;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int64_t kb0 = nb * wave / kWaves, kb1 = nb * (wave + 1) / kWaves;
  const int nchunk = (int)((kb1 - kb0 + CH - 1) / CH);
  const int nitem = nchunk > 0 ? nchunk : 1;  // items (chunks) per tile for this wave
  const bool xvalid = nl < M;
  const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x) + (int64_t)(xvalid ? nl : 0) * K + 16 * g;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // ---- issue the first chunk's loads before the table build so they overlap it
  auto load_chunk = [&](int64_t tile, int c, Chunk<BITS>& ch) {
    const int64_t n = tile * 16 + nl;
    const int64_t blk_row = (n < N ? n : N - 1) * nb;
    const int64_t kbs = kb0 + (int64_t)c * CH;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int64_t kb = kbs + u;
      if (kb < kb1) {
        const int64_t blk = blk_row + kb;
        ch.raw[u] = load_raw<BITS>(a.codes + blk * (8 * BITS), g);
        ch.q8[u] = a.q8[blk];
        ch.sc[u] = a.cst[blk >> 8];
      }
    }
  };

  int64_t tile = blockIdx.x;
  int item = 0;
  Chunk<BITS> bufA, bufB;
  if (tile < P.ntiles) load_chunk(tile, 0, bufA);

  // ---- fused adapter product: this workgroup's K-chunk, at most one block per wave
  const bool producer = FUSED && (int)blockIdx.x < P.nparts;
  int64_t tkb = -1;
  u32x4_t af[4][2];
  if constexpr (FUSED) {
    if (producer) {
      const int64_t c = blockIdx.x;
      const int64_t b0 = nb * c / P.nparts, b1 = nb * (c + 1) / P.nparts;
      if (b0 + wave < b1) {
        tkb = b0 + wave;
        const uint16_t* Ap = reinterpret_cast<const uint16_t*>(a.A);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int j = jt * 16 + nl;
          if (j < r) {
            const uint16_t* q = Ap + (int64_t)j * K + tkb * 64 + 16 * g;
            af[jt][0] = *reinterpret_cast<const u32x4_t*>(q);
            af[jt][1] = *reinterpret_cast<const u32x4_t*>(q + 8);
          } else {
            af[jt][0] = zero;
            af[jt][1] = zero;
          }
        }
      }
    }
  }

  stage_levels<1 << BITS>(lv, sL);
  __syncthreads();
  build_table<BITS>(tbl, sL, tid, kThreads);
  if constexpr (XLDS) {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);
    const int64_t per_row = K / 8;  // 16-byte pieces per row
    for (int64_t i = tid; i < (int64_t)M * per_row; i += kThreads) {
      const int64_t m = i / per_row, q = i % per_row;
      *reinterpret_cast<uint4*>(sX + m * xstride + q * 8) = *reinterpret_cast<const uint4*>(x + m * K + q * 8);
    }
  }
  __syncthreads();

  auto x_frag = [&](int64_t kb, u32x4_t& x0, u32x4_t& x1) {
    x0 = zero;
    x1 = zero;
    if (xvalid) {
      if constexpr (XLDS) {
        const uint16_t* xs = sX + (int64_t)nl * xstride + kb * 64 + 16 * g;
        x0 = *reinterpret_cast<const u32x4_t*>(xs);
        x1 = *reinterpret_cast<const u32x4_t*>(xs + 8);
      } else {
        x0 = *reinterpret_cast<const u32x4_t*>(xg + kb * 64);
        x1 = *reinterpret_cast<const u32x4_t*>(xg + kb * 64 + 8);
      }
    }
  };

  // ---- fused adapter product: reduce over waves, publish the partial sum
  if constexpr (FUSED) {
    if (producer) {
      f32x4_t at[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) at[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (tkb >= 0) {
        u32x4_t x0, x1;
        x_frag(tkb, x0, x1);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          at[jt] = mfma16x16x32(as_bf16x8(x0), as_bf16x8(af[jt][0]), at[jt]);
          at[jt] = mfma16x16x32(as_bf16x8(x1), as_bf16x8(af[jt][1]), at[jt]);
        }
      }
      float* dst = P.tpart + (int64_t)blockIdx.x * mr;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt * 16 < r) {
#pragma unroll
          for (int v = 0; v < 4; ++v) sRed[wave * 256 + lane * 4 + v] = at[jt][v];
          __syncthreads();
          if (tid < 256) {
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) sum += sRed[w * 256 + tid];
            const int l = tid >> 2, v = tid & 3;
            const int m = 4 * (l >> 4) + v, j = jt * 16 + (l & 15);
            if (m < M && j < r)
              __hip_atomic_store(dst + m * r + j, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          __syncthreads();
        }
      }
      // each thread's (agent-scope) stores complete, then one agent-scope release
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(&a.sync->arrive, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // sT[i] = sum over parts of src[part][i], in part order, staged through sRed
  auto stage_t = [&](const float* src, int nparts) {
    const int per = mr > 0 ? max(1, (kWaves * 256) / mr) : 1;
    for (int p0 = 0; p0 < nparts; p0 += per) {
      const int np = min(per, nparts - p0);
      for (int idx = tid; idx < np * mr; idx += kThreads) sRed[idx] = coherent_load(src + (int64_t)p0 * mr + idx);
      __syncthreads();
      for (int i = tid; i < mr; i += kThreads) {
        float acc = (p0 == 0) ? 0.0f : sT[i];
        for (int q = 0; q < np; ++q) acc += sRed[q * mr + i];
        sT[i] = acc;
      }
      __syncthreads();
    }
  };

  bool t_ready = !P.tlds || r == 0;
  if (!FUSED && !t_ready) {
    stage_t(a.t, P.nparts);
    t_ready = true;
  }

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Chunk<BITS>& ch, int64_t tl, int c) {
    const bool nvalid = tl * 16 + nl < N;
    const int64_t kbs = kb0 + (int64_t)c * CH;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int64_t kb = kbs + u;
      if (kb < kb1) {
        u32x4_t x0, x1;
        x_frag(kb, x0, x1);
        u32x4_t b0, b1;
        decode16<BITS>(ch.raw[u], tbl, lane4, b0, b1);
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
        d = mfma16x16x32(as_bf16x8(x0), as_bf16x8(b0), d);
        d = mfma16x16x32(as_bf16x8(x1), as_bf16x8(b1), d);
        const float ap = nvalid ? (float)ch.q8[u] * ch.sc[u] : 0.0f;
        acc[0] = fmaf(ap, d[0], acc[0]);
        acc[1] = fmaf(ap, d[1], acc[1]);
        acc[2] = fmaf(ap, d[2], acc[2]);
        acc[3] = fmaf(ap, d[3], acc[3]);
      }
    }
  };

  // reduce the 16 K slices of a finished tile and write its outputs
  auto finish_tile = [&](int64_t tl) {
    if (FUSED && !t_ready) {
      // all adapter partials published? (one lane polls, the workgroup waits on it)
      // Poll with relaxed loads (an acquire on every poll would invalidate the
      // cache under the in-flight code stream), then acquire once.
      if (tid == 0) {
        uint32_t it = 0;
        while (__hip_atomic_load(&a.sync->arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               (uint32_t)P.nparts) {
          __builtin_amdgcn_s_sleep(2);
          if (++it == kSpinLimit) {
            __hip_atomic_store(&a.sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
      stage_t(P.tpart, P.nparts);
      t_ready = true;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) sRed[wave * 256 + lane * 4 + v] = acc[v];
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (tid < 256) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += sRed[w * 256 + tid];
      const int l = tid >> 2, v = tid & 3;
      const int m = 4 * (l >> 4) + v;  // MFMA output row (x row)
      const int64_t nn = tl * 16 + (l & 15);
      if (m < M && nn < N) {
        float lo = 0.0f;
        if (r > 0) {
          const uint16_t* br = reinterpret_cast<const uint16_t*>(a.B) + nn * r;
          if (P.tlds) {
            const float* tr = sT + m * r;
            for (int j = 0; j < r; ++j) lo = fmaf(tr[j], bf16_bits_to_f32(br[j]), lo);
          } else {
            for (int j = 0; j < r; ++j) {
              float tj = 0.0f;
              for (int sp = 0; sp < P.nparts; ++sp) tj += a.t[((int64_t)sp * M + m) * r + j];
              lo = fmaf(tj, bf16_bits_to_f32(br[j]), lo);
            }
          }
        }
        const float out = fmaf(a.scale, lo, s);
        if constexpr (YDT == DT_F32) reinterpret_cast<float*>(a.y)[(int64_t)m * N + nn] = out;
        else reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * N + nn] = (uint16_t)f32_to_bf16_bits(out);
      }
    }
    __syncthreads();
  };

  // One item: prefetch the stream's next chunk into `fill`, compute `use`.
  auto step = [&](const Chunk<BITS>& use, Chunk<BITS>& fill) {
    const bool last = (item + 1 == nitem);
    const int64_t ntile = last ? tile + gridDim.x : tile;
    const int nitm = last ? 0 : item + 1;
    if (ntile < P.ntiles) load_chunk(ntile, nitm, fill);
    compute(use, tile, item);
    if (last) finish_tile(tile);
    tile = ntile;
    item = nitm;
  };

  // ping-pong between two register buffers (no copies of in-flight loads)
  while (tile < P.ntiles) {
    step(bufA, bufB);
    if (tile >= P.ntiles) break;
    step(bufB, bufA);
  }

  if constexpr (FUSED) {
    // the last workgroup past its wait resets the words for the next call
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&a.sync->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == gridDim.x) {
        __hip_atomic_store(&a.sync->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.sync->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

constexpr size_t kLdsMax = 160 * 1024;

int device_cus() {
  static int cus = 0;  // one device per process
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cus = std::max(n, 1);
    else
      return 1;
  }
  return cus;
}

template <int BITS, int YDT, bool XLDS, bool FUSED>
hipError_t launch_k(const Params& P, int64_t grid, size_t shmem, const Levels& lv, hipStream_t s) {
  auto kern = k_gemv<BITS, YDT, XLDS, FUSED>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), shmem, s, P, lv);
  return hipGetLastError();
}

template <int BITS, int YDT, bool FUSED>
hipError_t launch_x(const Params& P, int64_t grid, size_t with_t, bool xlds, size_t xbytes,
                    const Levels& lv, hipStream_t s) {
  if (xlds) return launch_k<BITS, YDT, true, FUSED>(P, grid, with_t + xbytes, lv, s);
  return launch_k<BITS, YDT, false, FUSED>(P, grid, with_t, lv, s);
}

template <int BITS, int YDT>
hipError_t launch_gemv_b(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  Params P;
  P.a = a;
  P.ntiles = (a.N + 15) / 16;
  const int64_t grid = std::min<int64_t>(P.ntiles, device_cus());
  const bool fused = gemv_fuses_adapter(a.M, a.N, a.K, a.r, a.xdt, a.abdt);
  const size_t base = PairTable<BITS>::kBytes + (size_t)(kWaves + 1) * 256 * sizeof(float);
  const size_t tbytes = (((size_t)a.M * (size_t)a.r + 3) & ~(size_t)3) * sizeof(float);
  P.tlds = (a.r > 0 && base + tbytes <= kLdsMax) ? 1 : 0;
  if (fused) {
    P.nparts = gemv_adapter_parts(a.N, a.K);
    P.tpart = reinterpret_cast<float*>(reinterpret_cast<char*>(a.sync) + kSyncBytes);
  } else {
    P.nparts = a.t_splits;
    P.tpart = nullptr;
  }
  const size_t with_t = base + (P.tlds ? tbytes : 0);
  const size_t xbytes = (size_t)a.M * (size_t)(a.K + 8) * 2;
  const bool xlds = with_t + xbytes <= kLdsMax;
  if (fused) return launch_x<BITS, YDT, true>(P, grid, with_t, xlds, xbytes, lv, s);
  return launch_x<BITS, YDT, false>(P, grid, with_t, xlds, xbytes, lv, s);
}

template <int BITS>
hipError_t launch_gemv_y(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  if (a.ydt == DT_F32) return launch_gemv_b<BITS, DT_F32>(a, lv, s);
  return launch_gemv_b<BITS, DT_BF16>(a, lv, s);
}

}  // namespace

int gemv_adapter_parts(int64_t N, int64_t K) {
  const int64_t nb = K / 64;
  const int64_t grid = std::min<int64_t>((N + 15) / 16, device_cus());
  return (int)std::min<int64_t>(std::min<int64_t>(kMaxFusedParts, nb), grid);
}

bool gemv_fuses_adapter(int64_t M, int64_t N, int64_t K, int r, int xdt, int abdt) {
  if (!(r > 0 && r <= 64 && M * r <= 256 && xdt == DT_BF16 && abdt == DT_BF16)) return false;
  const int64_t nb = K / 64;
  const int64_t parts = gemv_adapter_parts(N, K);
  return parts > 0 && parts * kWaves >= nb;  // at most one block per producer wave
}

hipError_t launch_gemv(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_gemv_y<2>(a, lv, s);
    case 3: return launch_gemv_y<3>(a, lv, s);
    case 4: return launch_gemv_y<4>(a, lv, s);
    default: return launch_gemv_y<8>(a, lv, s);
  }
}

}  // namespace qlr

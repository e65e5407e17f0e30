// Decode path (M <= 16, bf16 x): the dequantizing GEMV of the frozen base with
// the unmerged adapter added in the epilogue (t = x A^T comes from the
// adapter-product kernel launched just before; measured on this chip, a second
// launch costs less than handing t between workgroups of one launch, whose
// cross-XCD round trips sit on the critical path).
//
// The frozen base is read once, as packed k-bit codes (QLoRA page,
// memory-decomposition equation: the 4-bit base takes about half a byte per
// weight), so the kernel is bound by HBM bandwidth; the dequantization the
// QLoRA page's limitations section mentions is fused into the load path.
//
// Work decomposition: a persistent grid of 512-thread workgroups (one per CU)
// walks 16-row tiles of W; inside a workgroup the 8 waves split K (whole
// 64-element blocks) and are reduced through LDS at the end of every tile.
// Each wave streams its K slice in chunks of 4 blocks and keeps the next chunk
// in flight (in registers) while it computes the current one, across tile
// boundaries too.
//
// Loads are shaped for the vector memory pipeline, which serves a group of 4
// consecutive lanes per cycle when they read one 64-byte segment: the code
// bytes of a chunk (16 rows x 4 blocks) are read as 16-byte pieces, 8
// consecutive lanes per row, through a buffer resource (rows past N read as
// zero), and staged in a wave-private LDS slice; the absmax codes and group
// constants are read one (row, block) per lane, 4 consecutive blocks of a row
// per lane quad, turned into scales and staged beside them.
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

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int CH = 4;  // blocks per chunk and wave

// Per-chunk geometry for BITS-bit codes: the code bytes of 16 rows x CH blocks
// are loaded as PB-byte pieces (8 bytes for 3-bit codes, whose 24-byte blocks
// are only 8-byte aligned) and staged with a row stride RS chosen to keep the
// MFMA-layout reads within 2-way bank conflicts.
template <int BITS>
struct ChunkGeo {
  static constexpr int kRowBytes = CH * 8 * BITS;
  static constexpr int PB = (BITS == 3) ? 8 : 16;
  static constexpr int PR = kRowBytes / PB;          // pieces per row
  static constexpr int NP = (16 * PR + 63) / 64;     // pieces per lane
  static constexpr int RS = kRowBytes + (BITS == 8 ? 16 : 8);
  static constexpr int kStage = 16 * RS + 16 * CH * 4;  // codes + scales, one buffer
};

// One chunk of a wave's stream held in registers between its loads and its
// staging: raw code pieces, the (row, block) absmax code and group constant of
// this lane, and the x fragments of the chunk's blocks.
template <int BITS, bool XLDS>
struct Chunk {
  u32x4_t piece[ChunkGeo<BITS>::NP];
  uint32_t q8;
  float sc;
  u32x4_t x[XLDS ? 1 : CH][2];  // x fragments (unused when x is staged in LDS)
};

// Largest x (bytes) staged once per workgroup in LDS instead of being read per
// chunk in the MFMA layout (which repeats every x row 16 times per wave).
constexpr size_t kXLdsMax = 32 * 1024;

struct Params {
  LinearArgs a;
  int64_t ntiles;
  int tlds;     // summed adapter product staged in LDS (M x r float32)
};



// LDS byte address in the dynamic block (which starts at LDS address 0: the
// kernel has no static LDS).
__device__ __forceinline__ u32x4_t lds_rd128(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((uintptr_t)addr);
}
__device__ __forceinline__ void lds_wr128(uint32_t addr, u32x4_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>((uintptr_t)addr) = v;
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_rd64(uint32_t addr) {
  const u32x2_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>((uintptr_t)addr);
  return uint2{v.x, v.y};
}
__device__ __forceinline__ void lds_wr64(uint32_t addr, uint2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>((uintptr_t)addr) = u32x2_t{v.x, v.y};
}
__device__ __forceinline__ uint32_t lds_rd32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((uintptr_t)addr);
}
__device__ __forceinline__ uint32_t lds_rd16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>((uintptr_t)addr);
}

// Raw codes of lane group g (16 codes) of block u of staged row at `row_addr`.
template <int BITS>
__device__ __forceinline__ Raw<BITS> raw_from_lds(uint32_t row_addr, int u, int g) {
  Raw<BITS> r;
  const uint32_t ad = row_addr + (uint32_t)(u * 8 * BITS + g * 2 * BITS);
  if constexpr (BITS == 2) {
    r.v = lds_rd32(ad);
  } else if constexpr (BITS == 4) {
    const uint2 v = lds_rd64(ad);
    r.a = v.x; r.b = v.y;
  } else if constexpr (BITS == 8) {
    const u32x4_t v = lds_rd128(ad);
    r.a = v[0]; r.b = v[1]; r.c = v[2]; r.d = v[3];
  } else {
    r.lo = lds_rd16(ad) | (lds_rd16(ad + 2) << 16);
    r.hi = lds_rd16(ad + 4);
  }
  return r;
}

// The lane-private pair table, built straight from the by-value levels:
// thread t of wave w writes entry e = w + 8 i (i = 0, 1, ...) of its lane's copy,
// so the level indices are uniform across the wave and the levels are read
// with scalar loads (no LDS round trip per entry).
template <int BITS>
__device__ __forceinline__ void build_table_kernarg(uint32_t* tbl, const Levels& lv, int tid) {
  constexpr int NL = 1 << BITS;
  constexpr int E = PairTable<BITS>::kEntries;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll 4
  for (int e = w; e < E; e += kWaves) {
    uint32_t v;
    if constexpr (BITS == 8) v = f32_to_bf16_bits(lv.v[e]);
    else v = pack_bf16x2(lv.v[e & (NL - 1)], lv.v[e >> BITS]);
    tbl[e * 64 + lane] = v;
  }
}

// ADP: the call has an adapter branch (r > 0); calls without one run a separate
// instantiation, which also gives it its own kernel name.
template <int BITS, int YDT, bool XLDS, bool ADP>
__global__ __launch_bounds__(kThreads, 1) void k_gemv(Params P, Levels lv) {
  using G = ChunkGeo<BITS>;
  using Ch = Chunk<BITS, XLDS>;
  extern __shared__ uint32_t smem[];
  const LinearArgs& a = P.a;
  const int64_t N = a.N, K = a.K, nb = K >> 6;
  const int M = (int)a.M;
  const int r = a.r;
  const int mr = M * r;
  uint32_t* tbl = smem;
  // LDS: level table | per-wave staging (2 buffers) | sRed (waves x 256) | sT | sX
  const uint32_t stage0 = (uint32_t)PairTable<BITS>::kBytes;
  float* sRed = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + stage0 + kWaves * 2 * G::kStage);
  float* sT = sRed + kWaves * 256;
  const uint32_t sX = (uint32_t)((reinterpret_cast<char*>(sT) - reinterpret_cast<char*>(smem)) +
                                 (P.tlds ? ((mr + 3) & ~3) * 4 : 0));  // LDS byte address, 16-byte aligned

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int64_t kb0 = nb * wave / kWaves, kb1 = nb * (wave + 1) / kWaves;
  const int nchunk = (int)((kb1 - kb0 + CH - 1) / CH);
  const int nitem = nchunk > 0 ? nchunk : 1;  // items (chunks) per tile for this wave
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // x row of this lane's A fragments (rows past M are zeroed after the load)
  const bool xvalid = nl < M;
  const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x) + (int64_t)(xvalid ? nl : M - 1) * K + 16 * g;
  // code bytes as a buffer resource: pieces past the end read as zero
  const int64_t code_bytes = N * nb * 8 * BITS;
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.codes), (short)0, (int)code_bytes, 0x00020000);
  const uint32_t wstage = stage0 + (uint32_t)wave * 2 * G::kStage;
  // scale-loading lane: (row lane / 4, block lane % 4) of a chunk
  const int srow = lane >> 2, sblk = lane & 3;

  auto load_chunk = [&](int64_t tile, int c, Ch& ch) {
    const int64_t kbs = kb0 + (int64_t)c * CH;
    // code pieces: piece p -> row p / PR, byte (p % PR) * PB of the chunk row
#pragma unroll
    for (int i = 0; i < G::NP; ++i) {
      const int p = i * 64 + lane;
      const int row = p / G::PR, col = p % G::PR;
      const int64_t off = ((tile * 16 + row) * nb + kbs) * (8 * BITS) + (int64_t)col * G::PB;
      const bool in = (p < 16 * G::PR) && (tile * 16 + row < N);
      const uint32_t o32 = in ? (uint32_t)off : 0xFFFFFFF0u;  // out-of-range offsets read zero
      if constexpr (G::PB == 16) {
        ch.piece[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cr, o32, 0, 0));
      } else {
        const u32x2_t w2 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(cr, o32, 0, 0));
        ch.piece[i] = u32x4_t{w2.x, w2.y, 0u, 0u};
      }
    }
    // scale of (row srow, block kbs + sblk), clamped into the matrix
    {
      const int64_t n = tile * 16 + srow;
      const int64_t kb = min(kbs + sblk, nb - 1);
      const int64_t blk = (n < N ? n : N - 1) * nb + kb;
      ch.q8 = a.q8[blk];
      ch.sc = a.cst[blk >> 8];
    }
    // x fragments of the chunk's blocks (clamped into the row; unused past kb1)
    if constexpr (!XLDS) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int64_t kb = min(kbs + u, nb - 1);
        ch.x[u][0] = *reinterpret_cast<const u32x4_t*>(xg + kb * 64);
        ch.x[u][1] = *reinterpret_cast<const u32x4_t*>(xg + kb * 64 + 8);
      }
    }
  };

  // Small x: one coalesced copy into LDS per workgroup (rows at stride K + 8),
  // loaded before the code stream so that waiting for it does not wait for codes.
  constexpr int kXPer = (int)(kXLdsMax / 16 / kThreads);  // 16-byte pieces per thread (4)
  u32x4_t xst[kXPer];
  const int64_t xpieces = (int64_t)M * (K / 8);
  if constexpr (XLDS) {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int64_t q = tid + (int64_t)i * kThreads;
      const int64_t qc = q < xpieces ? q : 0;
      xst[i] = *reinterpret_cast<const u32x4_t*>(x + qc * 8);
    }
  }

  int64_t tile = blockIdx.x;
  int item = 0;
  Ch bufA, bufB;
  if (tile < P.ntiles) load_chunk(tile, 0, bufA);

  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int64_t q = tid + (int64_t)i * kThreads;
      if (q < xpieces) {
        const int64_t m = q / (K / 8), c8 = q % (K / 8);
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(
            (uintptr_t)(sX + (uint32_t)((m * (K + 8) + c8 * 8) * 2))) = xst[i];
      }
    }
  }
  build_table_kernarg<BITS>(tbl, lv, tid);
  __syncthreads();

  // sT[i] = sum over parts of src[part][i], in part order, staged through sRed
  auto stage_t = [&](const float* src, int nparts) {
    const int per = mr > 0 ? max(1, (kWaves * 256) / mr) : 1;
    for (int p0 = 0; p0 < nparts; p0 += per) {
      const int np = min(per, nparts - p0);
      for (int idx = tid; idx < np * mr; idx += kThreads) sRed[idx] = src[(int64_t)p0 * mr + idx];
      __syncthreads();
      for (int i = tid; i < mr; i += kThreads) {
        float acc = (p0 == 0) ? 0.0f : sT[i];
        for (int q = 0; q < np; ++q) acc += sRed[q * mr + i];
        sT[i] = acc;
      }
      __syncthreads();
    }
  };

  // t = x A^T (written by the previous kernel) summed into LDS; the code
  // stream is already in flight, so this round trip overlaps it
  if (ADP && P.tlds) stage_t(a.t, a.t_splits);

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};

  // Stage a chunk's codes and scales in this wave's LDS buffer `buf` (only this
  // wave reads them, and a wave's LDS instructions run in order), then compute.
  auto compute = [&](const Ch& ch, int64_t tl, int c, int buf) {
    const uint32_t sb = wstage + (uint32_t)buf * G::kStage;
#pragma unroll
    for (int i = 0; i < G::NP; ++i) {
      const int p = i * 64 + lane;
      if (p < 16 * G::PR) {
        const uint32_t ad = sb + (uint32_t)((p / G::PR) * G::RS + (p % G::PR) * G::PB);
        if constexpr (G::PB == 16) lds_wr128(ad, ch.piece[i]);
        else lds_wr64(ad, uint2{ch.piece[i][0], ch.piece[i][1]});
      }
    }
    const uint32_t sscale = sb + 16 * G::RS;
    {
      const bool nvalid = tl * 16 + srow < N;
      const float ap = nvalid ? (float)ch.q8 * ch.sc : 0.0f;
      *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)(sscale + (uint32_t)(srow * CH + sblk) * 4)) = ap;
    }
    const u32x4_t aps = lds_rd128(sscale + (uint32_t)nl * (CH * 4));
    const uint32_t rowad = sb + (uint32_t)nl * G::RS;
    const int64_t kbs = kb0 + (int64_t)c * CH;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (kbs + u < kb1) {
        u32x4_t x0, x1;
        if constexpr (XLDS) {
          const uint32_t xa = sX + (uint32_t)((nl * (K + 8) + (kbs + u) * 64 + 16 * g) * 2);
          x0 = xvalid ? lds_rd128(xa) : zero;
          x1 = xvalid ? lds_rd128(xa + 16) : zero;
        } else {
          x0 = xvalid ? ch.x[u][0] : zero;
          x1 = xvalid ? ch.x[u][1] : zero;
        }
        u32x4_t b0, b1;
        decode16<BITS>(raw_from_lds<BITS>(rowad, u, g), tbl, lane4, b0, b1);
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
        d = mfma16x16x32(as_bf16x8(x0), as_bf16x8(b0), d);
        d = mfma16x16x32(as_bf16x8(x1), as_bf16x8(b1), d);
        const float ap = __uint_as_float(aps[u]);
        acc[0] = fmaf(ap, d[0], acc[0]);
        acc[1] = fmaf(ap, d[1], acc[1]);
        acc[2] = fmaf(ap, d[2], acc[2]);
        acc[3] = fmaf(ap, d[3], acc[3]);
      }
    }
  };

  // reduce the K slices of a finished tile and write its outputs
  auto finish_tile = [&](int64_t tl) {
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
        if (ADP) {
          const uint16_t* br = reinterpret_cast<const uint16_t*>(a.B) + nn * r;
          if (P.tlds) {
            const float* tr = sT + m * r;
            for (int j = 0; j < r; ++j) lo = fmaf(tr[j], bf16_bits_to_f32(br[j]), lo);
          } else {
            for (int j = 0; j < r; ++j) {
              float tj = 0.0f;
              for (int sp = 0; sp < a.t_splits; ++sp) tj += a.t[((int64_t)sp * M + m) * r + j];
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
  int buf = 0;
  auto step = [&](const Ch& use, Ch& fill) {
    const bool last = (item + 1 == nitem);
    const int64_t ntile = last ? tile + gridDim.x : tile;
    const int nitm = last ? 0 : item + 1;
    if (ntile < P.ntiles) load_chunk(ntile, nitm, fill);
    if (nchunk > 0) compute(use, tile, item, buf);
    buf ^= 1;
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

template <int BITS, int YDT, bool XLDS, bool ADP>
hipError_t launch_k(const Params& P, int64_t grid, size_t shmem, const Levels& lv, hipStream_t s) {
  auto kern = k_gemv<BITS, YDT, XLDS, ADP>;
  static bool attr = false;
  if (!attr) {
    // the kernel addresses LDS from 0: it must not have static LDS
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsMax);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), shmem, s, P, lv);
  return hipGetLastError();
}

template <int BITS, int YDT>
hipError_t launch_gemv_b(const LinearArgs& a, const Levels& lv, hipStream_t s) {
  Params P;
  P.a = a;
  P.ntiles = (a.N + 15) / 16;
  // code bytes are addressed with 32-bit buffer offsets
  if (a.N * (a.K / 64) * 8 * a.bits >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const int64_t grid = std::min<int64_t>(P.ntiles, device_cus());
  const size_t base = PairTable<BITS>::kBytes + (size_t)kWaves * 2 * ChunkGeo<BITS>::kStage +
                      (size_t)kWaves * 256 * sizeof(float);
  const size_t tbytes = (((size_t)a.M * (size_t)a.r + 3) & ~(size_t)3) * sizeof(float);
  P.tlds = (a.r > 0 && base + tbytes <= kLdsMax) ? 1 : 0;
  const size_t with_t = base + (P.tlds ? tbytes : 0);
  // x staged in LDS (rows at stride K + 8 bf16) when small enough
  const size_t xbytes = (size_t)a.M * (size_t)(a.K + 8) * 2;
  const bool xlds = (size_t)a.M * (size_t)a.K * 2 <= kXLdsMax && with_t + xbytes <= kLdsMax;
  if (a.r > 0) {
    if (xlds) return launch_k<BITS, YDT, true, true>(P, grid, with_t + xbytes, lv, s);
    return launch_k<BITS, YDT, false, true>(P, grid, with_t, lv, s);
  }
  if (xlds) return launch_k<BITS, YDT, true, false>(P, grid, with_t + xbytes, lv, s);
  return launch_k<BITS, YDT, false, false>(P, grid, with_t, lv, s);
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

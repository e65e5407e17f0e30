// Host side of the qlr C ABI: argument validation, codebook construction,
// size and workspace queries, and dispatch onto the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "qlr.h"
#include "qlr_internal.h"

namespace {

thread_local std::string t_error;
thread_local qlr_path t_path = QLR_PATH_AUTO;

qlr_status fail(qlr_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_error = buf;
  return s;
}

qlr_status hip_fail(hipError_t e, const char* what) {
  return fail(QLR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- codebook
//
// QLoRA page, section "1. 4-bit NormalFloat (NF4) quantization": level i is
// the standard-normal quantile at (i + 1/2) / 2^b (0-based), divided by the
// largest such quantile so the levels span [-1, 1]; the lower half is computed
// and mirrored.  The quantile is found by bisection on Phi(z) = erfc(-z/sqrt2)/2
// in long double (64-bit significand) and each level is rounded once to float.

long double normal_cdf(long double z) { return 0.5L * std::erfc(-z / std::sqrt(2.0L)); }

long double normal_quantile(long double p) {
  long double lo = -40.0L, hi = 40.0L;
  for (int it = 0; it < 400; ++it) {
    const long double mid = 0.5L * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (normal_cdf(mid) < p) lo = mid;
    else hi = mid;
  }
  return 0.5L * (lo + hi);
}

struct CodebookCache {
  std::once_flag once[9];
  float levels[9][256];
};
CodebookCache g_cb;

const float* codebook_levels(int bits) {
  std::call_once(g_cb.once[bits], [bits]() {
    const int n = 1 << bits;
    const long double top = normal_quantile((2.0L * n - 1.0L) / (2.0L * n));
    float* L = g_cb.levels[bits];
    for (int i = 0; i < n / 2; ++i) {
      const long double z = normal_quantile((2.0L * i + 1.0L) / (2.0L * n));
      L[i] = (float)(z / top);
      L[n - 1 - i] = -L[i];
    }
  });
  return g_cb.levels[bits];
}

qlr::Levels levels_arg(int bits) {
  qlr::Levels lv;
  std::memset(&lv, 0, sizeof(lv));
  std::memcpy(lv.v, codebook_levels(bits), sizeof(float) << bits);
  return lv;
}

// ---------------------------------------------------------------- validation

bool bits_ok(int32_t bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t dtype_size(qlr_dtype d) { return d == QLR_F32 ? 4 : 2; }
bool dtype_ok(int d) { return d == QLR_F32 || d == QLR_F16 || d == QLR_BF16; }

void sizes_of(int64_t rows, int64_t cols, int bits, size_t* cb, size_t* qb, size_t* kb) {
  const int64_t numel = rows * cols;
  const int64_t nblk = (numel + QLR_BLOCK - 1) / QLR_BLOCK;
  const int64_t ngrp = (nblk + QLR_GROUP - 1) / QLR_GROUP;
  *cb = (size_t)nblk * 8 * (size_t)bits;
  *qb = (size_t)nblk;
  *kb = (size_t)ngrp * 4;
}

qlr_status check_qweight(const qlr_qweight* w) {
  if (!w) return fail(QLR_ERR_NULL, "qweight is NULL");
  if (w->format_version != QLR_FORMAT_VERSION)
    return fail(QLR_ERR_FORMAT, "format_version %u, expected %u", w->format_version, QLR_FORMAT_VERSION);
  if (!bits_ok(w->bits)) return fail(QLR_ERR_BITS, "bits %d not in {2,3,4,8}", w->bits);
  if (w->block != QLR_BLOCK || w->group != QLR_GROUP)
    return fail(QLR_ERR_BLOCK, "block %d / group %d, expected 64 / 256", w->block, w->group);
  if (w->rows < 0 || w->cols < 0) return fail(QLR_ERR_SHAPE, "negative rows/cols");
  if (w->rows > 0 && w->cols > (INT64_C(1) << 40) / w->rows) return fail(QLR_ERR_SHAPE, "weight too large");
  if (!w->codes || !w->absmax_q8 || !w->absmax_c) return fail(QLR_ERR_NULL, "qweight buffer is NULL");
  if (!aligned16(w->codes) || !aligned16(w->absmax_q8) || !aligned16(w->absmax_c))
    return fail(QLR_ERR_ALIGN, "qweight buffers must be 16-byte aligned");
  return QLR_OK;
}

// Workspace of one linear call: the adapter product x A^T as `splits` float32
// partial sums (M x r each) from the adapter-product kernel.  The count depends
// only on M and K (the bf16 count bounds the others).
size_t linear_ws_bytes(int64_t M, int64_t K, int32_t r) {
  if (M <= 0 || r <= 0) return 0;
  const size_t parts = (size_t)qlr::lora_t_splits(M, K, r, qlr::DT_BF16, qlr::DT_BF16);
  return ((parts * (size_t)M * (size_t)r * sizeof(float)) + 255) & ~(size_t)255;
}

// Workspace of one backward call, as four 256-byte-aligned regions: t = x A^T
// and u = dy B as float32 partial splits (the bf16 counts bound the others),
// B transposed (r x N, 4-byte elements bound both dtypes), and the float32
// partials of the adapter gradients.
struct BwdLayout {
  size_t t, u, bt, part, total;
};
BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdLayout L{0, 0, 0, 0, 0};
  if (r <= 0) return L;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t mr = (size_t)std::max<int64_t>(M, 0) * (size_t)r * sizeof(float);
  const size_t st = M > 0 ? (size_t)qlr::lora_t_splits(M, K, r, qlr::DT_BF16, qlr::DT_BF16) : 0;
  const size_t su = M > 0 ? (size_t)qlr::lora_t_splits(M, N, r, qlr::DT_BF16, qlr::DT_BF16) : 0;
  L.t = 0;
  L.u = L.t + up(st * mr);
  L.bt = L.u + up(su * mr);
  L.part = L.bt + up((size_t)r * (size_t)N * 4);
  L.total = L.part + up(M > 0 ? qlr::grad_partial_floats(M, N, K, r) * sizeof(float) : 0);
  return L;
}

// Workspace of a double-binary adapter call: t2 (splits x M x 2lR float32) and
// Beff (N x 2lR bf16), 256-byte aligned.
struct DbaLayout {
  size_t t2, beff, total;
  int splits;
};
DbaLayout dba_layout(int64_t M, int64_t N, int64_t K, int R, int ell, int xdt) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  DbaLayout L;
  L.splits = M > 0 ? qlr::dba_t_splits(M, K, xdt, R, ell) : 1;
  const size_t lr2 = 2 * (size_t)R * (size_t)ell;
  L.t2 = 0;
  L.beff = up((size_t)L.splits * (size_t)std::max<int64_t>(M, 0) * lr2 * 4);
  L.total = L.beff + up((size_t)N * lr2 * 2);
  return L;
}

// choose the kernel family for a linear call
// The Walsh-Hadamard branch is merged into the weight on the prefill GEMM when
// the bf16 copy fits the dense-weight GEMM's 32-bit offsets.
bool wha_merges(int64_t N, int64_t K) { return N > 0 && K > 0 && N <= (int64_t)0x7FFFFFFF / 2 / K; }

qlr_status pick_path(int64_t M, qlr_dtype xdt, qlr_dtype abdt, int32_t r, qlr_path* out) {
  const bool bf16_ok = xdt == QLR_BF16 && (r == 0 || abdt == QLR_BF16);
  qlr_path p = t_path;
  if (p == QLR_PATH_AUTO) {
    if (!bf16_ok) p = QLR_PATH_F32;
    else p = (M <= 16) ? QLR_PATH_GEMV : QLR_PATH_GEMM;
  }
  if ((p == QLR_PATH_GEMV || p == QLR_PATH_GEMM) && !bf16_ok)
    return fail(QLR_ERR_PATH, "the MFMA paths need bf16 x and bf16 adapters");
  if (p == QLR_PATH_GEMV && M > 16) return fail(QLR_ERR_PATH, "the GEMV path takes M <= 16");
  *out = p;
  return QLR_OK;
}

struct LinearCheck {
  const void* x;
  qlr_dtype xdt;
  int64_t M;
  const qlr_qweight* w;
  const void* A;
  const void* B;
  qlr_dtype abdt;
  int32_t r;
  void* y;
  qlr_dtype ydt;
};

qlr_status check_linear(const LinearCheck& c) {
  qlr_status st = check_qweight(c.w);
  if (st != QLR_OK) return st;
  if (c.M < 0) return fail(QLR_ERR_SHAPE, "M < 0");
  if (c.r < 0) return fail(QLR_ERR_SHAPE, "r < 0");
  if (c.w->cols % QLR_BLOCK != 0) return fail(QLR_ERR_SHAPE, "cols %lld is not a multiple of 64", (long long)c.w->cols);
  if (c.w->rows == 0 || c.w->cols == 0) return fail(QLR_ERR_SHAPE, "empty weight");
  if (!(c.xdt == QLR_F32 || c.xdt == QLR_BF16)) return fail(QLR_ERR_DTYPE, "x dtype must be f32 or bf16");
  if (!(c.ydt == QLR_F32 || c.ydt == QLR_BF16)) return fail(QLR_ERR_DTYPE, "y dtype must be f32 or bf16");
  if (c.r > 0 && !(c.abdt == QLR_F32 || c.abdt == QLR_BF16)) return fail(QLR_ERR_DTYPE, "adapter dtype must be f32 or bf16");
  if (c.M > 0) {
    if (!c.x || !c.y) return fail(QLR_ERR_NULL, "x or y is NULL");
    if (!aligned16(c.x) || !aligned16(c.y)) return fail(QLR_ERR_ALIGN, "x and y must be 16-byte aligned");
  }
  if (c.r > 0) {
    if (!c.A || !c.B) return fail(QLR_ERR_NULL, "A or B is NULL with r > 0");
    if (!aligned16(c.A) || !aligned16(c.B)) return fail(QLR_ERR_ALIGN, "A and B must be 16-byte aligned");
  }
  return QLR_OK;
}

qlr::LinearArgs make_args(const LinearCheck& c, float scale, char* ws, int splits) {
  qlr::LinearArgs a;
  a.x = c.x;
  a.xdt = (int)c.xdt;
  a.M = c.M;
  a.N = c.w->rows;
  a.K = c.w->cols;
  a.bits = c.w->bits;
  a.codes = reinterpret_cast<const uint8_t*>(c.w->codes);
  a.q8 = c.w->absmax_q8;
  a.cst = c.w->absmax_c;
  a.t = reinterpret_cast<const float*>(ws);
  a.t_splits = splits;
  a.A = c.A;
  a.B = c.B;
  a.abdt = (int)c.abdt;
  a.r = c.r;
  a.scale = scale;
  a.y = c.y;
  a.ydt = (int)c.ydt;
  return a;
}

// The sparse side channel, when given, is summed inside the decode kernel (the
// caller has checked sparse_fused); addend is the alternative, a precomputed term.
qlr_status run_linear(const LinearCheck& c, float scale, char* ws, qlr_path path, hipStream_t s,
                      const float* addend = nullptr, const qlr_sparse* sp = nullptr, int wht_lp = -1) {
  if (c.M == 0) return QLR_OK;
  hipError_t e = hipSuccess;
  const int splits = qlr::lora_t_splits(c.M, c.w->cols, c.r, (int)c.xdt, (int)c.abdt);
  qlr::LinearArgs a = make_args(c, scale, ws, splits);
  a.addend = addend;
  if (sp) {
    a.sp_row_ptr = sp->row_ptr;
    a.sp_col = sp->col;
    a.sp_val = sp->val;
    a.sp_nnz = sp->nnz;
    a.sp_wht_lp = wht_lp;
    a.sp_gemm = path == QLR_PATH_GEMM && wht_lp < 0;
  }
  if (c.r > 0 && !(path == QLR_PATH_GEMV && qlr::gemv_fuses_adapter(a))) {
    e = qlr::launch_lora_t(c.x, (int)c.xdt, c.M, c.w->cols, c.A, (int)c.abdt, c.r,
                           reinterpret_cast<float*>(ws), splits, s);
    if (e != hipSuccess) return hip_fail(e, "adapter product launch");
  }
  const qlr::Levels lv = levels_arg(c.w->bits);
  switch (path) {
    case QLR_PATH_F32: e = qlr::launch_linear_f32(a, lv, s); break;
    case QLR_PATH_GEMV: e = qlr::launch_gemv(a, lv, s); break;
    default: e = qlr::launch_gemm(a, lv, s); break;
  }
  if (e != hipSuccess) return hip_fail(e, "linear launch");
  return QLR_OK;
}

qlr_status quantize_common(const void* W, qlr_dtype wdt, int64_t rows, int64_t cols, int32_t bits,
                           int32_t block, qlr_qweight* out, void* ws, size_t ws_bytes,
                           hipStream_t s) {
  if (!W || !out) return fail(QLR_ERR_NULL, "W or out is NULL");
  if (!dtype_ok(wdt)) return fail(QLR_ERR_DTYPE, "W dtype must be f32, f16 or bf16");
  if (!bits_ok(bits)) return fail(QLR_ERR_BITS, "bits %d not in {2,3,4,8}", bits);
  if (block != QLR_BLOCK) return fail(QLR_ERR_BLOCK, "block %d, expected 64", block);
  if (rows <= 0 || cols <= 0) return fail(QLR_ERR_SHAPE, "rows and cols must be positive");
  if (out->rows != rows || out->cols != cols || out->bits != bits || out->block != block)
    return fail(QLR_ERR_SHAPE, "out header does not match rows/cols/bits/block");
  qlr_status st = check_qweight(out);
  if (st != QLR_OK) return st;
  if (!aligned16(W)) return fail(QLR_ERR_ALIGN, "W must be 16-byte aligned");
  if (!ws || ws_bytes < 256) return fail(QLR_ERR_WORKSPACE, "workspace of at least 256 bytes required");
  if (!aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  uint32_t* flag = reinterpret_cast<uint32_t*>(ws);
  hipError_t e = qlr::launch_fill_u32(flag, 0u, 1, s);
  if (e != hipSuccess) return hip_fail(e, "flag clear");
  const qlr::Levels lv = levels_arg(bits);
  e = qlr::launch_quantize(W, (int)wdt, rows * cols, bits, lv, reinterpret_cast<uint8_t*>(out->codes),
                           out->absmax_q8, out->absmax_c, flag, s);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return QLR_OK;
}

}  // namespace

// ---------------------------------------------------------------- allocation-free forward scratch
//
// The scratch of qlr_linear_fwd_static (the adapter product's float32 partial
// sums): one array per GPU, allocated with the code object when the library is
// first used on that GPU and held until the process ends.  Host code never uses
// the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept
// per device.
static __device__ __align__(256) unsigned char scratch[QLR_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that owns `stream`.
qlr_status scratch_for_stream(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(QLR_ERR_HIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return hip_fail(e2, "hipSetDevice");
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(QLR_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLR_OK;
}

}  // namespace

extern "C" {

int qlr_version(void) { return 100; }

const char* qlr_status_string(qlr_status s) {
  switch (s) {
    case QLR_OK: return "ok";
    case QLR_ERR_NULL: return "null pointer";
    case QLR_ERR_SHAPE: return "bad shape";
    case QLR_ERR_DTYPE: return "unsupported dtype";
    case QLR_ERR_BITS: return "unsupported bit width";
    case QLR_ERR_BLOCK: return "unsupported block or group size";
    case QLR_ERR_ALIGN: return "misaligned pointer";
    case QLR_ERR_NONFINITE: return "non-finite weight";
    case QLR_ERR_WORKSPACE: return "workspace too small";
    case QLR_ERR_ALIAS: return "overlapping buffers";
    case QLR_ERR_HIP: return "HIP error";
    case QLR_ERR_FORMAT: return "unknown qweight format";
    case QLR_ERR_PATH: return "path cannot run these arguments";
  }
  return "unknown status";
}

const char* qlr_last_error(void) { return t_error.c_str(); }

qlr_status qlr_codebook(int32_t bits, float* out) {
  if (!out) return fail(QLR_ERR_NULL, "out is NULL");
  if (!bits_ok(bits)) return fail(QLR_ERR_BITS, "bits %d not in {2,3,4,8}", bits);
  std::memcpy(out, codebook_levels(bits), sizeof(float) << bits);
  return QLR_OK;
}

qlr_status qlr_qweight_sizes(int64_t rows, int64_t cols, int32_t bits, int32_t block,
                             size_t* codes_bytes, size_t* absmax_q8_bytes, size_t* absmax_c_bytes) {
  if (!codes_bytes || !absmax_q8_bytes || !absmax_c_bytes) return fail(QLR_ERR_NULL, "output pointer is NULL");
  if (rows < 0 || cols < 0) return fail(QLR_ERR_SHAPE, "negative rows/cols");
  if (!bits_ok(bits)) return fail(QLR_ERR_BITS, "bits %d not in {2,3,4,8}", bits);
  if (block != QLR_BLOCK) return fail(QLR_ERR_BLOCK, "block %d, expected 64", block);
  if (rows > 0 && cols > (INT64_C(1) << 40) / rows) return fail(QLR_ERR_SHAPE, "weight too large");
  sizes_of(rows, cols, bits, codes_bytes, absmax_q8_bytes, absmax_c_bytes);
  return QLR_OK;
}

qlr_status qlr_workspace_bytes(qlr_op op, int64_t M, int64_t N, int64_t K, int32_t r, size_t* bytes) {
  (void)N;
  (void)K;
  if (!bytes) return fail(QLR_ERR_NULL, "bytes is NULL");
  if (op == QLR_OP_QUANTIZE) {
    *bytes = 256;
    return QLR_OK;
  }
  if (op == QLR_OP_QUANTIZE_OUTLIERS) {
    // N = rows, K = cols, M = the outlier count
    if (M < 0 || N < 0 || K < 0) return fail(QLR_ERR_SHAPE, "negative size");
    *bytes = std::max<size_t>(256, qlr::outlier_ws_bytes(N * K, M) + 256);
    return QLR_OK;
  }
  if (op == QLR_OP_LINEAR_OUTLIERS) {
    if (M < 0 || N < 0 || K < 0 || r < 0) return fail(QLR_ERR_SHAPE, "negative size");
    *bytes = linear_ws_bytes(M, K, r) + (((size_t)M * (size_t)N * 4 + 255) & ~(size_t)255);
    return QLR_OK;
  }
  if (op == QLR_OP_LINEAR_WHA) {
    if (M < 0 || N < 0 || K < 0) return fail(QLR_ERR_SHAPE, "negative size");
    // the float32 addend (M x N), or on the prefill GEMM the merged bf16 weight (N x K)
    size_t b = ((size_t)M * (size_t)N * 4 + 255) & ~(size_t)255;
    const bool gemm = t_path == QLR_PATH_GEMM || (t_path == QLR_PATH_AUTO && M > 16);
    if (M > 0 && gemm && wha_merges(N, K)) b = std::max(b, ((size_t)N * (size_t)K * 2 + 255) & ~(size_t)255);
    *bytes = b;
    return QLR_OK;
  }
  if (op == QLR_OP_LINEAR_DBA) {
    // r = ell * R of the double-binary adapter; the bf16 split count bounds the others
    if (M < 0 || N < 0 || K < 0 || r < 1) return fail(QLR_ERR_SHAPE, "negative size or r < 1");
    const int64_t lr2 = 2 * (int64_t)r;
    const size_t splits = M > 0 ? (size_t)qlr::dba_t_splits(M, K, qlr::DT_BF16, r, 1) : 1;
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    *bytes = up(splits * (size_t)M * (size_t)lr2 * 4) + up((size_t)N * (size_t)lr2 * 2);
    return QLR_OK;
  }
  if (op != QLR_OP_LINEAR && op != QLR_OP_LINEAR_BWD) return fail(QLR_ERR_SHAPE, "unknown op %d", (int)op);
  if (M < 0 || r < 0) return fail(QLR_ERR_SHAPE, "negative M or r");
  if (op == QLR_OP_LINEAR_BWD) {
    if (N < 0 || K < 0) return fail(QLR_ERR_SHAPE, "negative N or K");
    *bytes = bwd_layout(M, N, K, r).total;
    return QLR_OK;
  }
  *bytes = linear_ws_bytes(M, K, r);
  return QLR_OK;
}

qlr_status qlr_quantize_async(const void* W, qlr_dtype wdt, int64_t rows, int64_t cols, int32_t bits,
                              int32_t block, qlr_qweight* out, void* ws, size_t ws_bytes, void* stream) {
  return quantize_common(W, wdt, rows, cols, bits, block, out, ws, ws_bytes,
                         reinterpret_cast<hipStream_t>(stream));
}

qlr_status qlr_quantize(const void* W, qlr_dtype wdt, int64_t rows, int64_t cols, int32_t bits,
                        int32_t block, qlr_qweight* out, void* ws, size_t ws_bytes, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  qlr_status st = quantize_common(W, wdt, rows, cols, bits, block, out, ws, ws_bytes, s);
  if (st != QLR_OK) return st;
  uint32_t flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, ws, sizeof(flag), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "flag read");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  if (flag != 0) return fail(QLR_ERR_NONFINITE, "W holds NaN or Inf");
  return QLR_OK;
}

qlr_status qlr_dequantize(const qlr_qweight* w, void* out, qlr_dtype odt, void* stream) {
  qlr_status st = check_qweight(w);
  if (st != QLR_OK) return st;
  if (!out) return fail(QLR_ERR_NULL, "out is NULL");
  if (!(odt == QLR_F32 || odt == QLR_BF16)) return fail(QLR_ERR_DTYPE, "output dtype must be f32 or bf16");
  if (!aligned16(out)) return fail(QLR_ERR_ALIGN, "out must be 16-byte aligned");
  const int64_t numel = w->rows * w->cols;
  if (numel == 0) return QLR_OK;
  const qlr::Levels lv = levels_arg(w->bits);
  hipError_t e = qlr::launch_dequantize(reinterpret_cast<const uint8_t*>(w->codes), w->absmax_q8, w->absmax_c,
                                        numel, w->bits, lv, out, (int)odt,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return QLR_OK;
}

qlr_status qlr_linear_fwd(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w, const void* A,
                          const void* B, qlr_dtype abdt, int32_t r, float scale, void* y, qlr_dtype ydt,
                          void* ws, size_t ws_bytes, void* stream) {
  const LinearCheck c{x, xdt, M, w, A, B, abdt, r, y, ydt};
  qlr_status st = check_linear(c);
  if (st != QLR_OK) return st;
  const size_t need = linear_ws_bytes(M, w->cols, r);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QLR_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : (size_t)0);
  if (need > 0 && !aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  qlr_path path;
  st = pick_path(M, xdt, abdt, r, &path);
  if (st != QLR_OK) return st;
  return run_linear(c, scale, reinterpret_cast<char*>(ws), path, reinterpret_cast<hipStream_t>(stream));
}

qlr_status qlr_linear_fwd_static(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w, const void* A,
                                 const void* B, qlr_dtype abdt, int32_t r, float scale, void* y, qlr_dtype ydt,
                                 void* stream) {
  const LinearCheck c{x, xdt, M, w, A, B, abdt, r, y, ydt};
  qlr_status st = check_linear(c);
  if (st != QLR_OK) return st;
  const size_t need = linear_ws_bytes(M, w->cols, r);
  if (need > (size_t)QLR_STATIC_SCRATCH_BYTES)
    return fail(QLR_ERR_WORKSPACE, "the call needs %zu bytes of scratch; the static area holds %zu (use qlr_linear_fwd)",
                need, (size_t)QLR_STATIC_SCRATCH_BYTES);
  qlr_path path;
  st = pick_path(M, xdt, abdt, r, &path);
  if (st != QLR_OK) return st;
  if (M == 0) return QLR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_stream(s, &ws);
    if (st != QLR_OK) return st;
  }
  return run_linear(c, scale, reinterpret_cast<char*>(ws), path, s);
}

qlr_status qlr_linear_fwd_mixed(const qlr_layer* layers, int32_t n, int64_t M, qlr_dtype xdt, qlr_dtype abdt,
                                qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream) {
  if (n < 0) return fail(QLR_ERR_SHAPE, "n < 0");
  if (n > 0 && !layers) return fail(QLR_ERR_NULL, "layers is NULL");
  size_t need = 0;
  std::vector<std::pair<uintptr_t, uintptr_t>> outs, ins;
  for (int32_t i = 0; i < n; ++i) {
    const qlr_layer& L = layers[i];
    const LinearCheck c{L.x, xdt, M, L.w, L.A, L.B, abdt, L.r, L.y, ydt};
    qlr_status st = check_linear(c);
    if (st != QLR_OK) return fail(st, "layer %d: %s", i, t_error.c_str());
    qlr_path path;
    st = pick_path(M, xdt, abdt, L.r, &path);
    if (st != QLR_OK) return fail(st, "layer %d: %s", i, t_error.c_str());
    need += linear_ws_bytes(M, L.w->cols, L.r);
    if (M > 0) {
      const uintptr_t y0 = reinterpret_cast<uintptr_t>(L.y);
      outs.push_back({y0, y0 + (uintptr_t)(M * L.w->rows) * dtype_size(ydt)});
      const uintptr_t x0 = reinterpret_cast<uintptr_t>(L.x);
      ins.push_back({x0, x0 + (uintptr_t)(M * L.w->cols) * dtype_size(xdt)});
    }
    if (L.r > 0) {
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(L.A), b0 = reinterpret_cast<uintptr_t>(L.B);
      ins.push_back({a0, a0 + (uintptr_t)((int64_t)L.r * L.w->cols) * dtype_size(abdt)});
      ins.push_back({b0, b0 + (uintptr_t)((int64_t)L.r * L.w->rows) * dtype_size(abdt)});
    }
  }
  auto overlap = [](const std::pair<uintptr_t, uintptr_t>& p, const std::pair<uintptr_t, uintptr_t>& q) {
    return p.first < q.second && q.first < p.second;
  };
  for (size_t i = 0; i < outs.size(); ++i) {
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j])) return fail(QLR_ERR_ALIAS, "outputs %zu and %zu overlap", i, j);
    for (size_t j = 0; j < ins.size(); ++j)
      if (overlap(outs[i], ins[j])) return fail(QLR_ERR_ALIAS, "output %zu overlaps an input", i);
  }
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QLR_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  if (need > 0 && !aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* wsp = reinterpret_cast<char*>(ws);
  // GEMM-path layers run as grouped launches (one code width and adapter flag
  // per group, in layer order), after their adapter products; at M = 1 the
  // single-row decode layers run as grouped launches too (one code width per
  // group), after their adapter products in grouped launches; the others one by one
  std::vector<qlr::LinearArgs> groups[2][4];
  std::vector<qlr::LinearArgs> dgroups[4];
  std::vector<qlr::LoraTItem> tgroup, tsmall;
  auto widx = [](int bits) { return bits == 2 ? 0 : bits == 3 ? 1 : bits == 4 ? 2 : 3; };
  for (int32_t i = 0; i < n; ++i) {
    const qlr_layer& L = layers[i];
    const LinearCheck c{L.x, xdt, M, L.w, L.A, L.B, abdt, L.r, L.y, ydt};
    qlr_path path;
    pick_path(M, xdt, abdt, L.r, &path);
    const size_t need_l = linear_ws_bytes(M, L.w->cols, L.r);
    char* wl = need_l > 0 ? wsp : nullptr;
    wsp += need_l;
    if (path == QLR_PATH_GEMV && M == 1) {
      const int splits = qlr::lora_t_splits(M, L.w->cols, L.r, (int)xdt, (int)abdt);
      const qlr::LinearArgs a = make_args(c, L.scale, wl, splits);
      if (qlr::gemv_groupable(a)) {
        if (L.r > 0) tsmall.push_back(qlr::LoraTItem{L.x, L.A, reinterpret_cast<float*>(wl), L.w->cols, L.r, false});
        dgroups[widx(L.w->bits)].push_back(a);
        continue;
      }
    }
    if (path == QLR_PATH_GEMM && M > 0) {
      const int splits = qlr::lora_t_splits(M, L.w->cols, L.r, (int)xdt, (int)abdt);
      if (L.r > 0) {
        if (M > 16 && xdt == QLR_BF16 && abdt == QLR_BF16) {
          tgroup.push_back(qlr::LoraTItem{L.x, L.A, reinterpret_cast<float*>(wl), L.w->cols, L.r, false});
        } else {
          const hipError_t e = qlr::launch_lora_t(L.x, (int)xdt, M, L.w->cols, L.A, (int)abdt, L.r,
                                                  reinterpret_cast<float*>(wl), splits, s);
          if (e != hipSuccess) return hip_fail(e, "adapter product launch");
        }
      }
      groups[L.r > 0 ? 1 : 0][widx(L.w->bits)].push_back(make_args(c, L.scale, wl, splits));
      continue;
    }
    qlr_status st = run_linear(c, L.scale, wl, path, s);
    if (st != QLR_OK) return st;
  }
  // adapter products of the grouped decode layers, then their decode kernels
  for (size_t b = 0; b < tsmall.size(); b += qlr::lora_t_small_group_max()) {
    const int cnt = (int)std::min<size_t>(qlr::lora_t_small_group_max(), tsmall.size() - b);
    const hipError_t e = qlr::launch_lora_t_small_group(tsmall.data() + b, cnt, M, s);
    if (e != hipSuccess) return hip_fail(e, "grouped adapter product launch");
  }
  for (int w = 0; w < 4; ++w) {
    std::vector<qlr::LinearArgs>& g = dgroups[w];
    for (size_t b = 0; b < g.size(); b += qlr::gemv_group_max()) {
      const int cnt = (int)std::min<size_t>(qlr::gemv_group_max(), g.size() - b);
      const hipError_t e = qlr::launch_gemv_group(g.data() + b, cnt, levels_arg(g[b].bits), s);
      if (e != hipSuccess) return hip_fail(e, "grouped decode launch");
    }
  }
  // adapter products of the grouped layers, then their GEMMs
  for (size_t b = 0; b < tgroup.size(); b += qlr::lora_t_group_max()) {
    const int cnt = (int)std::min<size_t>(qlr::lora_t_group_max(), tgroup.size() - b);
    const hipError_t e = qlr::launch_lora_t_group(tgroup.data() + b, cnt, M, s);
    if (e != hipSuccess) return hip_fail(e, "grouped adapter product launch");
  }
  const int gmax = qlr::gemm_group_max();
  for (int ad = 0; ad < 2; ++ad)
    for (int w = 0; w < 4; ++w) {
      std::vector<qlr::LinearArgs>& g = groups[ad][w];
      // longest tiles (largest K) first: workgroups are dispatched in order, so
      // the short tiles fill in behind the long ones
      std::stable_sort(g.begin(), g.end(),
                       [](const qlr::LinearArgs& p, const qlr::LinearArgs& q) { return p.K > q.K; });
      for (size_t b = 0; b < g.size(); b += gmax) {
        const int cnt = (int)std::min<size_t>(gmax, g.size() - b);
        const hipError_t e = qlr::launch_gemm_group(g.data() + b, cnt, levels_arg(g[b].bits), s);
        if (e != hipSuccess) return hip_fail(e, "grouped linear launch");
      }
    }
  return QLR_OK;
}

qlr_status qlr_linear_bwd(const void* dy, qlr_dtype dydt, const void* x, qlr_dtype xdt, int64_t M,
                          const qlr_qweight* w, const void* A, const void* B, qlr_dtype abdt, int32_t r,
                          float scale, void* dx, qlr_dtype dxdt, float* dA, float* dB, void* ws,
                          size_t ws_bytes, void* stream) {
  qlr_status st = check_qweight(w);
  if (st != QLR_OK) return st;
  if (M < 0) return fail(QLR_ERR_SHAPE, "M < 0");
  if (r < 0) return fail(QLR_ERR_SHAPE, "r < 0");
  if (w->cols % QLR_BLOCK != 0) return fail(QLR_ERR_SHAPE, "cols %lld is not a multiple of 64", (long long)w->cols);
  if (w->rows == 0 || w->cols == 0) return fail(QLR_ERR_SHAPE, "empty weight");
  if (!(dydt == QLR_F32 || dydt == QLR_BF16)) return fail(QLR_ERR_DTYPE, "dy dtype must be f32 or bf16");
  if (!(dxdt == QLR_F32 || dxdt == QLR_BF16)) return fail(QLR_ERR_DTYPE, "dx dtype must be f32 or bf16");
  if (r > 0) {
    if (!(abdt == QLR_F32 || abdt == QLR_BF16)) return fail(QLR_ERR_DTYPE, "adapter dtype must be f32 or bf16");
    if (xdt != dydt) return fail(QLR_ERR_DTYPE, "x and dy must share a dtype when r > 0");
    if (!A || !B || !dA || !dB) return fail(QLR_ERR_NULL, "A, B, dA or dB is NULL with r > 0");
    if (!aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB))
      return fail(QLR_ERR_ALIGN, "A, B, dA and dB must be 16-byte aligned");
  }
  const int64_t N = w->rows, K = w->cols;
  if (M > 0) {
    if (!dy) return fail(QLR_ERR_NULL, "dy is NULL");
    if (r > 0 && !x) return fail(QLR_ERR_NULL, "x is NULL with r > 0");
    if (!aligned16(dy) || (dx && !aligned16(dx)) || (r > 0 && !aligned16(x)))
      return fail(QLR_ERR_ALIGN, "dy, x and dx must be 16-byte aligned");
  }
  // no output may overlap an input or another output
  {
    std::vector<std::pair<uintptr_t, uintptr_t>> outs, ins;
    auto span = [](const void* p, size_t n) {
      const uintptr_t a = reinterpret_cast<uintptr_t>(p);
      return std::make_pair(a, a + n);
    };
    if (M > 0 && dx) outs.push_back(span(dx, (size_t)(M * K) * dtype_size(dxdt)));
    if (r > 0) {
      outs.push_back(span(dA, (size_t)r * (size_t)K * 4));
      outs.push_back(span(dB, (size_t)r * (size_t)N * 4));
      ins.push_back(span(A, (size_t)r * (size_t)K * dtype_size(abdt)));
      ins.push_back(span(B, (size_t)r * (size_t)N * dtype_size(abdt)));
      if (M > 0) ins.push_back(span(x, (size_t)(M * K) * dtype_size(xdt)));
    }
    if (M > 0) ins.push_back(span(dy, (size_t)(M * N) * dtype_size(dydt)));
    auto overlap = [](const std::pair<uintptr_t, uintptr_t>& p, const std::pair<uintptr_t, uintptr_t>& q) {
      return p.first < q.second && q.first < p.second;
    };
    for (size_t i = 0; i < outs.size(); ++i) {
      for (size_t j = i + 1; j < outs.size(); ++j)
        if (overlap(outs[i], outs[j])) return fail(QLR_ERR_ALIAS, "two outputs overlap");
      for (const auto& in : ins)
        if (overlap(outs[i], in)) return fail(QLR_ERR_ALIAS, "an output overlaps an input");
    }
  }
  const BwdLayout lay = bwd_layout(M, N, K, r);
  if (lay.total > 0 && (!ws || ws_bytes < lay.total))
    return fail(QLR_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", lay.total, ws ? ws_bytes : (size_t)0);
  if (lay.total > 0 && !aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  // kernel family: the transposed bf16 GEMM needs bf16 operands and whole 64-row steps
  const bool bf16_ok = dydt == QLR_BF16 && (r == 0 || (xdt == QLR_BF16 && abdt == QLR_BF16)) && N % 64 == 0;
  qlr_path path = t_path;
  if (path == QLR_PATH_AUTO) path = bf16_ok ? QLR_PATH_GEMM : QLR_PATH_F32;
  if (path == QLR_PATH_GEMV) path = QLR_PATH_GEMM;
  if (path == QLR_PATH_GEMM && !bf16_ok)
    return fail(QLR_ERR_PATH, "the MFMA backward needs bf16 dy, x and adapters and rows %% 64 == 0");
  if (path == QLR_PATH_GEMM && M > 0 && qlr::gemm_max_rows_of(N) == 0)
    return fail(QLR_ERR_SHAPE, "rows too large for the MFMA backward");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* wsp = reinterpret_cast<char*>(ws);
  float* tws = r > 0 ? reinterpret_cast<float*>(wsp + lay.t) : nullptr;
  float* uws = r > 0 ? reinterpret_cast<float*>(wsp + lay.u) : nullptr;
  const int st_t = M > 0 ? qlr::lora_t_splits(M, K, r, (int)xdt, (int)abdt) : 1;
  const int st_u = M > 0 ? qlr::lora_t_splits(M, N, r, (int)dydt, (int)abdt) : 1;
  hipError_t e = hipSuccess;
  if (r > 0 && M > 0) {
    if (M > 16 && xdt == QLR_BF16 && abdt == QLR_BF16 && N % 64 == 0 && r % 8 == 0) {
      // t = x A^T and u = dy B as one grouped launch of the tiled product (B read as is)
      const qlr::LoraTItem items[2] = {{x, A, tws, K, r, false}, {dy, B, uws, N, r, true}};
      e = qlr::launch_lora_t_group(items, 2, M, s);
      if (e != hipSuccess) return hip_fail(e, "adapter products (x A^T, dy B) launch");
    } else {
      e = qlr::launch_transpose_nr(B, (int)abdt, N, r, wsp + lay.bt, s);
      if (e != hipSuccess) return hip_fail(e, "adapter transpose launch");
      e = qlr::launch_lora_t(x, (int)xdt, M, K, A, (int)abdt, r, tws, st_t, s);
      if (e != hipSuccess) return hip_fail(e, "adapter product (x A^T) launch");
      e = qlr::launch_lora_t(dy, (int)dydt, M, N, wsp + lay.bt, (int)abdt, r, uws, st_u, s);
      if (e != hipSuccess) return hip_fail(e, "adapter product (dy B) launch");
    }
  }
  if (dx && M > 0) {
    qlr::LinearArgs a;
    a.x = dy;
    a.xdt = (int)dydt;
    a.M = M;
    a.N = N;
    a.K = K;
    a.bits = w->bits;
    a.codes = reinterpret_cast<const uint8_t*>(w->codes);
    a.q8 = w->absmax_q8;
    a.cst = w->absmax_c;
    a.t = uws;
    a.t_splits = st_u;
    a.A = nullptr;
    a.B = A;
    a.abdt = (int)abdt;
    a.r = r;
    a.scale = scale;
    a.y = dx;
    a.ydt = (int)dxdt;
    const qlr::Levels lv = levels_arg(w->bits);
    e = path == QLR_PATH_F32 ? qlr::launch_dx_f32(a, lv, s) : qlr::launch_gemm_dx(a, lv, s);
    if (e != hipSuccess) return hip_fail(e, "input-gradient launch");
  }
  if (r > 0) {
    e = qlr::launch_lora_grads(uws, st_u, tws, st_t, x, dy, (int)xdt, path == QLR_PATH_GEMM, M, N, K, r, scale,
                               dA, dB, reinterpret_cast<float*>(wsp + lay.part), s);
    if (e != hipSuccess) return hip_fail(e, "adapter-gradient launch");
  }
  return QLR_OK;
}

qlr_status qlr_linear_fwd_dba(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w, const qlr_dba* ad,
                              void* y, qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream) {
  if (!ad) return fail(QLR_ERR_NULL, "adapter is NULL");
  if (ad->rank < 1 || ad->ell < 1 || (int64_t)ad->rank * ad->ell > 4096)
    return fail(QLR_ERR_SHAPE, "rank and ell must be >= 1 with rank * ell <= 4096");
  if (!ad->b1 || !ad->b2 || !ad->alpha || !ad->beta || !ad->gamma) return fail(QLR_ERR_NULL, "adapter array is NULL");
  if (!aligned16(ad->b1) || !aligned16(ad->b2) || !aligned16(ad->alpha) || !aligned16(ad->beta) ||
      !aligned16(ad->gamma))
    return fail(QLR_ERR_ALIGN, "adapter arrays must be 16-byte aligned");
  const LinearCheck c{x, xdt, M, w, nullptr, nullptr, QLR_BF16, 0, y, ydt};
  qlr_status st = check_linear(c);
  if (st != QLR_OK) return st;
  const int64_t N = w->rows, K = w->cols;
  const int R = ad->rank, ell = ad->ell;
  const DbaLayout lay = dba_layout(M, N, K, R, ell, (int)xdt);
  if (!ws || ws_bytes < lay.total)
    return fail(QLR_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", lay.total, ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  // the branch runs as an exact rank-2lR adapter of the bf16 kernels (B = Beff in bf16)
  const int32_t r2 = 2 * R * ell;
  qlr_path path;
  st = pick_path(M, xdt, QLR_BF16, r2, &path);
  if (st != QLR_OK) return st;
  if (M == 0) return QLR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* wsp = reinterpret_cast<char*>(ws);
  if (path == QLR_PATH_GEMV && ell == 1 && R <= 16) {
    // a single x row on the decode kernel: both stages of the branch inside it (scale 1, rank R)
    qlr::LinearArgs f = make_args(c, 1.0f, nullptr, 1);
    f.r = R;
    f.A = nullptr;
    f.B = nullptr;
    f.dba_b1 = ad->b1;
    f.dba_b2 = ad->b2;
    f.dba_alpha = ad->alpha;
    f.dba_beta = ad->beta;
    f.dba_gamma = ad->gamma;
    if (qlr::gemv_fuses_dba(f)) {
      const hipError_t e = qlr::launch_gemv(f, levels_arg(w->bits), s);
      if (e != hipSuccess) return hip_fail(e, "linear launch");
      return QLR_OK;
    }
  }
  const qlr::DbaArgs d{R, ell, ad->b1, ad->b2, ad->alpha, ad->beta, ad->gamma};
  float* t2 = reinterpret_cast<float*>(wsp + lay.t2);
  uint16_t* beff = reinterpret_cast<uint16_t*>(wsp + lay.beff);
  hipError_t e = qlr::launch_dba_prep(d, x, (int)xdt, M, N, K, t2, lay.splits, beff, s);
  if (e != hipSuccess) return hip_fail(e, "adapter stage launch");
  qlr::LinearArgs a = make_args(c, 1.0f, wsp + lay.t2, lay.splits);
  a.A = nullptr;
  a.B = beff;
  a.abdt = qlr::DT_BF16;
  a.r = r2;
  const qlr::Levels lv = levels_arg(w->bits);
  switch (path) {
    case QLR_PATH_F32: e = qlr::launch_linear_f32(a, lv, s); break;
    case QLR_PATH_GEMV: e = qlr::launch_gemv(a, lv, s); break;
    default: e = qlr::launch_gemm(a, lv, s); break;
  }
  if (e != hipSuccess) return hip_fail(e, "linear launch");
  return QLR_OK;
}

qlr_status qlr_quantize_outliers(const void* W, qlr_dtype wdt, int64_t rows, int64_t cols, int32_t bits,
                                 int32_t block, int64_t k, qlr_qweight* out, qlr_sparse* sp, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!W || !out || !sp) return fail(QLR_ERR_NULL, "W, out or sp is NULL");
  if (!dtype_ok(wdt)) return fail(QLR_ERR_DTYPE, "W dtype must be f32, f16 or bf16");
  if (!bits_ok(bits)) return fail(QLR_ERR_BITS, "bits %d not in {2,3,4,8}", bits);
  if (block != QLR_BLOCK) return fail(QLR_ERR_BLOCK, "block %d, expected 64", block);
  if (rows <= 0 || cols <= 0) return fail(QLR_ERR_SHAPE, "rows and cols must be positive");
  if (rows * cols >= (INT64_C(1) << 31)) return fail(QLR_ERR_SHAPE, "rows * cols must be below 2^31");
  if (k < 0 || k > rows * cols) return fail(QLR_ERR_SHAPE, "k must be in [0, rows * cols]");
  if (out->rows != rows || out->cols != cols || out->bits != bits || out->block != block)
    return fail(QLR_ERR_SHAPE, "out header does not match rows/cols/bits/block");
  qlr_status st = check_qweight(out);
  if (st != QLR_OK) return st;
  if (sp->rows != rows || sp->cols != cols || sp->nnz != k) return fail(QLR_ERR_SHAPE, "sp header does not match");
  if (!sp->row_ptr || (k > 0 && (!sp->col || !sp->val))) return fail(QLR_ERR_NULL, "sparse buffer is NULL");
  if (!aligned16(W) || !aligned16(sp->row_ptr) || (k > 0 && (!aligned16(sp->col) || !aligned16(sp->val))))
    return fail(QLR_ERR_ALIGN, "W and the sparse buffers must be 16-byte aligned");
  size_t need = 0;
  qlr_workspace_bytes(QLR_OP_QUANTIZE_OUTLIERS, k, rows, cols, 0, &need);
  if (!ws || ws_bytes < need) return fail(QLR_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  if (!aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const qlr::Levels lv = levels_arg(bits);
  hipError_t e;
  uint32_t* qflag = reinterpret_cast<uint32_t*>(ws);  // the dense quantize's non-finite flag
  char* rest = reinterpret_cast<char*>(ws) + 256;
  void* dense = const_cast<void*>(W);
  uint32_t* sflag = nullptr;
  int32_t* oidx = nullptr;
  float* oval = nullptr;
  e = qlr::launch_fill_u32(qflag, 0u, 1, s);
  if (e != hipSuccess) return hip_fail(e, "flag clear");
  if (k > 0) {
    e = qlr::launch_outlier_split(W, (int)wdt, rows * cols, k, rest, &dense, &sflag, &oidx, &oval, s);
    if (e != hipSuccess) return hip_fail(e, "outlier selection launch");
  }
  e = qlr::launch_quantize(dense, (int)wdt, rows * cols, bits, lv, reinterpret_cast<uint8_t*>(out->codes),
                           out->absmax_q8, out->absmax_c, qflag, s);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  e = qlr::launch_outlier_finish(rows, cols, k, bits, lv, reinterpret_cast<const uint8_t*>(out->codes),
                                 out->absmax_q8, out->absmax_c, oidx, oval, sp->row_ptr, sp->col, sp->val, s);
  if (e != hipSuccess) return hip_fail(e, "outlier finish launch");
  // the largest entry count of a 128-row group, read back with the flags
  uint32_t* gmax = qflag + 1;
  e = qlr::launch_group_max(rows, k, sp->row_ptr, gmax, s);
  if (e != hipSuccess) return hip_fail(e, "group count launch");
  uint32_t flags[3] = {0, 0, 0};
  e = hipMemcpyAsync(&flags[0], qflag, 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && sflag) e = hipMemcpyAsync(&flags[2], sflag, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "flag read");
  if (flags[0] || flags[2]) return fail(QLR_ERR_NONFINITE, "W holds NaN or Inf");
  sp->max_group_nnz = (int64_t)flags[1];
  return QLR_OK;
}

qlr_status qlr_linear_fwd_outliers(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w,
                                   const qlr_sparse* sp, const void* A, const void* B, qlr_dtype abdt, int32_t r,
                                   float scale, void* y, qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream) {
  if (!sp) return fail(QLR_ERR_NULL, "sp is NULL");
  const LinearCheck c{x, xdt, M, w, A, B, abdt, r, y, ydt};
  qlr_status st = check_linear(c);
  if (st != QLR_OK) return st;
  if (sp->rows != w->rows || sp->cols != w->cols || sp->nnz < 0) return fail(QLR_ERR_SHAPE, "sp does not match w");
  if (!sp->row_ptr || (sp->nnz > 0 && (!sp->col || !sp->val))) return fail(QLR_ERR_NULL, "sparse buffer is NULL");
  if (!aligned16(sp->row_ptr) || (sp->nnz > 0 && (!aligned16(sp->col) || !aligned16(sp->val))))
    return fail(QLR_ERR_ALIGN, "sparse buffers must be 16-byte aligned");
  size_t need = 0;
  qlr_workspace_bytes(QLR_OP_LINEAR_OUTLIERS, M, w->rows, w->cols, r, &need);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QLR_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : (size_t)0);
  if (need > 0 && !aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  qlr_path path;
  st = pick_path(M, xdt, abdt, r, &path);
  if (st != QLR_OK) return st;
  if (M == 0) return QLR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* wsp = reinterpret_cast<char*>(ws);
  // a single x row on the decode kernel: the side channel is summed inside it
  const qlr::LinearArgs probe = make_args(c, scale, wsp, qlr::lora_t_splits(M, w->cols, c.r, (int)xdt, (int)abdt));
  if (sp->nnz > 0 && path == QLR_PATH_GEMV && qlr::gemv_fuses_sparse(probe))
    return run_linear(c, scale, wsp, path, s, nullptr, sp);
  float* C = reinterpret_cast<float*>(wsp + linear_ws_bytes(M, w->cols, r));
  const float* addend = nullptr;
  // the prefill GEMM adds a 128-row tile's entries to its weights itself when they
  // fit (gemm_sparse_cap); the float32 addend then holds only the other tiles' rows
  const bool gemm_sp = path == QLR_PATH_GEMM && qlr::gemm_sparse_cap(w->bits) > 0;
  // when the split has said that every group's entries fit, no tile needs the addend
  // (a figure outside 1 .. nnz cannot be exact for nnz > 0: it counts as not known)
  const bool all_fit = gemm_sp && sp->max_group_nnz >= 1 && sp->max_group_nnz <= sp->nnz &&
                       sp->max_group_nnz <= qlr::gemm_sparse_cap(w->bits);
  if (sp->nnz > 0 && !all_fit) {
    const hipError_t e = qlr::launch_sparse_addend(x, (int)xdt, M, w->cols, w->rows, sp->row_ptr, sp->col, sp->val,
                                                   sp->nnz, C, s, gemm_sp ? qlr::gemm_sparse_cap(w->bits) : -1);
    if (e != hipSuccess) return hip_fail(e, "sparse term launch");
    addend = C;
  }
  return run_linear(c, scale, wsp, path, s, addend, gemm_sp && sp->nnz > 0 ? sp : nullptr);
}

qlr_status qlr_linear_fwd_wha(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w, const qlr_sparse* F,
                              int32_t hblock, void* y, qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream) {
  if (!F) return fail(QLR_ERR_NULL, "F is NULL");
  const LinearCheck c{x, xdt, M, w, nullptr, nullptr, QLR_BF16, 0, y, ydt};
  qlr_status st = check_linear(c);
  if (st != QLR_OK) return st;
  const int64_t K = w->cols;
  if (hblock < 1 || (hblock & (hblock - 1)) != 0 || K % hblock != 0)
    return fail(QLR_ERR_SHAPE, "hblock %d must be a power of two dividing cols %lld", hblock, (long long)K);
  if (K > qlr::wha_max_cols())
    return fail(QLR_ERR_SHAPE, "cols %lld above %lld (x rows are transformed in LDS)", (long long)K,
                (long long)qlr::wha_max_cols());
  if (F->rows != w->rows || F->cols != K || F->nnz < 0) return fail(QLR_ERR_SHAPE, "F does not match w");
  if (!F->row_ptr || (F->nnz > 0 && (!F->col || !F->val))) return fail(QLR_ERR_NULL, "F buffer is NULL");
  if (!aligned16(F->row_ptr) || (F->nnz > 0 && (!aligned16(F->col) || !aligned16(F->val))))
    return fail(QLR_ERR_ALIGN, "F buffers must be 16-byte aligned");
  size_t need = 0;
  qlr_workspace_bytes(QLR_OP_LINEAR_WHA, M, w->rows, K, 0, &need);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QLR_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : (size_t)0);
  if (need > 0 && !aligned16(ws)) return fail(QLR_ERR_ALIGN, "workspace must be 16-byte aligned");
  qlr_path path;
  st = pick_path(M, xdt, QLR_BF16, 0, &path);
  if (st != QLR_OK) return st;
  if (M == 0) return QLR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* C = reinterpret_cast<float*>(ws);
  const float* addend = nullptr;
  int lp = 0;
  while ((1 << lp) < hblock) ++lp;
  if (F->nnz > 0 && path == QLR_PATH_GEMV) {
    // a single x row on the decode kernel: the transform and the coefficients are summed inside it
    qlr::LinearArgs probe = make_args(c, 0.0f, nullptr, 1);
    probe.sp_row_ptr = F->row_ptr;
    probe.sp_col = F->col;
    probe.sp_val = F->val;
    probe.sp_nnz = F->nnz;
    probe.sp_wht_lp = lp;
    if (qlr::gemv_fuses_sparse(probe)) return run_linear(c, 0.0f, nullptr, path, s, nullptr, F, lp);
  }
  if (F->nnz > 0 && path == QLR_PATH_GEMM && wha_merges(w->rows, K)) {
    // prefill: the branch merged into a bf16 copy of the weight, then the dense-weight GEMM
    uint16_t* Wd = reinterpret_cast<uint16_t*>(ws);
    hipError_t e = qlr::launch_wha_merge(reinterpret_cast<const uint8_t*>(w->codes), w->absmax_q8, w->absmax_c,
                                         w->bits, levels_arg(w->bits), w->rows, K, lp, F->row_ptr, F->col, F->val,
                                         F->nnz, Wd, s);
    if (e != hipSuccess) return hip_fail(e, "adapter merge launch");
    qlr::LinearArgs a = make_args(c, 0.0f, nullptr, 1);
    a.codes = reinterpret_cast<const uint8_t*>(Wd);
    e = qlr::launch_gemm_dense(a, s);
    if (e != hipSuccess) return hip_fail(e, "linear launch");
    return QLR_OK;
  }
  if (F->nnz > 0) {
    const hipError_t e = qlr::launch_wha_addend(x, (int)xdt, M, K, w->rows, lp, F->row_ptr, F->col, F->val, F->nnz,
                                                C, s);
    if (e != hipSuccess) return hip_fail(e, "adapter transform launch");
    addend = C;
  }
  return run_linear(c, 0.0f, nullptr, path, s, addend);
}

qlr_status qlr_force_path(qlr_path path) {
  if (path < QLR_PATH_AUTO || path > QLR_PATH_GEMM) return fail(QLR_ERR_PATH, "unknown path %d", (int)path);
  t_path = path;
  return QLR_OK;
}

}  // extern "C"

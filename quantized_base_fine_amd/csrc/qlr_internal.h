// Internal launch interface between the host library (qlr_host.cpp) and the
// kernel translation units.  Arguments are validated by the host library
// before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlr_device.h"

namespace qlr {

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, int64_t n, hipStream_t s);

// Quantize numel elements of W (dtype wdt) into codes / absmax_q8 / absmax_c;
// sets *flag nonzero if W holds a non-finite value (flag must be zero before).
hipError_t launch_quantize(const void* W, int wdt, int64_t numel, int bits, const Levels& lv,
                           uint8_t* codes, uint8_t* q8, float* cst, uint32_t* flag,
                           hipStream_t s);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* q8, const float* cst,
                             int64_t numel, int bits, const Levels& lv, void* out, int odt,
                             hipStream_t s);

// Number of K-splits of the adapter product t = x A^T for M rows, K columns and
// rank r: the product is written as `splits` partial sums p[s][M][r] (float32)
// that the consumers add in split order; splits * M * r <= kTPartsMax (the
// decode kernel prefetches them all at once).  K need not be a multiple of 64
// (the backward's u = dy B contracts over the weight's rows); such products run
// one split on the float32 kernel.
constexpr int kTPartsMax = 4096;
int lora_t_splits(int64_t M, int64_t K, int r, int xdt, int abdt);

// p[s][m][j] = sum over split s's K range of x[m,k] A[j,k]  (float32 partials).
hipError_t launch_lora_t(const void* x, int xdt, int64_t M, int64_t K, const void* A, int abdt,
                         int r, float* t, int splits, hipStream_t s);

// bf16 products of several linears with one M > 16 (a mixed stack's adapters):
// up to lora_t_group_max() per launch, each written in one K pass (splits 1).
struct LoraTItem {
  const void* x;   // M x K bf16
  const void* A;   // r x K bf16, or K x r when bt (then r % 8 == 0)
  float* t;        // M x r float32
  int64_t K;
  int r;
  bool bt;
};
int lora_t_group_max();
hipError_t launch_lora_t_group(const LoraTItem* items, int n, int64_t M, hipStream_t s);
// The same for M <= 16 (bf16, K % 64 == 0, not bt): each item written as
// lora_t_splits(M, K, r) partial sums, as launch_lora_t would; up to
// lora_t_small_group_max() items per launch.
int lora_t_small_group_max();
hipError_t launch_lora_t_small_group(const LoraTItem* items, int n, int64_t M, hipStream_t s);

struct LinearArgs {
  const void* x;
  int xdt;
  int64_t M, N, K;
  int bits;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* cst;
  const float* t;  // splits x M x r float32 partials of x A^T (NULL if r == 0)
  int t_splits;
  const void* A;   // r x K
  const void* B;   // N x r
  int abdt;
  int r;
  float scale;
  void* y;
  int ydt;
  // optional float32 M x N term added to every output before rounding (the
  // sparse side channel's x S^T); null when absent
  const float* addend = nullptr;
  // optional CSR side channel (N rows) summed inside the single-row decode
  // kernel (see gemv_fuses_sparse); null when absent
  const int32_t* sp_row_ptr = nullptr;
  const int32_t* sp_col = nullptr;
  const float* sp_val = nullptr;
  int64_t sp_nnz = 0;
  // >= 0: the side channel multiplies the Walsh-Hadamard transform of x over
  // blocks of 2^sp_wht_lp columns, scaled by 2^-sp_wht_lp, instead of x
  int sp_wht_lp = -1;
  // prefill GEMM (forward): the CSR side channel's entries are added to the
  // dequantized weights of every 128-row tile whose entries number at most
  // gemm_sparse_cap(bits); the other tiles add `addend`, which then holds
  // their rows (launch_sparse_addend with that cap)
  bool sp_gemm = false;
  // optional double-binary branch (l = 1, r = its rank <= 16) summed inside the
  // single-row decode kernel in place of A and B (see gemv_fuses_dba)
  const uint32_t* dba_b1 = nullptr;
  const uint32_t* dba_b2 = nullptr;
  const uint16_t* dba_alpha = nullptr;
  const uint16_t* dba_beta = nullptr;
  const uint16_t* dba_gamma = nullptr;
};

// float32 path: any dtypes, any M.
hipError_t launch_linear_f32(const LinearArgs& a, const Levels& lv, hipStream_t s);
// bf16 decode path, M <= 16.
hipError_t launch_gemv(const LinearArgs& a, const Levels& lv, hipStream_t s);
// True when launch_gemv computes t = x A^T itself for this call (a single x
// row and a small rank): the adapter-product kernel is then not launched and
// a.t is not read.
bool gemv_fuses_adapter(const LinearArgs& a);
// True when launch_gemv can add a CSR side channel (a.sp_*) itself for this
// call: the single-row path with a short chunk stream.
bool gemv_fuses_sparse(const LinearArgs& a);
// True when launch_gemv can form the double-binary branch itself (a.dba_*, one
// envelope term, a.r = its rank <= 16, a single x row).
bool gemv_fuses_dba(const LinearArgs& a);
// Grouped single-row decode: up to gemv_group_max() linears of one code width
// and output dtype at M = 1 in one launch (a mixed stack's decode), each
// accepted by gemv_groupable (bits 2/4/8, bf16, x in LDS, adapter partials in t
// from the small-M adapter product, no side channel or addend).
int gemv_group_max();
bool gemv_groupable(const LinearArgs& a);
hipError_t launch_gemv_group(const LinearArgs* ls, int n, const Levels& lv, hipStream_t s);
// bf16 tiled GEMM path.
hipError_t launch_gemm(const LinearArgs& a, const Levels& lv, hipStream_t s);
// Weight rows per tile of the prefill GEMM, and the most side-channel entries a
// tile adds to its weights itself (0: none; widths whose level table fills LDS).
constexpr int64_t kGemmTileRows = 128;
int64_t gemm_sparse_cap(int bits);
// Up to gemm_group_max() independent linears of one code width, one M and one
// output dtype in one launch (mixed stacks); lv holds that width's levels.
int gemm_group_max();
hipError_t launch_gemm_group(const LinearArgs* ls, int n, const Levels& lv, hipStream_t s);

// ---- double-binary adapter branch
struct DbaArgs {
  int R, ell;
  const uint32_t* b1;     // N x ceil(R/32) words
  const uint32_t* b2;     // R x ceil(K/32) words
  const uint16_t* alpha;  // fp16, ell x N
  const uint16_t* beta;   // fp16, ell x R
  const uint16_t* gamma;  // fp16, ell x K
};
// K splits of the branch's first stage (float32 partials that the forward
// kernels add, like the adapter product's).
int dba_t_splits(int64_t M, int64_t K, int xdt, int R, int ell);
// t2 (splits x M x 2 ell R float32) = [t' | t'] and beff (N x 2 ell R bf16): the
// branch as an exact rank-2 ell R adapter with scale 1.
hipError_t launch_dba_prep(const DbaArgs& d, const void* x, int xdt, int64_t M, int64_t N, int64_t K, float* t2,
                           int splits, uint16_t* beff, hipStream_t s);

// ---- hybrid outlier split
size_t outlier_ws_bytes(int64_t numel, int64_t k);
// Select the k largest |w| (ties to the lower index), compact their flat
// indices (ascending) and values, and write W with them zeroed (same dtype) into
// the workspace; *flag (device) becomes nonzero if W holds NaN or Inf.
hipError_t launch_outlier_split(const void* W, int wdt, int64_t numel, int64_t k, void* ws, void** dense,
                                uint32_t** flag, int32_t** oidx, float** oval, hipStream_t s);
// After the dense part is quantized: row_ptr, columns, and residuals w - w'.
hipError_t launch_outlier_finish(int64_t rows, int64_t cols, int64_t k, int bits, const Levels& lv,
                                 const uint8_t* codes, const uint8_t* q8, const float* cst, const int32_t* oidx,
                                 const float* oval, int32_t* row_ptr, int32_t* col, float* val, hipStream_t s);
// *out = the largest entry count over the row groups [128 g, 128 g + 128) of a CSR
// with `rows` rows and k entries (one workgroup).
hipError_t launch_group_max(int64_t rows, int64_t k, const int32_t* row_ptr, uint32_t* out, hipStream_t s);
// C (M x N float32) = x S^T for S in CSR (N rows, K columns).  cap >= 0: only
// the rows of aligned kGemmTileRows-row groups holding more than cap entries
// are computed (the others are left as they are).
hipError_t launch_sparse_addend(const void* x, int xdt, int64_t M, int64_t K, int64_t N, const int32_t* row_ptr,
                                const int32_t* col, const float* val, int64_t nnz, float* C, hipStream_t s,
                                int64_t cap = -1);

// C (M x N float32) = z F^T, z = x blockdiag(H_P) / P (P = 2^lp), F in CSR (N rows, K columns);
// K % 8 == 0 and K <= wha_max_cols(); nnz >= 1.
hipError_t launch_wha_addend(const void* x, int xdt, int64_t M, int64_t K, int64_t N, int lp, const int32_t* row_ptr,
                             const int32_t* col, const float* val, int64_t nnz, float* C, hipStream_t s);
int64_t wha_max_cols();
// The branch merged into the weight for the prefill GEMM: Wd (N x K bf16) =
// bf16(W' + F blockdiag(H_P) / P), P = 2^lp, F in CSR (N rows, K columns);
// K % 64 == 0 and K <= wha_max_cols().
hipError_t launch_wha_merge(const uint8_t* codes, const uint8_t* q8, const float* cst, int bits, const Levels& lv,
                            int64_t N, int64_t K, int lp, const int32_t* row_ptr, const int32_t* col, const float* val,
                            int64_t nnz, uint16_t* out, hipStream_t s);
// Prefill GEMM on a dense bf16 weight held in a.codes (N x K row-major,
// N K 2 <= INT_MAX bytes): y = x Wd^T (+ a.addend); no adapter.
hipError_t launch_gemm_dense(const LinearArgs& a, hipStream_t s);

// ---- backward (adapter training)
// Input gradient dx = dy W' + scale u A on the transposed bf16 GEMM: a.x = dy
// (M x N bf16), a.y = dx (M x K), a.t = u partials (t_splits x M x r float32),
// a.B = A (r x K bf16), a.N / a.K the weight's rows / columns (both multiples
// of 64).
hipError_t launch_gemm_dx(const LinearArgs& a, const Levels& lv, hipStream_t s);
// Rows of x per GEMM launch for a contraction length KC (0: KC too large).
int64_t gemm_max_rows_of(int64_t KC);
// The same on the float32 path (any dtypes, any N).
hipError_t launch_dx_f32(const LinearArgs& a, const Levels& lv, hipStream_t s);
// Bt (r x N) = B^T for B (N x r) of dtype dt.
hipError_t launch_transpose_nr(const void* B, int dt, int64_t N, int r, void* Bt, hipStream_t s);
// dA = scale u^T x (r x K) and dB = scale dy^T t (N x r), float32, from the
// float32 partials of u (M x r) and t (M x r); x and dy share dtype qdt.
// mfma: bf16 MFMA kernel (qdt bf16, K and N multiples of 8), else float32 FMA.
// part: grad_partial_floats(M, N, K, r) floats of scratch.
size_t grad_partial_floats(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_lora_grads(const float* u, int u_splits, const float* t, int t_splits, const void* x,
                             const void* dy, int qdt, bool mfma, int64_t M, int64_t N, int64_t K, int r,
                             float scale, float* dA, float* dB, float* part, hipStream_t s);

}  // namespace qlr

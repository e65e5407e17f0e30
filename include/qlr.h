/*
 * qlr.h: C ABI of the quantized-base + low-rank-adapter linear layer for
 * AMD MI355X (gfx950).
 *
 * What the library computes (pages as printed; sections named on each call):
 *   - "QLoRA" (aizip.shop methodologies page), section "1. 4-bit NormalFloat
 *     (NF4) quantization": a k-bit codebook of normal quantiles.
 *   - same page, section "2. Double Quantization": blockwise absmax scaling with
 *     blocks of 64 weights, and the absmax constants themselves re-quantized to
 *     8 bits.
 *   - same page, memory-decomposition equation: frozen 4-bit base weights and
 *     bf16 adapters.
 *   - "LoRDBA" (gist.science summary), sections 1-2: the adapter is served
 *     unmerged ("adapter mode"), as a separate branch beside the frozen base.
 *   - "AutoQRA" (gist.science summary), section 3.1: every layer has its own
 *     bit width and adapter rank.
 *
 * Conventions for every call:
 *   - W is rows x cols = N x K, row-major ("out x in").  x is M x K, y is M x N,
 *     A is r x K, B is N x r, all row-major and densely packed.
 *   - Pointers marked (device) are HIP device pointers; the caller owns every
 *     buffer.  The library allocates nothing and keeps no per-call state; it
 *     holds no handle.  Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     calls are asynchronous on that stream unless stated otherwise.
 *   - Every call returns a qlr_status; nothing is thrown across the ABI.
 *     Argument errors are detected on the host before anything is launched.
 *     qlr_last_error() returns a thread-local description of the last failure.
 *   - Calls that share a workspace must not overlap in time (same stream, or
 *     ordered by the caller).
 */
#ifndef QLR_H
#define QLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLR_FORMAT_VERSION 1u /* codebook, tie rule, packing, double-quant format */
#define QLR_BLOCK 64          /* weights per first-level absmax constant */
#define QLR_GROUP 256         /* first-level constants per second-level constant */

typedef enum {
  QLR_OK = 0,
  QLR_ERR_NULL = 1,      /* a required pointer is NULL */
  QLR_ERR_SHAPE = 2,     /* a size is negative, zero where not allowed, or inconsistent */
  QLR_ERR_DTYPE = 3,     /* dtype not supported for this argument */
  QLR_ERR_BITS = 4,      /* bits not in {2, 3, 4, 8} */
  QLR_ERR_BLOCK = 5,     /* block != 64 or group != 256 */
  QLR_ERR_ALIGN = 6,     /* a device pointer is not 16-byte aligned */
  QLR_ERR_NONFINITE = 7, /* quantize: W holds NaN or Inf */
  QLR_ERR_WORKSPACE = 8, /* workspace NULL or smaller than qlr_workspace_bytes() */
  QLR_ERR_ALIAS = 9,     /* mixed: an output overlaps an input or another output */
  QLR_ERR_HIP = 10,      /* a HIP runtime call or launch failed (text in qlr_last_error) */
  QLR_ERR_FORMAT = 11,   /* qlr_qweight.format_version unknown */
  QLR_ERR_PATH = 12      /* forced path cannot run these arguments */
} qlr_status;

typedef enum { QLR_F32 = 0, QLR_F16 = 1, QLR_BF16 = 2 } qlr_dtype;

/* Kernel families of qlr_linear_fwd (QLR_PATH_AUTO picks by M and dtype). */
typedef enum {
  QLR_PATH_AUTO = 0,
  QLR_PATH_F32 = 1,  /* float32 arithmetic, any M and dtype; the accuracy-first path */
  QLR_PATH_GEMV = 2, /* bf16 x, M <= 16: bandwidth-bound decode (bf16 MFMA, fp32 accumulate) */
  QLR_PATH_GEMM = 3  /* bf16 x, any M: LDS-tiled prefill GEMM (bf16 MFMA, fp32 accumulate) */
} qlr_path;

typedef enum {
  QLR_OP_QUANTIZE = 0,
  QLR_OP_LINEAR = 1,
  QLR_OP_LINEAR_BWD = 2,
  QLR_OP_LINEAR_DBA = 3,
  QLR_OP_QUANTIZE_OUTLIERS = 4, /* M = the outlier count k, N = rows, K = cols */
  QLR_OP_LINEAR_OUTLIERS = 5,
  QLR_OP_LINEAR_WHA = 6 /* r is ignored */
} qlr_op;

/*
 * A quantized frozen weight (QLoRA page, sections "1. 4-bit NormalFloat" and
 * "2. Double Quantization"; format version 1):
 *   codes     (device) ceil(rows*cols/64) * 8*bits bytes.  Block j = the 64
 *             consecutive elements [64j, 64j+64) of the row-major flattened W;
 *             its codes fill bytes [8*bits*j, 8*bits*(j+1)), element e of the
 *             block at bits [bits*e, bits*e+bits) of that little-endian bit
 *             string.  Code i stands for codebook level i (ascending).
 *   absmax_q8 (device) one byte per block: the 8-bit code m of the block's
 *             absmax, which dequantizes to m * absmax_c[j / 256].
 *   absmax_c  (device) one float32 per 256 consecutive blocks: the step
 *             fl32(g / 255), g the largest absmax in the group.
 * A dequantized weight is fl32(level[code] * fl32(m * step)).
 */
typedef struct {
  uint32_t format_version; /* QLR_FORMAT_VERSION */
  int32_t bits;            /* 2, 3, 4 or 8 */
  int32_t block;           /* QLR_BLOCK */
  int32_t group;           /* QLR_GROUP */
  int64_t rows;            /* N */
  int64_t cols;            /* K */
  void* codes;             /* device */
  uint8_t* absmax_q8;      /* device */
  float* absmax_c;         /* device */
} qlr_qweight;

/* One entry of a mixed stack (AutoQRA page, section 3.1: per-layer bits and rank). */
typedef struct {
  const qlr_qweight* w; /* host pointer to the layer's quantized weight */
  const void* x;        /* device, M x w->cols */
  const void* A;        /* device, r x w->cols (NULL if r == 0) */
  const void* B;        /* device, w->rows x r (NULL if r == 0) */
  int32_t r;            /* adapter rank, >= 0 */
  float scale;          /* alpha / r */
  void* y;              /* device, M x w->rows */
} qlr_layer;

/*
 * A double-binary adapter (LoRDBA page, section 2 "Core architecture"):
 * dW = sum_{i<ell} diag(alpha_i) B1 diag(beta_i) B2 diag(gamma_i), with sign
 * factors B1 (rows x rank) and B2 (rank x cols) in {-1, +1} at one bit per
 * entry, shared by the ell terms, and fp16 channel scales.  Bit 1 stands for
 * +1, bit 0 for -1; a row of c entries is ceil(c/32) uint32 words, entry e at
 * bit e % 32 of word e / 32 (padding bits ignored).
 */
typedef struct {
  int32_t rank;          /* R >= 1 */
  int32_t ell;           /* envelope rank >= 1 (rank * ell <= 4096) */
  const uint32_t* b1;    /* device, rows x ceil(R/32) words */
  const uint32_t* b2;    /* device, R x ceil(cols/32) words */
  const uint16_t* alpha; /* device, fp16 bits, ell x rows */
  const uint16_t* beta;  /* device, fp16 bits, ell x R */
  const uint16_t* gamma; /* device, fp16 bits, ell x cols */
} qlr_dba;

/*
 * Sparse side channel of a weight's outliers (QFT page, section 2.2 "Hybrid
 * feature quantizer"): CSR by weight row, columns ascending within a row.
 * val holds float32 residuals w - w' against the dense part's dequantized value
 * at that position (the quantile codebook has no exact zero level).
 */
typedef struct {
  int64_t rows;     /* = the weight's rows */
  int64_t cols;     /* = the weight's cols */
  int64_t nnz;      /* k */
  int32_t* row_ptr; /* device, rows + 1 */
  int32_t* col;     /* device, nnz */
  float* val;       /* device, nnz */
  /* host: the largest number of entries in a group of 128 rows starting at a
   * multiple of 128 (rows 128 g .. 128 g + 127), as qlr_quantize_outliers sets
   * it.  A caller that fills the CSR itself sets -1 (not known) or the exact
   * figure; any value outside 1 .. nnz counts as not known.  Lets the prefill
   * forward skip work it would otherwise do to find this out on the device. */
  int64_t max_group_nnz;
} qlr_sparse;

/* Library version (major*10000 + minor*100 + patch). */
int qlr_version(void);
/* Static text for a status code. */
const char* qlr_status_string(qlr_status s);
/* Thread-local text of the last error raised on this thread ("" if none). */
const char* qlr_last_error(void);

/*
 * Codebook (QLoRA page, section "1. 4-bit NormalFloat (NF4) quantization",
 * codebook equation).  Writes the 2^bits ascending float32 levels to `out`
 * (host).  Level i = Q((i + 1/2) / 2^bits) / Q((2^bits - 1/2) / 2^bits),
 * Q the standard-normal quantile (0-based i; the printed equation's
 * (i - 1/2) is read with a 1-based index), the lower half computed and the
 * upper half its mirror image, each rounded once to float32.
 * Host only.  Errors: QLR_ERR_NULL, QLR_ERR_BITS.
 */
qlr_status qlr_codebook(int32_t bits, float* out);

/*
 * Sizes in bytes of the three arrays of a rows x cols quantized weight
 * (QLoRA page, section "2. Double Quantization": bits + 8/64 + 32/(64*256)
 * bits per weight).  Any rows, cols >= 0 (a trailing partial block and group
 * are allowed).  Host only.  Errors: QLR_ERR_NULL, QLR_ERR_SHAPE,
 * QLR_ERR_BITS, QLR_ERR_BLOCK.
 */
qlr_status qlr_qweight_sizes(int64_t rows, int64_t cols, int32_t bits, int32_t block,
                             size_t* codes_bytes, size_t* absmax_q8_bytes,
                             size_t* absmax_c_bytes);

/*
 * Device workspace needed by an operation.  QLR_OP_QUANTIZE: 256 bytes (the
 * non-finite flag); M, N, K, r are ignored.  QLR_OP_LINEAR: the adapter
 * product t = x A^T for M rows and rank r as float32 partial sums over K
 * splits, rounded up to 256 bytes (0 bytes when M or r is 0).
 * QLR_OP_LINEAR_BWD (N = rows, K = cols of the weight): the partial sums of
 * x A^T and dy B, B transposed, and float32 partials of the adapter gradients
 * (0 bytes when r is 0).  Contents need no initialisation.  Host only.
 */
qlr_status qlr_workspace_bytes(qlr_op op, int64_t M, int64_t N, int64_t K, int32_t r,
                               size_t* bytes);

/*
 * Quantize (QLoRA page, sections "1. 4-bit NormalFloat (NF4) quantization" and
 * "2. Double Quantization").  W (device) rows x cols in wdt (f32, f16, bf16),
 * widened exactly to float32.  For block j with float32 absmax a, element w
 * gets the code of the nearest level*a, ties to the lower code
 * (#{i : 2w > (level[i] + level[i+1]) * a}, decided exactly); a == 0 gives
 * code 0.  Groups of 256 absmax values get step s = fl32(g / 255) and each
 * absmax the code of the nearest multiple m*s, ties to the lower m.
 * `out` (host struct) must carry format_version, bits, block, group, rows,
 * cols and the three device buffers sized by qlr_qweight_sizes; the call fills
 * the buffers.  ws (device) >= qlr_workspace_bytes(QLR_OP_QUANTIZE).
 * BLOCKING: synchronises `stream` to read the non-finite flag.
 * Errors: QLR_ERR_NULL, QLR_ERR_SHAPE, QLR_ERR_DTYPE, QLR_ERR_BITS,
 * QLR_ERR_BLOCK, QLR_ERR_ALIGN, QLR_ERR_WORKSPACE, QLR_ERR_FORMAT,
 * QLR_ERR_NONFINITE (buffers then hold unspecified data), QLR_ERR_HIP.
 */
qlr_status qlr_quantize(const void* W, qlr_dtype wdt, int64_t rows, int64_t cols, int32_t bits,
                        int32_t block, qlr_qweight* out, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * Same as qlr_quantize but asynchronous: the non-finite flag is left in the
 * first 4 bytes of ws (uint32, nonzero if W held NaN or Inf) for the caller.
 */
qlr_status qlr_quantize_async(const void* W, qlr_dtype wdt, int64_t rows, int64_t cols,
                              int32_t bits, int32_t block, qlr_qweight* out, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Dequantize (QLoRA page, section "Limitations": the base is dequantized
 * whenever it is used).  out (device) rows*cols elements of odt:
 * QLR_F32 gives fl32(level[c] * fl32(m * step)) exactly (two float32
 * multiplies in that order, signed zeros kept); QLR_BF16 gives that value
 * rounded to nearest-even bf16.  Errors: QLR_ERR_NULL, QLR_ERR_DTYPE,
 * QLR_ERR_BITS, QLR_ERR_BLOCK, QLR_ERR_ALIGN, QLR_ERR_FORMAT, QLR_ERR_SHAPE,
 * QLR_ERR_HIP.
 */
qlr_status qlr_dequantize(const qlr_qweight* w, void* out, qlr_dtype odt, void* stream);

/*
 * Forward of the frozen base with an unmerged adapter (QLoRA page,
 * memory-decomposition equation; LoRDBA page, "adapter mode"):
 *     y = x W'^T + scale * (x A^T) B^T,   W' the dequantized weight.
 * x (device) M x K in xdt (f32 or bf16); A (device) r x K and B (device) N x r
 * in abdt (f32 or bf16), both NULL when r == 0; y (device) M x N in ydt
 * (f32 or bf16).  Requires cols % 64 == 0 (whole blocks per row).  M may be 0
 * (nothing is launched).  Error bound per y element, S = sum_k |x[m,k] w'[n,k]|
 * (plus half a bf16 ulp of the result when ydt is bf16), on any input:
 *   - QLR_PATH_F32 and QLR_PATH_GEMV: 1e-3 * S + 1e-5.  The single-row
 *     decode kernels (M = 1 with 2-, 4- or 8-bit codes, and every width in
 *     qlr_linear_fwd_mixed) take each codebook level as one fp16 number
 *     (within 2^-11 of it) times x as fp16 numbers scaled by a power of two
 *     per 64-column block, exact whenever the block's values fit (otherwise
 *     that part of the row is summed in float32); the other decode kernels
 *     carry each level as two bf16 halves (about 16 significant bits); the
 *     float32 kernels work in float32; sums are float32.
 *   - QLR_PATH_GEMM: 5e-3 * S + 1e-5.  The prefill kernel rounds each
 *     dequantized weight once to bf16 (relative error up to 2^-8) for the bf16
 *     matrix cores.  When those rounding errors do not all share a sign, as
 *     for zero-mean x or weights, the error stays far inside 1e-3 * S; a caller
 *     that needs 1e-3 * S on every input at M > 16 forces QLR_PATH_F32.
 * ws (device) >= qlr_workspace_bytes(QLR_OP_LINEAR,
 * M, N, K, r) (scratch for x A^T; any contents).
 * Asynchronous, allocation-free, no host synchronisation.
 * Errors: QLR_ERR_NULL, QLR_ERR_SHAPE, QLR_ERR_DTYPE, QLR_ERR_BITS,
 * QLR_ERR_BLOCK, QLR_ERR_ALIGN, QLR_ERR_FORMAT, QLR_ERR_WORKSPACE,
 * QLR_ERR_PATH, QLR_ERR_HIP.
 */
qlr_status qlr_linear_fwd(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w,
                          const void* A, const void* B, qlr_dtype abdt, int32_t r, float scale,
                          void* y, qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): qlr_linear_fwd without the workspace arguments, same arguments
 * otherwise, same kernels and results.  Its scratch (the adapter product's
 * float32 partial sums) is a file-scope device array of
 * QLR_STATIC_SCRATCH_BYTES on each GPU the library runs on, held until the
 * process ends; the call allocates nothing.  A call whose
 * qlr_workspace_bytes(QLR_OP_LINEAR, M, rows, cols, r) exceeds that size fails
 * with QLR_ERR_WORKSPACE (nothing launched).  Every call on one GPU shares that
 * GPU's array and leaves its contents behind: calls that overlap in time on one
 * GPU (different streams or host threads) race and give wrong results.  The
 * kernels need no initial contents.  Asynchronous.  Errors: as qlr_linear_fwd.
 */
#define QLR_STATIC_SCRATCH_BYTES (8u << 20)
qlr_status qlr_linear_fwd_static(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w,
                                 const void* A, const void* B, qlr_dtype abdt, int32_t r, float scale,
                                 void* y, qlr_dtype ydt, void* stream);

/*
 * Mixed stack (AutoQRA page, section 3.1: each layer has its own bit width
 * and rank).  `layers` (host array of n entries) are independent linears, all
 * with the same M and dtypes, each computed as qlr_linear_fwd would.  No y
 * may overlap any x, A, B or other y of the call (QLR_ERR_ALIAS, checked on
 * the host).  ws >= the sum over entries of qlr_workspace_bytes(QLR_OP_LINEAR,
 * M, rows, cols, r).  Asynchronous.
 */
qlr_status qlr_linear_fwd_mixed(const qlr_layer* layers, int32_t n, int64_t M, qlr_dtype xdt,
                                qlr_dtype abdt, qlr_dtype ydt, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Quantize with a hybrid outlier split (QFT page, section 2.2: about 1 % of
 * the weights, the outliers that stretch the range, kept at full precision;
 * the dense rest quantized).  The k entries of largest |w| (float32 after
 * exact widening; ties to the lower flat index) are set to 0 and the result is
 * quantized as qlr_quantize does (out); sp receives, for each of them in
 * row-major order, its column and the float32 residual fl32(w - w'), w' the
 * dense part's dequantized value there, and sp->row_ptr the CSR row offsets;
 * sp->max_group_nnz is set on the host.  The caller sets sp->rows, sp->cols,
 * sp->nnz = k and provides its buffers.
 * rows * cols < 2^31, 0 <= k <= rows * cols.  ws (device) >=
 * qlr_workspace_bytes(QLR_OP_QUANTIZE_OUTLIERS, k, rows, cols, 0).
 * BLOCKING (reads the non-finite flags).  Errors: as qlr_quantize, plus
 * QLR_ERR_SHAPE for k or a mismatching sp header.
 */
qlr_status qlr_quantize_outliers(const void* W, qlr_dtype wdt, int64_t rows, int64_t cols, int32_t bits,
                                 int32_t block, int64_t k, qlr_qweight* out, qlr_sparse* sp, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Forward with the sparse side channel: y = x W'^T + x S^T + scale (x A^T) B^T,
 * S the CSR outliers of qlr_quantize_outliers, or any CSR of the weight's shape
 * with row_ptr nondecreasing from 0 to nnz and columns in [0, cols) (a
 * malformed one gives wrong values; the kernels clamp every index they read).
 * The sparse term is formed in float32 (outliers in CSR order) and added to
 * each output before rounding, except on the prefill GEMM family with 2- or
 * 4-bit codes: there each 128-row tile of the weight whose entries fit the
 * kernel's spare LDS (about 2000 with 4-bit codes, 1500 with 2-bit) adds them
 * to its dequantized bf16 weights, rounding each changed weight to bf16 again
 * (within that family's bound), and only the other tiles take the float32 term
 * (its kernel is not launched when sp->max_group_nnz says that every tile's
 * entries fit).  Arguments otherwise as qlr_linear_fwd; the error bound's S also sums
 * |x[m, col] val| over the row's outliers.
 * ws >= qlr_workspace_bytes(QLR_OP_LINEAR_OUTLIERS, M, rows, cols, r).
 * Asynchronous, allocation-free.
 */
qlr_status qlr_linear_fwd_outliers(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w,
                                   const qlr_sparse* sp, const void* A, const void* B, qlr_dtype abdt, int32_t r,
                                   float scale, void* y, qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream);

/*
 * Forward with a Walsh-Hadamard adapter (QWHA page, section 2.1 "Adapter
 * design"): y = x W'^T + x dW^T with dW = F H^-1, H the natural-order +-1
 * Walsh-Hadamard matrix (H[i][j] = (-1)^popcount(i & j)) applied in blocks of
 * hblock columns (a power of two dividing cols; hblock = cols is one full
 * transform), so H^-1 = H / hblock, and F the sparse coefficient matrix
 * (rows x cols CSR in the qlr_sparse format: row_ptr, col = transform index,
 * val = the coefficient values c in float32; repeated columns of a row add).
 * On the decode and float32 families it is computed as z F^T with
 * z = x blockdiag(H) / hblock: each x row is transformed by butterflies
 * (additions and subtractions, float32), scaled exactly by 1 / hblock, then
 * multiplied by F (float32), and the result is added to each output before
 * rounding.  On the prefill GEMM family (bf16 x, M > 16, rows * cols * 2 <
 * 2^31) the branch is merged into a bf16 copy of the weight in the workspace
 * instead: each row of F is transformed the same way (float32), scaled by
 * 1 / hblock, added to the row's dequantized weights w' and rounded once to
 * bf16, and the GEMM multiplies that copy (the stored weight and F are not
 * changed).  No low-rank adapter in this call (the branch replaces it).
 *   x: M x cols, bf16 or f32 (bf16 on the decode and prefill kernels); cols <= 32768.
 *   ws >= qlr_workspace_bytes(QLR_OP_LINEAR_WHA, M, rows, cols, 0): M x rows
 *   float32, or where the prefill GEMM runs (M > 16 or that path forced, on
 *   the calling thread) the larger of that and rows x cols bf16.
 * Tolerance as qlr_linear_fwd for the family that runs (on the GEMM family
 * its bf16 weights are W' + F H / hblock), with S extended by sum_j |c_j|
 * (sum of |x| over j's block) / hblock.  Asynchronous, allocation-free.
 * Errors: as qlr_linear_fwd, plus QLR_ERR_SHAPE for hblock, cols or a
 * mismatching F.
 */
qlr_status qlr_linear_fwd_wha(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w, const qlr_sparse* F,
                              int32_t hblock, void* y, qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream);

/*
 * Forward with a double-binary adapter in adapter mode (LoRDBA page,
 * sections 1-2: the adapter stays unmerged beside the frozen base):
 *     y = x W'^T + sum_i alpha_i * (((x * gamma_i) B2^T) * beta_i) B1^T
 * (* the per-channel product).  x, y, M, w as in qlr_linear_fwd (cols % 64 ==
 * 0).  The branch runs as an exact rank-2*ell*R branch of the forward kernels:
 * its first stage (float32 sums of +-x*gamma, times beta) and the alpha-signed
 * second factor (alpha split exactly into two bf16 halves) are formed in the
 * workspace, then the quantized-base kernel adds it in its epilogue or its
 * adapter K blocks.  Same error bound as qlr_linear_fwd, with S extended by
 * sum_i |alpha_i[n]| sum_j |beta_i[j]| sum_k |x[m,k] gamma_i[k]|.
 * ws (device) >= qlr_workspace_bytes(QLR_OP_LINEAR_DBA, M, rows, cols,
 * rank * ell).  Asynchronous, allocation-free.
 * Errors: as qlr_linear_fwd (QLR_ERR_SHAPE also for rank or ell < 1).
 */
qlr_status qlr_linear_fwd_dba(const void* x, qlr_dtype xdt, int64_t M, const qlr_qweight* w, const qlr_dba* adapter,
                              void* y, qlr_dtype ydt, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward for adapter training (the step after the forward in fine-tuning:
 * QLoRA page, memory-decomposition equation, frozen 4-bit base with trained
 * bf16 adapters; AutoQRA page, "1. Problem statement", frozen quantized
 * backbone with trained adapters).  For the forward of qlr_linear_fwd and an
 * upstream gradient dy, with u = dy B and t = x A^T:
 *     dx = dy W' + scale * u A      (M x K)  input gradient through the frozen base
 *     dA = scale * u^T x            (r x K)
 *     dB = scale * dy^T t           (N x r)
 * W' gets no gradient (it is frozen).  dy (device) M x N in dydt (f32 or bf16);
 * x (device) M x K in xdt, which must equal dydt when r > 0 (x is not read
 * when r == 0 and may be NULL); A, B as in qlr_linear_fwd; dx (device) M x K
 * in dxdt (f32 or bf16), or NULL to skip the input gradient; dA (device, r x K)
 * and dB (device, N x r) float32, overwritten (zero when M == 0), required when
 * r > 0.  No output may overlap an input or another output (QLR_ERR_ALIAS).
 * Requires cols % 64 == 0.  Kernel families: with bf16 dy, x and adapters and
 * rows % 64 == 0 the input gradient runs on bf16 MFMA (the weight dequantized
 * to bf16, float32 accumulation); otherwise, or under QLR_PATH_F32, on float32
 * arithmetic (qlr_force_path: QLR_PATH_GEMV selects the MFMA family here, as
 * the backward has no separate decode kernel).  u, t, dA and dB are float32
 * sums of exactly widened inputs.  Per element, each result is within
 * 1e-3 * S + 1e-5 of the exact value, S the sum of the absolute values of the
 * terms that define it (with |u| and |t| likewise bounded by sums of absolute
 * products), plus half a bf16 ulp for a bf16 dx; on the MFMA family dx is
 * within 5e-3 * S + 1e-5 (the weight enters rounded to bf16, as on the
 * prefill GEMM of qlr_linear_fwd).  ws (device) >=
 * qlr_workspace_bytes(QLR_OP_LINEAR_BWD, M, rows, cols, r).  Asynchronous,
 * allocation-free; the results do not depend on timing.
 * Errors: QLR_ERR_NULL, QLR_ERR_SHAPE, QLR_ERR_DTYPE, QLR_ERR_BITS,
 * QLR_ERR_BLOCK, QLR_ERR_ALIGN, QLR_ERR_FORMAT, QLR_ERR_WORKSPACE,
 * QLR_ERR_ALIAS, QLR_ERR_PATH, QLR_ERR_HIP.
 */
qlr_status qlr_linear_bwd(const void* dy, qlr_dtype dydt, const void* x, qlr_dtype xdt, int64_t M,
                          const qlr_qweight* w, const void* A, const void* B, qlr_dtype abdt, int32_t r,
                          float scale, void* dx, qlr_dtype dxdt, float* dA, float* dB, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Force the kernel family used by qlr_linear_fwd and qlr_linear_fwd_mixed on
 * the calling thread (for tests, measurement, and callers that need a
 * family's error bound; see qlr_linear_fwd).  QLR_PATH_AUTO restores the
 * default choice: F32 for float32 x or float32 adapters, GEMV for M <= 16,
 * GEMM otherwise.  Host only.  Errors: QLR_ERR_PATH for an unknown value.
 */
qlr_status qlr_force_path(qlr_path path);

#ifdef __cplusplus
}
#endif

#endif /* QLR_H */

/*
 * rnq - RMSNorm -> partial NeoX RoPE -> per-row FP8 e4m3fn on AMD MI355X (gfx950).
 *
 * C ABI of librnq.so. Plain pointers and sizes only; no HIP or torch types.
 *
 * Sources of the operations (tilelang-tutorial pages):
 *  - chapter 13 fusion page "rmsnorm_rope_quant.py": torch_reference_fused and
 *    the two fused kernels (RMSNorm + RoPE on the last rope_dim columns, then
 *    per-row absmax FP8 quantisation);
 *  - chapter 17 page "rmsnorm_tl.py": the RMSNorm forward kernel and
 *    RMSNormTileLang.backward;
 *  - chapter 28 page "case_norm_rope_quant.py": the QK-norm prologue (rows are
 *    (token, head) pairs, one cos/sin row per token shared by every head, one
 *    fp32 scale per row).
 *
 * Common rules for every entry point
 *  - Memory: every tensor pointer is a device pointer owned by the caller; the
 *    library never allocates, frees or synchronises. Work is enqueued on
 *    `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 *    runs asynchronously; outputs are fully overwritten. Inputs and outputs
 *    must not alias.
 *  - Layout: contiguous row-major. 16-bit float tensors are raw bf16 or fp16
 *    storage, chosen by `dtype` (rnq_dtype). cos/sin are fp32. FP8 outputs are
 *    raw e4m3fn bytes (OCP: bias 7, max 448).
 *  - Alignment: x/q/k/y/grad tensors, weights and cos/sin must be 16-byte
 *    aligned; FP8 outputs 8-byte aligned; fp32 vectors 4-byte aligned.
 *  - Arithmetic: fp32 with IEEE rounding at every step and no fused
 *    multiply-add; the sum of squares of a row is accumulated in fp64, which is
 *    exact whenever the row's total stays below 2^53 times the lowest set bit
 *    of its smallest nonzero square (every row of the test workloads), and is
 *    rounded once to fp32; rsqrt is 1/sqrt with both steps correctly rounded; the normalised
 *    row and the rotated row are each rounded to the input dtype (nearest
 *    even); codes are round-to-nearest-even e4m3fn of clamp(y/scale, +-fp8_max).
 *  - Errors: every argument is validated before anything is enqueued; on a
 *    non-OK status nothing has been launched (except RNQ_ERR_HIP, reported
 *    from hipGetLastError after a launch). rnq_status_string() names a status;
 *    rnq_last_error() gives a per-thread message for the last failed call.
 *    A call with zero rows returns RNQ_OK and launches nothing.
 *  - Thread safety: no global mutable state apart from the per-thread error
 *    message; concurrent calls on different streams are independent. (The
 *    one exception is rnq_rmsnorm_rope_bwd_noalloc, which shares a static
 *    device scratch array per GPU; see there.)
 */
#ifndef RNQ_H_
#define RNQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rnq_status {
  RNQ_OK = 0,
  RNQ_ERR_NULL = 1,        /* a required pointer is NULL */
  RNQ_ERR_SHAPE = 2,       /* negative size, odd or too large rope_dim, rows not divisible, ... */
  RNQ_ERR_UNSUPPORTED = 3, /* a width or alignment outside what the kernels are built for */
  RNQ_ERR_ARG = 4,         /* eps < 0 or non-finite, fp8_max outside (0, 448], unknown dtype */
  RNQ_ERR_WORKSPACE = 5,   /* workspace too small */
  RNQ_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} rnq_status;

typedef enum rnq_dtype { RNQ_BF16 = 0, RNQ_F16 = 1 } rnq_dtype;

/* Name of a status code (static string). */
const char* rnq_status_string(int status);

/* Message describing the last non-OK status returned on the calling thread ("" if none). */
const char* rnq_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int rnq_abi_version(void);

/*
 * RMSNorm forward (chapter 17 page, forward kernel; chapter 13 fusion page,
 * first half of torch_reference_fused):
 *   rstd[m] = 1 / sqrt(sum_j x[m,j]^2 / N + eps)
 *   y[m,j]  = round_dtype((x[m,j] * rstd[m]) * w[j])
 *
 * x [M,N], w [N], y [M,N] in `dtype`; rstd_out [M] fp32 may be NULL.
 * N must be a multiple of 8 and at most 16384.
 */
rnq_status rnq_rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd_out,
                           int64_t M, int64_t N, float eps, int dtype, void* stream);

/* Bytes of device workspace rnq_rmsnorm_bwd needs for an [M,N] problem:
 * P * N * 4, where the rows are split into P contiguous blocks,
 * P = ceil(M / ceil(M / T)) with T = 512 for M <= 8192 and 256 above
 * (0 when M or N is 0). */
size_t rnq_rmsnorm_bwd_workspace_size(int64_t M, int64_t N);

/*
 * RMSNorm backward (chapter 17 page, RMSNormTileLang.backward):
 *   xn = x * rstd, g = grad_y * w, C = sum_j(g * xn) / N
 *   grad_x = round_dtype(rstd * (g - xn * C))          [M,N] in `dtype`
 *   grad_w = sum over rows of grad_y * xn              [N] fp32 (the page casts it to
 *                                                      w's dtype afterwards; the caller may)
 * rstd [M] fp32 may be NULL, in which case it is recomputed from x as in the
 * forward. grad_w is reduced deterministically: per-block partial sums over a
 * fixed row partition are written to `workspace`, then summed per column in
 * a fixed order; results are bitwise reproducible for a given (M, N).
 * workspace_bytes must be >= rnq_rmsnorm_bwd_workspace_size(M, N); the
 * workspace is scratch owned by the caller (16-byte aligned).
 * Requirements: N a multiple of 8, at most 16384; M < 2^31; for N of 64..512,
 * 1024, 2048 or 4096 one partition block's rows (about M / 256 rows of x)
 * below 2 GiB (UNSUPPORTED otherwise).
 */
rnq_status rnq_rmsnorm_bwd(const void* x, const void* w, const void* grad_y, const float* rstd,
                           void* grad_x, float* grad_w, void* workspace, size_t workspace_bytes,
                           int64_t M, int64_t N, float eps, int dtype, void* stream);

/*
 * RMSNorm + partial NeoX RoPE (chapter 13 fusion page, rms_norm_rope_fused and
 * _torch_rope_neox):
 *   n = RMSNorm(x, w) rounded to dtype (as rnq_rmsnorm_fwd)
 *   on the last R = rope_dim columns, for p < R/2, with c = cos[t,p], s = sin[t,p]:
 *     y[N-R+p]     = round_dtype(n[N-R+p] * c - n[N-R+R/2+p] * s)
 *     y[N-R+R/2+p] = round_dtype(n[N-R+R/2+p] * c + n[N-R+p] * s)
 *   other columns: y = n.
 * x, y [M,N]; w [N]; cos, sin [M/rows_per_token, R/2] fp32; row m uses table
 * row t = m / rows_per_token (rows_per_token = heads per token for a
 * [tokens*heads, head_dim] layout; 1 for one table row per row).
 * Requirements: N a multiple of 8, at most 16384; R a multiple of 16 with
 * R <= N, and R <= 1024 unless N is 64, 128, 256 or 512 (head-sized rows, the
 * row kernel; other widths take one workgroup per row); M % rows_per_token == 0;
 * the cos/sin table below 2 GiB. cos/sin may be NULL when R == 0.
 */
rnq_status rnq_rmsnorm_rope(const void* x, const void* w, const float* cos, const float* sin,
                            void* y, int64_t M, int64_t N, int64_t rope_dim, int64_t rows_per_token,
                            float eps, int dtype, void* stream);

/*
 * rnq_rmsnorm_rope on a strided, position-indexed input: x_token_stride
 * elements between the first rows of consecutive tokens (each token's
 * rows_per_token rows contiguous; 0 = contiguous), and token t (rows
 * t*rows_per_token ..) uses row positions[t] of cos/sin [table_rows, R/2]
 * when positions (int32 [M / rows_per_token]) is given, with the clamping and
 * stride rules of rnq_qk_norm_rope_fp8_ex. y is contiguous [M, N].
 */
rnq_status rnq_rmsnorm_rope_ex(const void* x, int64_t x_token_stride, const void* w, const float* cos,
                               const float* sin, const int32_t* positions, int64_t table_rows, void* y, int64_t M,
                               int64_t N, int64_t rope_dim, int64_t rows_per_token, float eps, int dtype,
                               void* stream);

/*
 * Backward of rnq_rmsnorm_rope (the rotation of the chapter 13 fusion page
 * followed back, then the chapter 17 RMSNorm backward). The two casts to
 * `dtype` in the forward count as identities. On the last R = rope_dim
 * columns the output gradient goes through the transposed rotation, for
 * p < R/2 with c = cos[t,p], s = sin[t,p], t = m / rows_per_token:
 *   gn[N-R+p]     = grad_y[N-R+p] * c + grad_y[N-R+R/2+p] * s
 *   gn[N-R+R/2+p] = grad_y[N-R+R/2+p] * c - grad_y[N-R+p] * s
 * (gn = grad_y elsewhere; fp32), then, as rnq_rmsnorm_bwd with gn for grad_y:
 *   grad_x = round_dtype(rstd * (gn * w - xn * C)), C = sum_j(gn * w * xn) / N
 *   grad_w = sum over rows of gn * xn                  [N] fp32
 * Layouts, rstd (NULL: recomputed), the workspace (rnq_rmsnorm_bwd_workspace_size(M, N)
 * bytes) and the fixed-order grad_w reduction are those of rnq_rmsnorm_bwd;
 * cos, sin and rows_per_token those of rnq_rmsnorm_rope.
 * Requirements: N a multiple of 8, at most 16384 (the widths rnq_rmsnorm_bwd
 * takes); R a multiple of 16 with R <= N, and R <= 1024 unless N is 64, 128,
 * 256 or 512; M % rows_per_token == 0; M < 2^31; the cos/sin table below
 * 2 GiB, and for N of 64..512, or 1024, 2048, 4096 with R <= 512, one
 * partition block's rows (about M / 256 rows of x) below 2 GiB
 * (UNSUPPORTED otherwise). cos/sin may be NULL when R == 0.
 */
rnq_status rnq_rmsnorm_rope_bwd(const void* x, const void* w, const void* grad_y, const float* cos,
                                const float* sin, const float* rstd, void* grad_x, float* grad_w,
                                void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                                int64_t rope_dim, int64_t rows_per_token, float eps, int dtype,
                                void* stream);

/* Size of the library's static device scratch used by rnq_rmsnorm_rope_bwd_noalloc:
 * 32 MiB, enough for the grad_w partials of every shape the backward accepts
 * (at most 512 partial rows of N <= 16384 fp32 values). */
#define RNQ_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

/*
 * rnq_rmsnorm_rope_bwd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, kernels, results (bit for
 * bit) and rules as rnq_rmsnorm_rope_bwd, minus workspace / workspace_bytes:
 * the grad_w partials go to a file-scope device array of
 * RNQ_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends). The call allocates nothing: on its first call on a device it
 * looks up that device's copy of the array (hipGetSymbolAddress, the device
 * of `stream`); later calls reuse the address.
 * Errors: RNQ_ERR_WORKSPACE when rnq_rmsnorm_bwd_workspace_size(M, N) exceeds
 * RNQ_NOALLOC_SCRATCH_BYTES (not reached for N <= 16384); RNQ_ERR_HIP when the
 * lookup fails; otherwise as rnq_rmsnorm_rope_bwd.
 * Concurrency: every call on one GPU uses that GPU's one array. Calls on one
 * stream are ordered and safe; calls that overlap on one GPU (different
 * streams, or threads without ordering) race on the array and give undefined
 * grad_w. Nothing in the array needs to start at zero (every partial row a call
 * reads is written by the same call first).
 */
rnq_status rnq_rmsnorm_rope_bwd_noalloc(const void* x, const void* w, const void* grad_y, const float* cos,
                                        const float* sin, const float* rstd, void* grad_x, float* grad_w,
                                        int64_t M, int64_t N, int64_t rope_dim, int64_t rows_per_token,
                                        float eps, int dtype, void* stream);

/*
 * RMSNorm + partial NeoX RoPE + FP8 with one scale per group (chapter 13
 * fusion page, rms_norm_rope_quant_fused: every group_size consecutive
 * elements of a row share one scale):
 *   y     = RMSNorm + RoPE as rnq_rmsnorm_rope (row m uses table row
 *           m / rows_per_token), rounded to dtype
 *   for every group g of row m (elements g*group_size .. (g+1)*group_size-1):
 *     scale[m,g] = max(max |y| over the group, 1e-4) / fp8_max    (fp32)
 *     code       = e4m3fn(clamp(y / scale[m,g], -fp8_max, fp8_max))  (nearest even)
 * x [M,N] in dtype; w [N]; cos, sin [M/rows_per_token, R/2] fp32 (NULL allowed
 * when R == 0); outputs codes [M,N] bytes (8-byte aligned), scales
 * [M, N/group_size] fp32, y [M,N] in dtype (optional, NULL = not written).
 * Requirements: N a multiple of 8, at most 16384; group_size = N (one scale per
 * row) or a power of two in [8, 512] dividing N (SHAPE if it does not divide,
 * UNSUPPORTED otherwise);
 * R = rope_dim a multiple of 16, R <= N, R <= 1024; M % rows_per_token == 0;
 * 0 < fp8_max <= 448; M < 2^31; each of cos and sin below 2 GiB (UNSUPPORTED).
 * 16-bit tensors and the table 16-byte aligned.
 */
rnq_status rnq_rmsnorm_rope_fp8_grouped(const void* x, const void* w, const float* cos, const float* sin,
                                        void* y, uint8_t* codes, float* scales, int64_t M, int64_t N,
                                        int64_t rope_dim, int64_t rows_per_token, int64_t group_size, float eps,
                                        float fp8_max, int dtype, void* stream);

/*
 * QK-norm + partial NeoX RoPE + per-row FP8 (chapter 28 page, the prologue;
 * chapter 13 fusion page, rms_norm_rope_quant_fused with one group per row):
 *   for every (token t, head h) row of q [T,Hq,D] (weight wq) and of
 *   k [T,Hk,D] (weight wk):
 *     y     = RMSNorm + RoPE as rnq_rmsnorm_rope, with table row t for every head
 *     amax  = max_j |y_j|
 *     scale = max(amax, 1e-4) / fp8_max                      (fp32, one per row)
 *     code  = e4m3fn(clamp(y_j / scale, -fp8_max, fp8_max))  (nearest even)
 * Outputs: q_fp8 [T,Hq,D], k_fp8 [T,Hk,D] bytes; q_scale [T,Hq], k_scale [T,Hk]
 * fp32; q_y / k_y [same as q / k] in dtype, optional (NULL = not written).
 * k, wk, k_fp8, k_scale may be NULL iff kv_heads == 0.
 * cos, sin: [T, R/2] fp32 (may be NULL iff rope_dim == 0).
 * Requirements: D = head_dim in {64, 128, 256, 512}; R = rope_dim a multiple of
 * 16 with R <= D; 0 < fp8_max <= 448; T*(Hq+Hk) < 2^31.
 */
rnq_status rnq_qk_norm_rope_fp8(const void* q, const void* k, const void* wq, const void* wk,
                                const float* cos, const float* sin,
                                uint8_t* q_fp8, uint8_t* k_fp8, float* q_scale, float* k_scale,
                                void* q_y, void* k_y,
                                int64_t tokens, int64_t q_heads, int64_t kv_heads,
                                int64_t head_dim, int64_t rope_dim,
                                float eps, float fp8_max, int dtype, void* stream);

/*
 * rnq_qk_norm_rope_fp8 on strided, position-indexed inputs (the chapter 28
 * page's prologue reads q and k straight from the projection output and
 * looks the rotation up by token position; chapter 13 fusion page, the
 * [tokens, rope_dim/2] cos/sin layout):
 *   * q_token_stride / k_token_stride: elements between the first rows of
 *     consecutive tokens; the Hq (Hk) rows of a token are contiguous. 0 means
 *     contiguous (Hq*D, Hk*D). Otherwise at least Hq*D (Hk*D) (SHAPE) and a
 *     multiple of 8 (UNSUPPORTED), e.g. q and k as views into a fused QKV
 *     output [T, (Hq + 2*Hk) * D].
 *   * positions: optional int32 [T] (4-byte aligned). When given, token t uses
 *     row positions[t] of cos/sin [table_rows, R/2]; a position outside
 *     [0, table_rows) reads row table_rows - 1 (nothing is read out of range).
 *     When NULL, cos/sin are [T, R/2] and table_rows is ignored.
 * Everything else (outputs contiguous) is as rnq_qk_norm_rope_fp8, which is
 * this call with strides 0 and no positions.
 */
rnq_status rnq_qk_norm_rope_fp8_ex(const void* q, int64_t q_token_stride, const void* k, int64_t k_token_stride,
                                   const void* wq, const void* wk, const float* cos, const float* sin,
                                   const int32_t* positions, int64_t table_rows,
                                   uint8_t* q_fp8, uint8_t* k_fp8, float* q_scale, float* k_scale,
                                   void* q_y, void* k_y,
                                   int64_t tokens, int64_t q_heads, int64_t kv_heads,
                                   int64_t head_dim, int64_t rope_dim,
                                   float eps, float fp8_max, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RNQ_H_ */

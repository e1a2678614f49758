// C ABI of librnq.so: argument validation and dispatch to the HIP kernels.
// The contract of every entry point is documented in include/rnq.h (the
// measurement baselines in include/rnq_baselines.h).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "rnq.h"
#include "rnq_baselines.h"
#include "rnq_launch.h"

namespace rnq {

static thread_local std::string g_last_error;

static rnq_status fail(rnq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static rnq_status fail(rnq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

static rnq_status ok() {
  g_last_error.clear();
  return RNQ_OK;
}

static rnq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RNQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static bool row_width_ok(int64_t n) { return n == 64 || n == 128 || n == 256 || n == 512; }

static rnq_status check_eps(float eps) {
  if (!(eps >= 0.0f) || !isfinite(eps)) return fail(RNQ_ERR_ARG, "eps must be finite and >= 0 (got %g)", (double)eps);
  return RNQ_OK;
}

static rnq_status check_dtype(int dtype) {
  if (dtype != RNQ_BF16 && dtype != RNQ_F16) return fail(RNQ_ERR_ARG, "unknown dtype %d", dtype);
  return RNQ_OK;
}

// rope_dim rules: even and <= width (the pages' checks), and a multiple of 16
// (both halves of the tail split into whole 16-byte chunks)
static rnq_status check_rope(int64_t rope_dim, int64_t width) {
  if (rope_dim < 0 || rope_dim % 2 != 0) return fail(RNQ_ERR_SHAPE, "rope_dim must be even and >= 0 (got %lld)", (long long)rope_dim);
  if (rope_dim > width) return fail(RNQ_ERR_SHAPE, "rope_dim %lld exceeds the row width %lld", (long long)rope_dim, (long long)width);
  if (rope_dim % 16 != 0) return fail(RNQ_ERR_UNSUPPORTED, "rope_dim must be a multiple of 16 (got %lld)", (long long)rope_dim);
  return RNQ_OK;
}

}  // namespace rnq

using namespace rnq;

extern "C" {

const char* rnq_status_string(int status) {
  switch (status) {
    case RNQ_OK: return "RNQ_OK";
    case RNQ_ERR_NULL: return "RNQ_ERR_NULL: a required pointer is NULL";
    case RNQ_ERR_SHAPE: return "RNQ_ERR_SHAPE: invalid shape";
    case RNQ_ERR_UNSUPPORTED: return "RNQ_ERR_UNSUPPORTED: width or alignment not supported";
    case RNQ_ERR_ARG: return "RNQ_ERR_ARG: invalid scalar argument";
    case RNQ_ERR_WORKSPACE: return "RNQ_ERR_WORKSPACE: workspace too small";
    case RNQ_ERR_HIP: return "RNQ_ERR_HIP: HIP runtime error";
    default: return "RNQ_ERR_UNKNOWN";
  }
}

const char* rnq_last_error(void) { return g_last_error.c_str(); }

int rnq_abi_version(void) { return 100; }

// One row-kernel launch over tensor 0 (heads0 heads per token) and tensor 1
// (heads1 heads per token), rows in token-major order.
static hipError_t launch_qk(const void* x0, int64_t xs0, const void* w0, uint8_t* c0, float* s0, void* y0,
                            const void* x1, int64_t xs1, const void* w1, uint8_t* c1, float* s1, void* y1,
                            const float* cos, const float* sin, const int32_t* positions, int64_t table_rows,
                            int64_t tokens, int64_t heads0, int64_t heads1, int64_t head_dim, int64_t rope_dim,
                            float eps, float fp8_max, int dtype, hipStream_t stream) {
  RowParams p = {};
  p.xs0 = (uint64_t)xs0;
  p.xs1 = (uint64_t)xs1;
  p.positions = positions;
  p.max_pos = (uint32_t)table_rows;
  p.x0 = (const uint16_t*)x0;
  p.w0 = (const uint16_t*)w0;
  p.c0 = c0;
  p.s0 = s0;
  p.y0 = (uint16_t*)y0;
  p.x1 = (const uint16_t*)x1;
  p.w1 = (const uint16_t*)w1;
  p.c1 = c1;
  p.s1 = s1;
  p.y1 = (uint16_t*)y1;
  p.cos = cos;
  p.sin = sin;
  p.rstd = nullptr;
  p.total_rows = (uint32_t)(tokens * (heads0 + heads1));
  p.heads = (uint32_t)(heads0 + heads1);
  p.heads0 = (uint32_t)heads0;
  p.rope = (uint32_t)rope_dim;
  p.eps = eps;
  p.fp8_max = fp8_max;
  return launch_rows(p, (int)head_dim, dtype == RNQ_BF16, true, stream);
}

// A token stride (elements between the first rows of consecutive tokens):
// 0 means contiguous; otherwise at least the token's rows and a multiple of 8
// (every row 16-byte aligned).
static rnq_status check_stride(const char* what, int64_t stride, int64_t rows_per_token, int64_t width) {
  if (stride == 0) return RNQ_OK;
  if (stride < rows_per_token * width)
    return fail(RNQ_ERR_SHAPE, "%s token stride %lld is below the token's %lld elements", what, (long long)stride,
                (long long)(rows_per_token * width));
  if (stride % 8 != 0)
    return fail(RNQ_ERR_UNSUPPORTED, "%s token stride %lld is not a multiple of 8 elements", what, (long long)stride);
  return RNQ_OK;
}

static rnq_status check_positions(const int32_t* positions, int64_t table_rows, int64_t rope_dim) {
  if (positions == nullptr || rope_dim == 0) return RNQ_OK;
  if (table_rows < 1) return fail(RNQ_ERR_SHAPE, "table_rows must be >= 1 when positions are given");
  if (table_rows >= ((int64_t)1 << 31)) return fail(RNQ_ERR_UNSUPPORTED, "table_rows must stay below 2^31");
  if (!aligned(positions, 4)) return fail(RNQ_ERR_UNSUPPORTED, "positions must be 4-byte aligned");
  return RNQ_OK;
}

rnq_status rnq_qk_norm_rope_fp8_ex(const void* q, int64_t q_token_stride, const void* k, int64_t k_token_stride,
                                   const void* wq, const void* wk, const float* cos, const float* sin,
                                   const int32_t* positions, int64_t table_rows,
                                   uint8_t* q_fp8, uint8_t* k_fp8, float* q_scale, float* k_scale,
                                   void* q_y, void* k_y,
                                   int64_t tokens, int64_t q_heads, int64_t kv_heads,
                                   int64_t head_dim, int64_t rope_dim,
                                   float eps, float fp8_max, int dtype, void* stream) {
  rnq_status s;
  if ((s = check_dtype(dtype)) != RNQ_OK) return s;
  if (tokens < 0 || q_heads < 0 || kv_heads < 0 || head_dim < 0)
    return fail(RNQ_ERR_SHAPE, "negative size (tokens %lld, q_heads %lld, kv_heads %lld, head_dim %lld)",
                (long long)tokens, (long long)q_heads, (long long)kv_heads, (long long)head_dim);
  if ((s = check_rope(rope_dim, head_dim)) != RNQ_OK) return s;
  if (!row_width_ok(head_dim)) return fail(RNQ_ERR_UNSUPPORTED, "head_dim must be 64, 128, 256 or 512 (got %lld)", (long long)head_dim);
  if ((s = check_stride("q", q_token_stride, q_heads, head_dim)) != RNQ_OK) return s;
  if ((s = check_stride("k", k_token_stride, kv_heads, head_dim)) != RNQ_OK) return s;
  if ((s = check_positions(positions, table_rows, rope_dim)) != RNQ_OK) return s;
  if ((s = check_eps(eps)) != RNQ_OK) return s;
  if (!(fp8_max > 0.0f && fp8_max <= 448.0f)) return fail(RNQ_ERR_ARG, "fp8_max must lie in (0, 448] (got %g)", (double)fp8_max);
  const int64_t heads = q_heads + kv_heads;
  if (heads > 0 && tokens > ((int64_t)1 << 31) / heads)
    return fail(RNQ_ERR_UNSUPPORTED, "tokens * heads must stay below 2^31");
  const int64_t rows = tokens * heads;
  if (rows == 0) return ok();
  if (q_heads > 0 && (!q || !wq || !q_fp8 || !q_scale)) return fail(RNQ_ERR_NULL, "q, wq, q_fp8 and q_scale are required when q_heads > 0");
  if (kv_heads > 0 && (!k || !wk || !k_fp8 || !k_scale)) return fail(RNQ_ERR_NULL, "k, wk, k_fp8 and k_scale are required when kv_heads > 0");
  if (rope_dim > 0 && (!cos || !sin)) return fail(RNQ_ERR_NULL, "cos and sin are required when rope_dim > 0");
  const void* a16[] = {q, k, wq, wk, cos, sin, q_y, k_y};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(RNQ_ERR_UNSUPPORTED, "tensor pointer %p is not 16-byte aligned", ptr);
  if (!aligned(q_fp8, 8) || !aligned(k_fp8, 8)) return fail(RNQ_ERR_UNSUPPORTED, "fp8 outputs must be 8-byte aligned");
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4)) return fail(RNQ_ERR_UNSUPPORTED, "scale outputs must be 4-byte aligned");

  const hipStream_t st = (hipStream_t)stream;
  if (q_heads > 0 && kv_heads > 0 && (q_y == nullptr) != (k_y == nullptr)) {
    // y for one tensor only: one launch per tensor, so that each launch writes y for all its rows or none
    hipError_t e = launch_qk(q, q_token_stride, wq, q_fp8, q_scale, q_y, nullptr, 0, nullptr, nullptr, nullptr,
                             nullptr, cos, sin, positions, table_rows, tokens, q_heads, 0, head_dim, rope_dim, eps,
                             fp8_max, dtype, st);
    if (e == hipSuccess)
      e = launch_qk(k, k_token_stride, wk, k_fp8, k_scale, k_y, nullptr, 0, nullptr, nullptr, nullptr, nullptr, cos,
                    sin, positions, table_rows, tokens, kv_heads, 0, head_dim, rope_dim, eps, fp8_max, dtype, st);
    return hip_status(e, "rnq_qk_norm_rope_fp8");
  }
  const bool q_first = q_heads > 0;  // tensor 0 is q unless there are no q heads
  const hipError_t e =
      q_first ? launch_qk(q, q_token_stride, wq, q_fp8, q_scale, q_y, k, k_token_stride, wk, k_fp8, k_scale, k_y, cos,
                          sin, positions, table_rows, tokens, q_heads, kv_heads, head_dim, rope_dim, eps, fp8_max,
                          dtype, st)
              : launch_qk(k, k_token_stride, wk, k_fp8, k_scale, k_y, nullptr, 0, nullptr, nullptr, nullptr, nullptr,
                          cos, sin, positions, table_rows, tokens, kv_heads, 0, head_dim, rope_dim, eps, fp8_max,
                          dtype, st);
  return hip_status(e, "rnq_qk_norm_rope_fp8");
}

rnq_status rnq_qk_norm_rope_fp8(const void* q, const void* k, const void* wq, const void* wk,
                                const float* cos, const float* sin,
                                uint8_t* q_fp8, uint8_t* k_fp8, float* q_scale, float* k_scale,
                                void* q_y, void* k_y,
                                int64_t tokens, int64_t q_heads, int64_t kv_heads,
                                int64_t head_dim, int64_t rope_dim,
                                float eps, float fp8_max, int dtype, void* stream) {
  return rnq_qk_norm_rope_fp8_ex(q, 0, k, 0, wq, wk, cos, sin, nullptr, 0, q_fp8, k_fp8, q_scale, k_scale, q_y, k_y,
                                 tokens, q_heads, kv_heads, head_dim, rope_dim, eps, fp8_max, dtype, stream);
}

rnq_status rnq_rmsnorm_rope_ex(const void* x, int64_t x_token_stride, const void* w, const float* cos,
                               const float* sin, const int32_t* positions, int64_t table_rows, void* y, int64_t M,
                               int64_t N, int64_t rope_dim, int64_t rows_per_token, float eps, int dtype,
                               void* stream) {
  rnq_status s;
  if ((s = check_dtype(dtype)) != RNQ_OK) return s;
  if (M < 0 || N < 0) return fail(RNQ_ERR_SHAPE, "negative size (M %lld, N %lld)", (long long)M, (long long)N);
  if ((s = check_rope(rope_dim, N)) != RNQ_OK) return s;
  if (rows_per_token < 1) return fail(RNQ_ERR_SHAPE, "rows_per_token must be >= 1");
  if (M % rows_per_token != 0) return fail(RNQ_ERR_SHAPE, "M (%lld) is not a multiple of rows_per_token (%lld)", (long long)M, (long long)rows_per_token);
  if (N % 8 != 0 || N > 16384)
    return fail(RNQ_ERR_UNSUPPORTED, "N must be a multiple of 8 and at most 16384 (got %lld)", (long long)N);
  const bool narrow = row_width_ok(N);
  if (!narrow && rope_dim > 1024)
    return fail(RNQ_ERR_UNSUPPORTED, "rope_dim must be at most 1024 on rows other than 64..512 wide (got %lld)", (long long)rope_dim);
  if ((s = check_stride("x", x_token_stride, rows_per_token, N)) != RNQ_OK) return s;
  if ((s = check_positions(positions, table_rows, rope_dim)) != RNQ_OK) return s;
  if ((s = check_eps(eps)) != RNQ_OK) return s;
  if (M >= ((int64_t)1 << 31)) return fail(RNQ_ERR_UNSUPPORTED, "M must stay below 2^31");
  if (!narrow && (positions != nullptr ? table_rows : M / rows_per_token) * (rope_dim / 2) * 4 >= ((int64_t)1 << 31))
    return fail(RNQ_ERR_UNSUPPORTED, "the cos/sin table must stay below 2 GiB");
  if (M == 0 || N == 0) return ok();
  if (!x || !w || !y) return fail(RNQ_ERR_NULL, "x, w and y are required");
  if (rope_dim > 0 && (!cos || !sin)) return fail(RNQ_ERR_NULL, "cos and sin are required when rope_dim > 0");
  const void* a16[] = {x, w, y, cos, sin};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(RNQ_ERR_UNSUPPORTED, "tensor pointer %p is not 16-byte aligned", ptr);

  if (!narrow) {
    // rows wider (or other) than a head: one workgroup per row
    GroupQuantParams g = {};
    g.x = (const uint16_t*)x;
    g.xs = (uint64_t)x_token_stride;
    g.w = (const uint16_t*)w;
    g.cos = cos;
    g.sin = sin;
    g.positions = rope_dim > 0 ? positions : nullptr;
    g.max_pos = (uint32_t)table_rows;
    g.y = (uint16_t*)y;
    g.M = (uint32_t)M;
    g.N = (uint32_t)N;
    g.rope = (uint32_t)rope_dim;
    g.rows_per_token = (uint32_t)rows_per_token;
    g.eps = eps;
    return hip_status(launch_wide_norm_rope(g, dtype == RNQ_BF16, (hipStream_t)stream), "rnq_rmsnorm_rope");
  }

  RowParams p = {};
  p.x0 = (const uint16_t*)x;
  p.xs0 = (uint64_t)x_token_stride;
  p.w0 = (const uint16_t*)w;
  p.y0 = (uint16_t*)y;
  p.cos = cos;
  p.sin = sin;
  p.positions = positions;
  p.max_pos = (uint32_t)table_rows;
  p.total_rows = (uint32_t)M;
  p.heads = (uint32_t)rows_per_token;
  p.heads0 = (uint32_t)rows_per_token;
  p.rope = (uint32_t)rope_dim;
  p.eps = eps;
  p.fp8_max = 448.0f;
  return hip_status(launch_rows(p, (int)N, dtype == RNQ_BF16, false, (hipStream_t)stream), "rnq_rmsnorm_rope");
}

rnq_status rnq_rmsnorm_rope(const void* x, const void* w, const float* cos, const float* sin,
                            void* y, int64_t M, int64_t N, int64_t rope_dim, int64_t rows_per_token,
                            float eps, int dtype, void* stream) {
  return rnq_rmsnorm_rope_ex(x, 0, w, cos, sin, nullptr, 0, y, M, N, rope_dim, rows_per_token, eps, dtype, stream);
}

rnq_status rnq_rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd_out,
                           int64_t M, int64_t N, float eps, int dtype, void* stream) {
  rnq_status s;
  if ((s = check_dtype(dtype)) != RNQ_OK) return s;
  if (M < 0 || N < 0) return fail(RNQ_ERR_SHAPE, "negative size (M %lld, N %lld)", (long long)M, (long long)N);
  if (N % 8 != 0 || N > 16384) return fail(RNQ_ERR_UNSUPPORTED, "N must be a multiple of 8 and at most 16384 (got %lld)", (long long)N);
  if ((s = check_eps(eps)) != RNQ_OK) return s;
  if (M >= ((int64_t)1 << 31)) return fail(RNQ_ERR_UNSUPPORTED, "M must stay below 2^31");
  if (M == 0 || N == 0) return ok();
  if (!x || !w || !y) return fail(RNQ_ERR_NULL, "x, w and y are required");
  const void* a16[] = {x, w, y};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(RNQ_ERR_UNSUPPORTED, "tensor pointer %p is not 16-byte aligned", ptr);
  if (!aligned(rstd_out, 4)) return fail(RNQ_ERR_UNSUPPORTED, "rstd_out must be 4-byte aligned");

  if (row_width_ok(N)) {
    RowParams p = {};
    p.x0 = (const uint16_t*)x;
    p.w0 = (const uint16_t*)w;
    p.y0 = (uint16_t*)y;
    p.rstd = rstd_out;
    p.total_rows = (uint32_t)M;
    p.heads = 1;
    p.heads0 = 1;
    p.rope = 0;
    p.eps = eps;
    p.fp8_max = 448.0f;
    return hip_status(launch_rows(p, (int)N, dtype == RNQ_BF16, false, (hipStream_t)stream), "rnq_rmsnorm_fwd");
  }
  WideFwdParams p = {};
  p.x = (const uint16_t*)x;
  p.w = (const uint16_t*)w;
  p.y = (uint16_t*)y;
  p.rstd = rstd_out;
  p.M = (uint32_t)M;
  p.N = (uint32_t)N;
  p.eps = eps;
  return hip_status(launch_wide_fwd(p, dtype == RNQ_BF16, (hipStream_t)stream), "rnq_rmsnorm_fwd");
}

rnq_status rnq_rmsnorm_rope_fp8_grouped(const void* x, const void* w, const float* cos, const float* sin,
                                        void* y, uint8_t* codes, float* scales, int64_t M, int64_t N,
                                        int64_t rope_dim, int64_t rows_per_token, int64_t group_size, float eps,
                                        float fp8_max, int dtype, void* stream) {
  rnq_status s;
  if ((s = check_dtype(dtype)) != RNQ_OK) return s;
  if (M < 0 || N < 0) return fail(RNQ_ERR_SHAPE, "negative size (M %lld, N %lld)", (long long)M, (long long)N);
  if ((s = check_rope(rope_dim, N)) != RNQ_OK) return s;
  if (rope_dim > 1024) return fail(RNQ_ERR_UNSUPPORTED, "rope_dim must be at most 1024 (got %lld)", (long long)rope_dim);
  if (rows_per_token < 1) return fail(RNQ_ERR_SHAPE, "rows_per_token must be >= 1");
  if (M % rows_per_token != 0)
    return fail(RNQ_ERR_SHAPE, "M (%lld) is not a multiple of rows_per_token (%lld)", (long long)M, (long long)rows_per_token);
  if (group_size <= 0 || (N > 0 && N % group_size != 0))
    return fail(RNQ_ERR_SHAPE, "group_size must divide N (N %lld, group_size %lld)", (long long)N, (long long)group_size);
  if (group_size != N && (group_size < 8 || group_size > 512 || (group_size & (group_size - 1)) != 0))
    return fail(RNQ_ERR_UNSUPPORTED, "group_size must be N or a power of two in [8, 512] (got %lld)", (long long)group_size);
  if (N % 8 != 0 || N > 16384) return fail(RNQ_ERR_UNSUPPORTED, "N must be a multiple of 8 and at most 16384 (got %lld)", (long long)N);
  if ((s = check_eps(eps)) != RNQ_OK) return s;
  if (!(fp8_max > 0.0f && fp8_max <= 448.0f)) return fail(RNQ_ERR_ARG, "fp8_max must lie in (0, 448] (got %g)", (double)fp8_max);
  if (M >= ((int64_t)1 << 31)) return fail(RNQ_ERR_UNSUPPORTED, "M must stay below 2^31");
  if ((M / rows_per_token) * (rope_dim / 2) * 4 >= ((int64_t)1 << 31))
    return fail(RNQ_ERR_UNSUPPORTED, "the cos/sin table must stay below 2 GiB");
  if (M == 0 || N == 0) return ok();
  if (!x || !w || !codes || !scales) return fail(RNQ_ERR_NULL, "x, w, codes and scales are required");
  if (rope_dim > 0 && (!cos || !sin)) return fail(RNQ_ERR_NULL, "cos and sin are required when rope_dim > 0");
  const void* a16[] = {x, w, y, cos, sin};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(RNQ_ERR_UNSUPPORTED, "tensor pointer %p is not 16-byte aligned", ptr);
  if (!aligned(codes, 8)) return fail(RNQ_ERR_UNSUPPORTED, "codes must be 8-byte aligned");
  if (!aligned(scales, 4)) return fail(RNQ_ERR_UNSUPPORTED, "scales must be 4-byte aligned");

  GroupQuantParams p = {};
  p.x = (const uint16_t*)x;
  p.w = (const uint16_t*)w;
  p.cos = cos;
  p.sin = sin;
  p.y = (uint16_t*)y;
  p.codes = codes;
  p.scales = scales;
  p.M = (uint32_t)M;
  p.N = (uint32_t)N;
  p.rope = (uint32_t)rope_dim;
  p.rows_per_token = (uint32_t)rows_per_token;
  p.group_size = (uint32_t)group_size;
  p.eps = eps;
  p.fp8_max = fp8_max;
  return hip_status(launch_group_quant(p, dtype == RNQ_BF16, (hipStream_t)stream), "rnq_rmsnorm_rope_fp8_grouped");
}

size_t rnq_rmsnorm_bwd_workspace_size(int64_t M, int64_t N) {
  if (M <= 0 || N <= 0) return 0;
  // (rope_dim 0, and 1024: past the wave-per-row kernel's tails, the largest partition)
  const uint32_t blocks = std::max(bwd_blocks(M, N, 0), bwd_blocks(M, N, 1024));
  return (size_t)blocks * (size_t)N * sizeof(float);
}

}  // extern "C"

namespace rnq {

// ------------------------------------------- allocation-free backward scratch
// For callers that cannot allocate: the grad_w partials of
// rnq_rmsnorm_rope_bwd_noalloc live in this file-scope device array (one copy
// per GPU, held until the process ends). Host code never passes `scratch`
// itself to a kernel (on the host it is only a stand-in for the symbol): each
// device's address is looked up once with hipGetSymbolAddress and kept here.
static __device__ __align__(256) float scratch[RNQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that runs `stream` (looked up on the
// first call on that device, with that device current).
static rnq_status scratch_for_stream(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RNQ_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(RNQ_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RNQ_OK;
}

// Shared by the three backward entry points: validation, then the narrow-row
// kernel for widths 64..512 (with or without the RoPE tail) or the wide one.
// With use_scratch the grad_w partials go to the static scratch above (looked
// up after every argument has been validated) instead of the caller's workspace.
static rnq_status rmsnorm_bwd_common(const char* name, const void* x, const void* w, const void* grad_y,
                                     const float* cos, const float* sin, const float* rstd, void* grad_x,
                                     float* grad_w, void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                                     int64_t rope_dim, int64_t rows_per_token, float eps, int dtype, void* stream,
                                     bool use_scratch = false) {
  rnq_status s;
  if ((s = check_dtype(dtype)) != RNQ_OK) return s;
  if (M < 0 || N < 0) return fail(RNQ_ERR_SHAPE, "negative size (M %lld, N %lld)", (long long)M, (long long)N);
  if (N % 8 != 0 || N > 16384) return fail(RNQ_ERR_UNSUPPORTED, "N must be a multiple of 8 and at most 16384 (got %lld)", (long long)N);
  if ((s = check_rope(rope_dim, N)) != RNQ_OK) return s;
  if (rope_dim > 1024 && !narrow_bwd_width(N))
    return fail(RNQ_ERR_UNSUPPORTED, "rope_dim must be at most 1024 on rows other than 64..512 wide (got %lld)", (long long)rope_dim);
  if (rows_per_token < 1) return fail(RNQ_ERR_SHAPE, "rows_per_token must be >= 1");
  if (M % rows_per_token != 0)
    return fail(RNQ_ERR_SHAPE, "M (%lld) is not a multiple of rows_per_token (%lld)", (long long)M, (long long)rows_per_token);
  if ((s = check_eps(eps)) != RNQ_OK) return s;
  if (M >= ((int64_t)1 << 31)) return fail(RNQ_ERR_UNSUPPORTED, "M must stay below 2^31");
  if (M == 0 || N == 0) return ok();
  if (!x || !w || !grad_y || !grad_x || !grad_w) return fail(RNQ_ERR_NULL, "x, w, grad_y, grad_x and grad_w are required");
  if (rope_dim > 0 && (!cos || !sin)) return fail(RNQ_ERR_NULL, "cos and sin are required when rope_dim > 0");
  const size_t need = rnq_rmsnorm_bwd_workspace_size(M, N);
  if (use_scratch) {
    if (need > (size_t)RNQ_NOALLOC_SCRATCH_BYTES)
      return fail(RNQ_ERR_WORKSPACE, "%s: M %lld, N %lld needs %zu bytes of scratch; the static scratch holds %zu", name,
                  (long long)M, (long long)N, need, (size_t)RNQ_NOALLOC_SCRATCH_BYTES);
  } else if (workspace == nullptr || workspace_bytes < need) {
    return fail(RNQ_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes, workspace);
  }
  const void* a16[] = {x, w, grad_y, grad_x, grad_w, use_scratch ? nullptr : workspace, cos, sin};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(RNQ_ERR_UNSUPPORTED, "tensor pointer %p is not 16-byte aligned", ptr);
  if (!aligned(rstd, 4)) return fail(RNQ_ERR_UNSUPPORTED, "rstd must be 4-byte aligned");
  const uint32_t blocks = bwd_blocks(M, N, rope_dim);
  const uint32_t rows_per_block = (uint32_t)((M + blocks - 1) / blocks);
  // the kernels address the tables (and the narrow and wave-per-row ones a
  // block's rows) with 32-bit offsets
  const int64_t table_bytes = (M / rows_per_token) * (rope_dim / 2) * 4;
  if (table_bytes >= ((int64_t)1 << 31) || ((narrow_bwd_width(N) || row_bwd_fits(N, rope_dim)) &&
                                            (int64_t)rows_per_block * N * 2 >= ((int64_t)1 << 31)))
    return fail(RNQ_ERR_UNSUPPORTED, "a block's rows or the cos/sin table exceed 2 GiB");
  if (use_scratch) {
    const rnq_status ss = scratch_for_stream((hipStream_t)stream, &workspace);
    if (ss != RNQ_OK) return ss;
  }

  WideBwdParams p = {};
  p.x = (const uint16_t*)x;
  p.w = (const uint16_t*)w;
  p.gy = (const uint16_t*)grad_y;
  p.rstd = rstd;
  p.gx = (uint16_t*)grad_x;
  p.gw = grad_w;
  p.partial = (float*)workspace;
  p.M = (uint32_t)M;
  p.N = (uint32_t)N;
  p.blocks = blocks;
  p.rows_per_block = rows_per_block;
  p.eps = eps;
  p.cos = cos;
  p.sin = sin;
  p.rope = (uint32_t)rope_dim;
  p.rows_per_token = (uint32_t)rows_per_token;
  p.table_bytes = (uint32_t)table_bytes;
  if (!narrow_bwd_width(N)) return hip_status(launch_wide_bwd(p, dtype == RNQ_BF16, (hipStream_t)stream), name);
  return hip_status(launch_narrow_bwd(p, dtype == RNQ_BF16, (hipStream_t)stream), name);
}

}  // namespace rnq

extern "C" {

rnq_status rnq_rmsnorm_bwd(const void* x, const void* w, const void* grad_y, const float* rstd,
                           void* grad_x, float* grad_w, void* workspace, size_t workspace_bytes,
                           int64_t M, int64_t N, float eps, int dtype, void* stream) {
  return rmsnorm_bwd_common("rnq_rmsnorm_bwd", x, w, grad_y, nullptr, nullptr, rstd, grad_x, grad_w, workspace,
                            workspace_bytes, M, N, 0, 1, eps, dtype, stream);
}

rnq_status rnq_rmsnorm_rope_bwd(const void* x, const void* w, const void* grad_y, const float* cos, const float* sin,
                                const float* rstd, void* grad_x, float* grad_w, void* workspace,
                                size_t workspace_bytes, int64_t M, int64_t N, int64_t rope_dim,
                                int64_t rows_per_token, float eps, int dtype, void* stream) {
  return rmsnorm_bwd_common("rnq_rmsnorm_rope_bwd", x, w, grad_y, cos, sin, rstd, grad_x, grad_w, workspace,
                            workspace_bytes, M, N, rope_dim, rows_per_token, eps, dtype, stream);
}

rnq_status rnq_rmsnorm_rope_bwd_noalloc(const void* x, const void* w, const void* grad_y, const float* cos,
                                        const float* sin, const float* rstd, void* grad_x, float* grad_w,
                                        int64_t M, int64_t N, int64_t rope_dim, int64_t rows_per_token, float eps,
                                        int dtype, void* stream) {
  return rmsnorm_bwd_common("rnq_rmsnorm_rope_bwd_noalloc", x, w, grad_y, cos, sin, rstd, grad_x, grad_w, nullptr,
                            0, M, N, rope_dim, rows_per_token, eps, dtype, stream, true);
}

// ------------------------------------------------------ measurement baselines

rnq_status rnq_baseline_norm_rope_quant_unfused(const void* x, const void* w, const float* cos, const float* sin,
                                                void* normed, void* rotated, uint8_t* codes, float* scales,
                                                int64_t M, int64_t N, int64_t rope_dim, int64_t rows_per_token,
                                                float eps, float fp8_max, int dtype, void* stream) {
  rnq_status s;
  if ((s = check_dtype(dtype)) != RNQ_OK) return s;
  if (M < 0 || N < 0) return fail(RNQ_ERR_SHAPE, "negative size (M %lld, N %lld)", (long long)M, (long long)N);
  if ((s = check_rope(rope_dim, N)) != RNQ_OK) return s;
  if (rows_per_token < 1) return fail(RNQ_ERR_SHAPE, "rows_per_token must be >= 1");
  if (M % rows_per_token != 0) return fail(RNQ_ERR_SHAPE, "M is not a multiple of rows_per_token");
  if (N % 8 != 0 || N > 16384) return fail(RNQ_ERR_UNSUPPORTED, "N must be a multiple of 8 and at most 16384 (got %lld)", (long long)N);
  if ((s = check_eps(eps)) != RNQ_OK) return s;
  if (!(fp8_max > 0.0f && fp8_max <= 448.0f)) return fail(RNQ_ERR_ARG, "fp8_max must lie in (0, 448] (got %g)", (double)fp8_max);
  if (M >= ((int64_t)1 << 31)) return fail(RNQ_ERR_UNSUPPORTED, "M must stay below 2^31");
  if (M == 0 || N == 0) return ok();
  if (!x || !w || !normed || !rotated || !codes || !scales) return fail(RNQ_ERR_NULL, "x, w, normed, rotated, codes and scales are required");
  if (rope_dim > 0 && (!cos || !sin)) return fail(RNQ_ERR_NULL, "cos and sin are required when rope_dim > 0");
  const void* a16[] = {x, w, normed, rotated, cos, sin};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(RNQ_ERR_UNSUPPORTED, "tensor pointer %p is not 16-byte aligned", ptr);
  if (!aligned(codes, 8) || !aligned(scales, 4)) return fail(RNQ_ERR_UNSUPPORTED, "codes 8-byte, scales 4-byte aligned");
  // step 1: the library's RMSNorm forward
  if ((s = rnq_rmsnorm_fwd(x, w, normed, nullptr, M, N, eps, dtype, stream)) != RNQ_OK) return s;
  // steps 2 and 3
  return hip_status(launch_unfused_rope_quant((const uint16_t*)normed, cos, sin, (uint16_t*)rotated, codes, scales,
                                              (uint32_t)M, (uint32_t)N, (uint32_t)rope_dim, (uint32_t)rows_per_token,
                                              fp8_max, dtype == RNQ_BF16, (hipStream_t)stream),
                    "rnq_baseline_norm_rope_quant_unfused");
}

rnq_status rnq_baseline_qk_design(const void* q, const void* k, const void* wq, const void* wk, const float* cos,
                                  const float* sin, uint8_t* q_fp8, uint8_t* k_fp8, float* q_scale, float* k_scale,
                                  int64_t tokens, int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                                  int64_t rope_dim, int64_t rows_per_block, float eps, float fp8_max, int dtype,
                                  void* stream) {
  rnq_status s;
  if ((s = check_dtype(dtype)) != RNQ_OK) return s;
  if (tokens < 0 || q_heads < 0 || kv_heads < 0 || head_dim < 0) return fail(RNQ_ERR_SHAPE, "negative size");
  if ((s = check_rope(rope_dim, head_dim)) != RNQ_OK) return s;
  if (!row_width_ok(head_dim)) return fail(RNQ_ERR_UNSUPPORTED, "head_dim must be 64, 128, 256 or 512 (got %lld)", (long long)head_dim);
  const int64_t heads = q_heads + kv_heads;
  if (rows_per_block < 1 || heads % rows_per_block != 0)
    return fail(RNQ_ERR_SHAPE, "rows_per_block (%lld) must divide the heads per token (%lld)", (long long)rows_per_block, (long long)heads);
  if (rows_per_block * (head_dim / 8) > 1024)
    return fail(RNQ_ERR_UNSUPPORTED, "rows_per_block * head_dim / 8 must be at most 1024 threads");
  if ((s = check_eps(eps)) != RNQ_OK) return s;
  if (!(fp8_max > 0.0f && fp8_max <= 448.0f)) return fail(RNQ_ERR_ARG, "fp8_max must lie in (0, 448] (got %g)", (double)fp8_max);
  if (heads > 0 && tokens > ((int64_t)1 << 31) / heads) return fail(RNQ_ERR_UNSUPPORTED, "tokens * heads must stay below 2^31");
  if (tokens * heads == 0) return ok();
  if (q_heads > 0 && (!q || !wq || !q_fp8 || !q_scale)) return fail(RNQ_ERR_NULL, "q, wq, q_fp8 and q_scale are required");
  if (kv_heads > 0 && (!k || !wk || !k_fp8 || !k_scale)) return fail(RNQ_ERR_NULL, "k, wk, k_fp8 and k_scale are required");
  if (rope_dim > 0 && (!cos || !sin)) return fail(RNQ_ERR_NULL, "cos and sin are required when rope_dim > 0");
  const void* a16[] = {q, k, wq, wk, cos, sin};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(RNQ_ERR_UNSUPPORTED, "tensor pointer %p is not 16-byte aligned", ptr);
  if (!aligned(q_fp8, 8) || !aligned(k_fp8, 8) || !aligned(q_scale, 4) || !aligned(k_scale, 4))
    return fail(RNQ_ERR_UNSUPPORTED, "codes 8-byte, scales 4-byte aligned");
  const bool q_first = q_heads > 0;
  RowParams p = {};
  p.x0 = (const uint16_t*)(q_first ? q : k);
  p.w0 = (const uint16_t*)(q_first ? wq : wk);
  p.c0 = q_first ? q_fp8 : k_fp8;
  p.s0 = q_first ? q_scale : k_scale;
  p.x1 = (const uint16_t*)(q_first ? k : nullptr);
  p.w1 = (const uint16_t*)(q_first ? wk : nullptr);
  p.c1 = q_first ? k_fp8 : nullptr;
  p.s1 = q_first ? k_scale : nullptr;
  p.cos = cos;
  p.sin = sin;
  p.total_rows = (uint32_t)(tokens * heads);
  p.heads = (uint32_t)heads;
  p.heads0 = (uint32_t)(q_first ? q_heads : kv_heads);
  p.rope = (uint32_t)rope_dim;
  p.eps = eps;
  p.fp8_max = fp8_max;
  return hip_status(launch_design(p, (uint32_t)rows_per_block, (int)head_dim, dtype == RNQ_BF16, (hipStream_t)stream),
                    "rnq_baseline_qk_design");
}

static rnq_status baseline_stream(const char* name, const void* src, int64_t src_bytes, void* dst,
                                  int store_policy, void* stream) {
  if (store_policy != 0 && store_policy != 1)
    return fail(RNQ_ERR_ARG, "store_policy must be 0 (nontemporal) or 1 (device scope), got %d", store_policy);
  if (src_bytes < 0 || src_bytes % 2048 != 0)
    return fail(RNQ_ERR_SHAPE, "src_bytes must be a non-negative multiple of 2048 (got %lld)", (long long)src_bytes);
  if (src_bytes / 2048 >= ((int64_t)1 << 31)) return fail(RNQ_ERR_UNSUPPORTED, "src_bytes / 2048 must stay below 2^31");
  if (src_bytes > 0 && (!src || !dst)) return fail(RNQ_ERR_NULL, "src and dst are required");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(RNQ_ERR_UNSUPPORTED, "src and dst must be 16-byte aligned");
  if (src_bytes > 0) {
    const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (uintptr_t)src_bytes;
    const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (uintptr_t)(src_bytes / 2);
    if (s0 < d1 && d0 < s1) return fail(RNQ_ERR_ARG, "src and dst overlap");
  }
  return hip_status(launch_stream(src, dst, (uint32_t)(src_bytes / 2048), store_policy == 1, (hipStream_t)stream),
                    name);
}

rnq_status rnq_baseline_stream(const void* src, int64_t src_bytes, void* dst, void* stream) {
  return baseline_stream("rnq_baseline_stream", src, src_bytes, dst, 0, stream);
}

rnq_status rnq_baseline_stream_policy(const void* src, int64_t src_bytes, void* dst, int store_policy,
                                      void* stream) {
  return baseline_stream("rnq_baseline_stream_policy", src, src_bytes, dst, store_policy, stream);
}

}  // extern "C"

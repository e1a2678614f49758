/*
 * rnq measurement baselines: the designs the fused prologue is compared with.
 * Not part of the hot path; same conventions as rnq.h (device pointers, int64
 * sizes, status codes, every argument validated before anything is enqueued,
 * asynchronous on `stream`, the caller owns all memory).
 */
#ifndef RNQ_BASELINES_H
#define RNQ_BASELINES_H

#include "rnq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The unfused plan of the chapter 13 ledger page ("norm+rope+quant, 3
 * kernels"): RMSNorm -> RoPE -> per-row FP8 as three launches whose
 * intermediates go through memory:
 *   1. normed  [M,N] = rnq_rmsnorm_fwd(x, w)                   (rounded to dtype)
 *   2. rotated [M,N] = normed with the last R columns rotated  (rounded to dtype;
 *      table row m / rows_per_token of cos/sin [M/rows_per_token, R/2] fp32)
 *   3. scales[m] = max(max_j |rotated[m,j]|, 1e-4) / fp8_max, codes = e4m3fn(clamp(rotated / scale))
 * The arithmetic is that of rnq_rmsnorm_rope_fp8_grouped with group_size = N, so
 * codes and scales are identical to it; normed and rotated are caller-owned
 * scratch [M,N] in dtype. Requirements: N a multiple of 8 and at most 16384;
 * R a multiple of 16, R <= N; M % rows_per_token == 0; 0 < fp8_max <= 448.
 */
rnq_status rnq_baseline_norm_rope_quant_unfused(const void* x, const void* w, const float* cos, const float* sin,
                                                void* normed, void* rotated, uint8_t* codes, float* scales,
                                                int64_t M, int64_t N, int64_t rope_dim, int64_t rows_per_token,
                                                float eps, float fp8_max, int dtype, void* stream);

/*
 * The chapter 28 page's designs for QK-norm + RoPE + FP8 (its `Design`: rows
 * per block, and the lookups a block makes): each workgroup owns
 * rows_per_block consecutive (token, head) rows and loads both weight vectors
 * and the token's cos/sin row once into LDS. rows_per_block = 1 is design A,
 * 8 design B, q_heads + kv_heads (one token per block) design C. Arguments and
 * outputs as rnq_qk_norm_rope_fp8 (no y), whose results these equal.
 * Requirements: rows_per_block divides q_heads + kv_heads and
 * rows_per_block * head_dim / 8 <= 1024.
 */
rnq_status rnq_baseline_qk_design(const void* q, const void* k, const void* wq, const void* wk, const float* cos,
                                  const float* sin, uint8_t* q_fp8, uint8_t* k_fp8, float* q_scale, float* k_scale,
                                  int64_t tokens, int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                                  int64_t rope_dim, int64_t rows_per_block, float eps, float fp8_max, int dtype,
                                  void* stream);

/*
 * The HBM floor the prologue is measured against: a kernel with the same kind
 * of traffic and no arithmetic. Reads src_bytes (a multiple of 2048) and
 * writes src_bytes / 2 to dst: the 1 KB block b of dst is the bytewise XOR of
 * the two 1 KB halves of the 2 KB block b of src (one wave per block, 16-byte
 * nontemporal accesses). src_bytes == 0 launches one empty workgroup (the cost
 * of a launch). src and dst 16-byte aligned and not overlapping (ARG);
 * src_bytes / 2048 < 2^31.
 */
rnq_status rnq_baseline_stream(const void* src, int64_t src_bytes, void* dst, void* stream);

/*
 * The same floor with dst stored under a chosen cache policy: store_policy 0 is
 * nontemporal (as rnq_baseline_stream), 1 is device scope (the sc1 bit alone).
 * Which is faster depends on the size (measured on MI355X: device scope at tens
 * to hundreds of MB, nontemporal at a few MB and at gigabytes), so a floor is
 * the faster of the two. Errors as rnq_baseline_stream, and ARG for another
 * store_policy.
 */
rnq_status rnq_baseline_stream_policy(const void* src, int64_t src_bytes, void* dst, int store_policy,
                                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RNQ_BASELINES_H */

/*
 * rmsnorm_matmul.h - C ABI of RMSNorm followed by a MatMul on MI355X (gfx950),
 * in the same library as attn_mi355x.h (whose status codes, dtypes and
 * attn_last_error() it shares).
 *
 *   Y = RMSNorm(X) W^T,  RMSNorm(x)_k = x_k g_k / sqrt(mean_k(x^2) + eps)
 *
 * computed in the rewritten form of the Cleave paper (§1 and Fig. 1, "RMSNorm
 * followed by a Matmul"): the row scale 1 / sqrt(mean(x^2) + eps) is applied
 * after the Matmul, so one pass over each X tile feeds both reductions (the
 * dot products and the row's sum of squares) and the normalised input is
 * never formed.  When there are too few output tiles to fill the GPU (the
 * decode setting of Cleave §7.3: a few tokens) the K axis is split in s parts
 * (Cleave §2.2 "Split-K"); a second launch adds the parts up and scales.
 *
 * Conventions: X [m, k], g [k], W [n, k] (linear-layer weights, one row per
 * output column), Y [m, n], each row-major with the given row stride (in
 * elements) and a contiguous last dimension.  x, g, w, y and ws are DEVICE
 * pointers; problem and plan are host pointers.  The caller owns every buffer;
 * the library allocates nothing.  Calls only enqueue work on `stream`
 * (hipStream_t as void*, NULL = default stream).  All checks happen before
 * anything is enqueued; a failing call returns a nonzero attn_status and
 * attn_last_error() describes it.
 */
#ifndef RMSNORM_MATMUL_H
#define RMSNORM_MATMUL_H

#include <stddef.h>
#include <stdint.h>

#include "attn_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One problem.  Zero-initialise, then fill every field. */
typedef struct rmsnorm_matmul_problem {
  int32_t dtype;     /* attn_dtype of X, g and W: ATTN_BF16 (ATTN_F32 is unsupported) */
  int32_t y_dtype;   /* attn_dtype of Y: ATTN_BF16 (round to nearest even) or ATTN_F32 */
  int32_t m;         /* tokens (rows of X and Y), >= 0 */
  int32_t k;         /* hidden size, >= 8 and a multiple of 8 */
  int32_t n;         /* output columns (rows of W), >= 0 */
  float eps;         /* >= 0, finite; Llama-3 uses 1e-5 */
  int64_t x_stride;  /* elements between rows of X (>= k, a multiple of 8) */
  int64_t w_stride;  /* elements between rows of W (>= k, a multiple of 8) */
  int64_t y_stride;  /* elements between rows of Y (>= n) */
} rmsnorm_matmul_problem;

/* The split of K chosen by rmsnorm_matmul_plan.  Valid only for problems with
 * the same dtype, m, k and n. */
typedef struct rmsnorm_matmul_config {
  int32_t s;            /* K parts, >= 1 */
  int32_t k_chunk;      /* columns per part, a multiple of 32 */
  uint32_t grid[3];     /* split-kernel grid: tile_n-column tiles of n, s, 32-row tiles of m */
  uint32_t block;       /* split-kernel threads per workgroup */
  int32_t kernel;       /* 0: split-K streaming kernel (decode setting); 1: tiled GEMM
                           (prefill setting, m >= 256 and k a multiple of 64) */
  int32_t tile_n;       /* kernel 0: output columns (rows of W) per workgroup, a multiple
                           of 4 in [4, 64], grid[0] = ceil(n / tile_n); kernel 1: 0 */
  uint64_t ws_bytes;    /* workspace bytes: kernel 0: (s*m*n + s*m) * 4 when s > 1, else 0;
                           kernel 1: m*k*4 (X * g as bf16 pairs) rounded up to 256,
                           plus m*4 */
  uint64_t problem_key; /* fingerprint of the planned problem */
} rmsnorm_matmul_config;

/*
 * rmsnorm_matmul_plan - choose s (Cleave §2.2 "Split-K"; §7.3 decode setting).
 *
 * With m >= 256 tokens and k a multiple of 64 the plan is the tiled GEMM
 * (kernel 1; s = 1, s_request is ignored); otherwise kernel 0:
 * s_request  <= 0: the planner picks the largest s whose workgroups (one
 *            per 64 x 32 output tile and part; the four waves of a workgroup
 *            split the part's columns among themselves) fit on num_cus compute
 *            units at once, with at least 512 columns of K per part.  > 0:
 *            s = min(s_request, k / 32), rounded to whole 32-column steps.
 * num_cus    compute units to plan for; <= 0 queries the current device.
 * Returns ATTN_OK, ATTN_ERR_ARG, ATTN_ERR_UNSUPPORTED or ATTN_ERR_HIP (device
 * query failed).  Enqueues nothing.
 */
int rmsnorm_matmul_plan(const rmsnorm_matmul_problem* problem, int32_t s_request,
                        int32_t num_cus, rmsnorm_matmul_config* out);

/*
 * rmsnorm_matmul - Y = RMSNorm(X) W^T.
 * Kernel 0 (decode setting): with plan->s == 1 one launch writes Y;
 * otherwise the split launch writes each part's dot products U_j [m, n] and
 * sums of squares SSQ_j [m] to ws, and the combine launch writes
 * Y = (sum_j U_j) / sqrt(sum_j SSQ_j / k + eps).
 * Kernel 1 (prefill setting, Cleave §7.3): a first pass writes X * g,
 * exactly, as a pair of bf16 matrices hi + lo, and every row's scale
 * 1 / sqrt(mean(x^2) + eps) to ws; the tiled MFMA GEMM then computes
 * (hi + lo) W^T and multiplies each row by its scale in its epilogue (the
 * division after the MatMul, Cleave §1).
 * ws may be NULL when plan->ws_bytes == 0.  x, g and w must be 16-byte
 * aligned (ATTN_ERR_UNSUPPORTED otherwise).  Calls sharing one workspace must
 * not overlap.
 */
int rmsnorm_matmul(const rmsnorm_matmul_problem* problem, const rmsnorm_matmul_config* plan,
                   const void* x, const void* g, const void* w, void* y, float* ws,
                   size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MATMUL_H */

/*
 * swiglu.h - C ABI of SwiGLU on MI355X (gfx950), in the same library as
 * attn_mi355x.h (whose status codes, dtypes and attn_last_error() it shares).
 *
 *   H = silu(X W_gate^T) * (X W_up^T),  silu(z) = z / (1 + exp(-z))
 *
 * Both MatMuls reduce over K and read the same X, so they are fused
 * horizontally (Cleave §7.3): each X tile feeds both reductions in one loop
 * and each weight matrix is read once.
 * When there are too few output tiles to fill the GPU (the decode setting:
 * a few tokens) the K axis is split in s parts (Cleave §2.2 "Split-K"); the
 * parts of both MatMuls are added up in a second launch, which then applies
 * the gate (silu is nonlinear, so it cannot act on the parts).
 *
 * Conventions: X [m, k], W_gate and W_up [n, k] (linear-layer weights, one
 * row per output column), H [m, n], row-major with the given row strides (in
 * elements) and a contiguous last dimension.  x, w_gate, w_up, y and ws are
 * DEVICE pointers; problem and config are host pointers.  The caller owns
 * every buffer; the library allocates nothing.  Calls only enqueue work on
 * `stream` (hipStream_t as void*, NULL = default stream).  All checks happen
 * before anything is enqueued; a failing call returns a nonzero attn_status
 * and attn_last_error() describes it.
 */
#ifndef SWIGLU_H
#define SWIGLU_H

#include <stddef.h>
#include <stdint.h>

#include "attn_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One problem.  Zero-initialise, then fill every field. */
typedef struct swiglu_problem {
  int32_t dtype;      /* attn_dtype of X, W_gate and W_up: ATTN_BF16 (ATTN_F32 is unsupported) */
  int32_t y_dtype;    /* attn_dtype of H: ATTN_BF16 (round to nearest even) or ATTN_F32 */
  int32_t m;          /* tokens, >= 0 */
  int32_t k;          /* hidden size, >= 8 and a multiple of 8 */
  int32_t n;          /* output columns (rows of each weight matrix), >= 0 */
  int32_t reserved0;  /* must be 0 */
  int64_t x_stride;   /* elements between rows of X (>= k, a multiple of 8) */
  int64_t wg_stride;  /* elements between rows of W_gate (>= k, a multiple of 8) */
  int64_t wu_stride;  /* elements between rows of W_up (>= k, a multiple of 8) */
  int64_t y_stride;   /* elements between rows of H (>= n) */
} swiglu_problem;

/* The split of K chosen by swiglu_plan.  Valid only for problems with the
 * same dtype, m, k and n. */
typedef struct swiglu_config {
  int32_t s;            /* K parts, >= 1 */
  int32_t k_chunk;      /* columns per part, a multiple of 32 */
  uint32_t grid[3];     /* split-kernel grid: tile_n-column tiles of n, s, 32-row tiles of m */
  uint32_t block;       /* split-kernel threads per workgroup */
  int32_t kernel;       /* 0: split-K streaming kernel (decode setting); 1: tiled GEMM
                           of both MatMuls at once (prefill setting, m >= 256 and k a
                           multiple of 64; no workspace) */
  int32_t tile_n;       /* kernel 0: output columns (rows of each W) per workgroup, a
                           multiple of 4 in [4, 64], grid[0] = ceil(n / tile_n); kernel 1: 0 */
  uint64_t ws_bytes;    /* fp32 workspace: 2 * s * m * n * 4 bytes when s > 1, else 0 */
  uint64_t problem_key; /* fingerprint of the planned problem */
} swiglu_config;

/*
 * swiglu_plan - choose s (Cleave §2.2 "Split-K"; §7.3 decode and prefill).
 * With m >= 256 tokens and k a multiple of 64 the plan is the tiled GEMM
 * (kernel 1; s = 1, s_request is ignored); otherwise kernel 0:
 * s_request  <= 0: the largest s whose workgroups (one per 64 x 32 output
 *            tile and part; two waves split each part's columns) fit on
 *            num_cus compute units at once, with at least 256 columns of K per
 *            part.  > 0: s = min(s_request, k / 32).
 * num_cus    compute units to plan for; <= 0 queries the current device.
 * Returns ATTN_OK, ATTN_ERR_ARG, ATTN_ERR_UNSUPPORTED or ATTN_ERR_HIP.
 */
int swiglu_plan(const swiglu_problem* problem, int32_t s_request, int32_t num_cus,
                swiglu_config* out);

/*
 * swiglu - H = silu(X W_gate^T) * (X W_up^T).  With config->s == 1 one launch
 * writes H; otherwise the split launch writes each part's G_j and U_j [m, n]
 * to ws (G parts first, then U parts), and the combine launch writes
 * H = silu(sum_j G_j) * sum_j U_j.  ws may be NULL when config->ws_bytes == 0.
 * x, w_gate and w_up must be 16-byte aligned (ATTN_ERR_UNSUPPORTED
 * otherwise).  Calls sharing one workspace must not overlap.
 */
int swiglu(const swiglu_problem* problem, const swiglu_config* config, const void* x,
           const void* w_gate, const void* w_up, void* y, float* ws, size_t ws_bytes,
           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_H */

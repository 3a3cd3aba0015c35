/*
 * attn_mi355x.h - C ABI of the MI355X (gfx950, CDNA4) fused-attention library.
 *
 * The library computes softmax attention O = softmax(tau * Q K^T) V for
 * grouped-query heads, in the rewritten form of the Cleave paper ("Cleave:
 * Scaling Tensor Program Optimization via Decoupled Algebraic Search and
 * Operator Scheduling"), §2.2 "FlashAttention" and Fig. 2: the softmax
 * division is moved after the V-matmul, so a kernel streams one K/V tile at a
 * time, keeps a running row max and row sum, and never materialises S or P.
 * Decode splits the key/value reduction into s parts (§2.2 "Split-K",
 * Fig. 3; §4, Fig. 5(b)) and merges them in a second launch.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are described by an attn_problem.  Q is [B, Lq, Hq, Dqk], K is
 *   [B, Lcap, Hkv, Dqk], V is [B, Lcap, Hkv, Dv], O is [B, Lq, Hq, Dv], each
 *   addressed with explicit element strides for (batch, token, head); the
 *   head dimension is contiguous.  Any layout expressible that way works,
 *   e.g. token-major [B, L, H, D] or head-major [B, H, L, D].
 * - GQA: query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 * - Causal masking is bottom-right aligned: query row i of a request with
 *   Lq query rows and L_b keys sees key j iff j <= i + L_b - Lq.  A row that
 *   sees no key gets O = 0 and LSE = -inf.
 * - MLA (one latent KV head whose first Dv columns are V): pass v = k with
 *   v_stride = k_stride and head_dim_v < head_dim_qk.
 * - Variable-length and paged layouts (the paged and ragged attention
 *   operators of the Cleave paper's dynamic-operator benchmark, §7.1 and
 *   §7.4).  Three optional DEVICE index arrays change how rows are found;
 *   each is NULL for the plain layout above:
 *     kv_indptr  packed keys: request b owns rows kv_indptr[b] ..
 *                kv_indptr[b+1] - 1 of K [T, Hkv, Dqk] and V [T, Hkv, Dv]; key
 *                t is at (kv_indptr[b] + t) * k_stride[1] + head * k_stride[2]
 *                (k_stride[0] unused) and L_b = kv_indptr[b+1] - kv_indptr[b].
 *     page_table paged keys: K and V are pools of num_pages pages of
 *                page_size rows; request b's key t lives on page
 *                page_table[b * pages_per_req + t / page_size] at row
 *                t % page_size: offset page * k_stride[0] +
 *                (t % page_size) * k_stride[1] + head * k_stride[2].  Page ids
 *                are clamped to [0, num_pages) before use, so a bad id reads
 *                the wrong page but never outside the pool.  L_b comes from
 *                kv_lens (or is Lcap), as in the plain layout.
 *     q_indptr   packed (ragged) queries, attn_prefill only: request b owns
 *                rows q_indptr[b] .. q_indptr[b+1] - 1 of Q [T, Hq, Dqk] and
 *                O [T, Hq, Dv] (q_stride[0] and o_stride[0] unused), so it has
 *                Lq_b = q_indptr[b+1] - q_indptr[b] query rows, with Lq an
 *                upper bound on every Lq_b; lse_out is then [T, Hq].  Causal
 *                masking uses Lq_b: row i sees key j iff j <= i + L_b - Lq_b.
 *                O and LSE rows of the packed tensor that no request owns are
 *                not written.
 *   Lengths taken from an indptr are clamped to [0, Lq] / [0, Lcap] on the
 *   device; an indptr must be non-decreasing.  kv_indptr excludes kv_lens and
 *   page_table.
 * - Pointers named q, k, v, o, ws_*, lse_out and problem->kv_lens are DEVICE
 *   pointers.  Pointers to attn_problem / attn_plan and kv_lens_host are host
 *   pointers.  The caller owns every buffer; the library allocates no device
 *   memory and keeps no per-call state.
 * - stream is a hipStream_t passed as void* (NULL = the default stream).
 *   Every compute call only enqueues work and returns; buffers must stay
 *   valid until that work has finished.
 * - Errors: every argument and shape check happens before anything is
 *   enqueued; a failing call returns a nonzero attn_status and enqueues
 *   nothing.  A failed launch returns ATTN_ERR_HIP.  attn_last_error()
 *   returns a message for the calling thread's last failure.  No C++
 *   exception crosses this interface.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_MI355X_VERSION 7

typedef enum attn_dtype {
  ATTN_F32 = 0,   /* IEEE binary32 */
  ATTN_BF16 = 1   /* bfloat16; outputs are rounded to nearest, ties to even */
} attn_dtype;

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_ARG = 1,          /* a null pointer, a negative size, Hq % Hkv != 0, a bad stride ... */
  ATTN_ERR_UNSUPPORTED = 2,  /* a valid problem this library has no kernel for */
  ATTN_ERR_WORKSPACE = 3,    /* a workspace smaller than the plan asks for */
  ATTN_ERR_HIP = 4           /* a HIP runtime call or a kernel launch failed */
} attn_status;

/* One attention problem.  Zero-initialise, then fill every field. */
typedef struct attn_problem {
  int32_t dtype;        /* attn_dtype of Q, K and V */
  int32_t o_dtype;      /* attn_dtype of O */
  int32_t batch;        /* B >= 0 requests */
  int32_t q_heads;      /* Hq >= 1 */
  int32_t kv_heads;     /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim_qk;  /* Dqk >= 1 */
  int32_t head_dim_v;   /* Dv >= 1 (Dv <= Dqk when V aliases K) */
  int32_t q_len;        /* Lq >= 1 query rows per request */
  int32_t kv_len_max;   /* Lcap >= 0: K/V capacity rows per request */
  int32_t causal;       /* 0 or 1; bottom-right aligned */
  float scale;          /* softmax scale tau; <= 0 selects 1/sqrt(Dqk) */
  int32_t reserved0;    /* must be 0 */
  /* DEVICE pointer to B int32 key counts; each is clamped to [0, Lcap] on the
   * device.  NULL means every request has Lcap keys. */
  const int32_t* kv_lens;
  int64_t q_stride[3];  /* element strides of Q for (batch, token, head) */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  /* Variable-length and paged layouts (see above); NULL / 0 when unused. */
  const int32_t* q_indptr;    /* DEVICE int32 [B + 1] or NULL */
  const int32_t* kv_indptr;   /* DEVICE int32 [B + 1] or NULL */
  const int32_t* page_table;  /* DEVICE int32 [B * pages_per_req] or NULL */
  int32_t page_size;          /* rows per page >= 1 (0 without page_table) */
  int32_t pages_per_req;      /* page_table row length >= ceil(Lcap / page_size) */
  int32_t num_pages;          /* pages in the K and V pools >= 1 */
  int32_t reserved1;          /* must be 0 */
} attn_problem;

/* Kernel families the decode planner can pick. */
typedef enum attn_decode_kernel {
  ATTN_KERNEL_GENERIC = 0,  /* vector-ALU kernel: any head dim, f32 or bf16 */
  ATTN_KERNEL_GQA_D128 = 1, /* bf16 MFMA, Dqk = Dv = 128, G*Lq <= 16 rows per KV head */
  ATTN_KERNEL_MLA = 2       /* bf16 MFMA, Dqk = 576, Dv = 512, V aliases K */
} attn_decode_kernel;

/* The split decomposition chosen by attn_decode_plan.  Treat as opaque
 * except for the workspace sizes; it is valid only with problems of the same
 * shapes, input dtype and causal flag as the one it was planned for (the
 * output dtype and the strides may differ). */
typedef struct attn_plan {
  int32_t kernel;         /* attn_decode_kernel */
  int32_t s_max;          /* split slots: ceil(max planned length / chunk), >= 1 */
  int32_t chunk;          /* keys per split, a multiple of tile_n */
  int32_t tile_n;         /* keys per inner tile of the chosen kernel */
  int32_t rows_per_unit;  /* G * Lq query rows that share one KV head */
  int32_t row_tiles;      /* row tiles per (request, KV head) */
  uint32_t grid[3];       /* split-kernel grid */
  uint32_t block;         /* split-kernel threads per workgroup */
  uint64_t ws_o_bytes;    /* bytes needed for ws_o: s_max*B*Lq*Hq*Dv floats */
  uint64_t ws_lse_bytes;  /* bytes needed for ws_lse: s_max*B*Lq*Hq floats */
  uint64_t ws_cnt_bytes;  /* bytes needed for ws_cnt (attn_decode): B*Hkv*row_tiles int32 */
  int64_t n_items;        /* (request, KV head, split) work items from kv_lens_host:
                             Hkv * max(1, s_b) summed over requests */
  /* attn_decode, GQA family: the keys of every (request, KV head) in rounds of
   * tile_n keys laid end to end (an empty one counts one round), split into
   * stream_grid equal runs, one per workgroup; a (request, KV head) is cut
   * into at most stream_pieces pieces. */
  int64_t stream_rounds;
  int32_t stream_grid;
  int32_t stream_pieces;
  uint64_t problem_key;   /* fingerprint of the planned problem */
} attn_plan;

/*
 * attn_decode_plan - choose the split count s and the keys per split.
 *
 * Decode has one query row per request, so one workgroup per (request, KV
 * head) leaves too few output tiles to fill the GPU; the reduction over keys
 * is split instead (Cleave §2.2 "Split-K"; §7.4 on when splitting pays).
 * Request b uses s_b = ceil(L_b / chunk) contiguous splits of chunk keys; the
 * last one may be short; splits past L_b do nothing.
 *
 * s_request    <= 0: the planner picks s from the total key count, the
 *              number of (request, KV head) units and num_cus.  > 0: use
 *              s_max = min(s_request, ceil(Lmax / tile_n)) with
 *              chunk = round_up(ceil(Lmax / s_max), tile_n).
 * kv_lens_host host copy of the B key counts used to size the split (values
 *              clamped to [0, Lcap]), or NULL for "all Lcap".  The device
 *              counts (problem->kv_lens or kv_indptr) of every call made with
 *              the plan must not exceed these: the split count, the chunk
 *              and (GQA family) the grid of work items cover exactly these
 *              lengths.  Where the device counts need more (a request longer
 *              than s_max * chunk keys, or more GQA work items than n_items),
 *              the affected output rows are written as NaN rather than a
 *              truncated result (all launched rows, in the second case), and
 *              ws_cnt is left as it was.
 * num_cus      compute units to plan for; <= 0 queries the current device.
 * out          receives the plan.
 * With a page table, the MFMA kernels stage one split's page ids on chip, so
 * the planner bounds a split to 8447 (GQA) or 4095 (MLA) pages, adding
 * splits where needed.  Decode takes no packed queries: a problem with
 * q_indptr gives ATTN_ERR_UNSUPPORTED here and in every decode call.
 * Returns ATTN_OK, ATTN_ERR_ARG, ATTN_ERR_UNSUPPORTED or ATTN_ERR_HIP (only
 * when num_cus <= 0 and the device query fails).  Enqueues nothing.
 */
int attn_decode_plan(const attn_problem* problem, int32_t s_request,
                     const int32_t* kv_lens_host, int32_t num_cus, attn_plan* out);

/*
 * attn_decode_split - the split kernel (Cleave §4, Fig. 5(b)).
 *
 * For every request b, KV head, row tile and split j < s_b, streams keys
 * [j*chunk, min((j+1)*chunk, L_b)) tile by tile with an online max and sum,
 * and writes the split's partial output, already divided by its own row sum,
 * and its log-sum-exp:
 *   ws_o  [s_max, B, Lq, Hq, Dv] float32   O_j = U_j / l_j
 *   ws_lse[s_max, B, Lq, Hq]     float32   LSE_j = m_j + ln l_j (natural log;
 *                                          -inf when the split sees no key)
 * Entries for splits j >= s_b are not written.  ws_o_bytes / ws_lse_bytes are
 * the sizes of the caller's buffers; smaller than the plan's gives
 * ATTN_ERR_WORKSPACE.  V may alias K (MLA).
 */
int attn_decode_split(const attn_problem* problem, const attn_plan* plan,
                      const void* q, const void* k, const void* v,
                      float* ws_o, size_t ws_o_bytes,
                      float* ws_lse, size_t ws_lse_bytes, void* stream);

/*
 * attn_decode - split decode in one call, in as few launches as the kernel
 * family allows.  The result equals attn_decode_split followed by
 * attn_combine (same O and LSE definitions).
 *
 * For the GQA D=128 and MLA families this is a single launch; the partials
 * it keeps in ws_o / ws_lse are private to it (their layout is not the one
 * attn_decode_split documents; an MLA request of at most four splits keeps
 * its partial outputs rounded to bf16, so the result then differs from the
 * two-launch one by that rounding, well inside the bf16 output tolerance).
 *   GQA with one split per request (s_max == 1): one workgroup per
 *   (request, KV head) writes O directly.  GQA with s_max > 1:
 *   the keys of all (request, KV head) units, in rounds of tile_n keys,
 *   are laid end to end and every workgroup of the plan's stream_grid takes
 *   an equal run of them (one long stream per compute unit, balanced
 *   whatever the request lengths; the split of Cleave §2.2 "Split-K" then
 *   falls where the runs end).  A unit inside one run is written directly;
 *   the pieces of a unit cut by run boundaries coordinate through an atomic
 *   counter in ws_cnt and the last one to finish merges them.
 *   MLA: the plan's s_max splits per request; the last split of each
 *   (request, KV head) to finish merges them.
 * Either way this is the combine of Cleave §4 without the second launch (the
 * cost the pages' §7.4 attributes to the two-launch design), summing the
 * pieces in order, so the result does not depend on which finishes last.
 *   Generic (vector-ALU) family: the plan's s_max splits per (request, KV
 *   head, row tile); the last one to finish merges them.
 * An MLA problem whose partials exceed 2 GiB (or whose pointers the MLA
 * kernel cannot take) runs the split launch and then the combine launch.
 *
 * ws_cnt  DEVICE int32 arrival counters, plan->ws_cnt_bytes of them (one per
 *         (request, KV head), times the row tiles for the generic family);
 *         it must be all zero
 *         before the first call; every call leaves it all zero again.  One
 *         workspace (ws_o, ws_lse, ws_cnt) serves one call at a time: calls
 *         that overlap on the same workspace race.
 * o, lse_out as for attn_combine.  Errors as for attn_decode_split.
 */
int attn_decode(const attn_problem* problem, const attn_plan* plan,
                const void* q, const void* k, const void* v,
                float* ws_o, size_t ws_o_bytes, float* ws_lse, size_t ws_lse_bytes,
                int32_t* ws_cnt, size_t ws_cnt_bytes, void* o, float* lse_out,
                void* stream);

/*
 * attn_decode_noalloc - attn_decode for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and results as attn_decode, with the
 * workspace in a device-resident array of the library instead of caller
 * buffers.  The caller still passes Q, K, V, O and (optionally) lse_out.
 *
 * The array is 96 MiB per GPU: 1 MiB of arrival counters (plan->ws_cnt_bytes
 * must fit) and 95 MiB for ws_lse and ws_o (each rounded up to 256 bytes).
 * A plan that needs more returns ATTN_ERR_WORKSPACE before anything is
 * enqueued (e.g. an MLA decode of 64 requests x 128 heads with s = 4 needs
 * 64 MiB and fits).  Each GPU the library runs on holds its own array until
 * the process ends; the first call on a GPU looks up its address and clears
 * its counters on `stream`.  No call allocates (no hipMalloc or allocating
 * library routine).  Every call on a GPU shares that GPU's array, so calls
 * that overlap on one GPU (on different streams or threads) race; calls in
 * one stream are ordered and safe.  Errors as for attn_decode.
 */
int attn_decode_noalloc(const attn_problem* problem, const attn_plan* plan,
                        const void* q, const void* k, const void* v, void* o,
                        float* lse_out, void* stream);

/*
 * attn_combine - the combine kernel (Cleave §4, Fig. 5(b)): reduces the
 * partials over the s_b splits of each row and divides.  With
 * M = max_j LSE_j and w_j = exp(LSE_j - M):
 *   O = sum_j w_j O_j / sum_j w_j,   LSE = M + ln sum_j w_j.
 * o       [B, Lq, Hq, Dv] with problem->o_stride, in problem->o_dtype.
 * lse_out optional float32 [B, Lq, Hq] contiguous (natural log), or NULL.
 * Rows with no visible key get O = 0 and LSE = -inf.
 */
int attn_combine(const attn_problem* problem, const attn_plan* plan,
                 const float* ws_o, const float* ws_lse, void* o, float* lse_out,
                 void* stream);

/*
 * attn_prefill - one fused launch, no split (Cleave §5.1: one workgroup per
 * output row tile, the key loop tiled inside with the row sum and the
 * V-matmul fused on the same exp tile; §7.4: splitting does not pay when the
 * grid is already full of query tiles).
 * o       [B, Lq, Hq, Dv] with problem->o_stride, in problem->o_dtype.
 * lse_out optional float32 [B, Lq, Hq] contiguous (natural log), or NULL.
 * bf16 with Dqk = Dv = 128 runs the MFMA kernel; other shapes run the
 * vector-ALU kernel; V aliasing K is accepted.
 */
int attn_prefill(const attn_problem* problem, const void* q, const void* k,
                 const void* v, void* o, float* lse_out, void* stream);

/* MatMul+MatMul: O[b, i, h, :] = sum over visible keys j of
 *   (tau * sum_d Q[b, i, h, d] K[b, j, h / G, d]) * V[b, j, h / G, :]
 * i.e. O = (tau Q K^T) V per (request, query head) with no softmax between the
 * two products (Cleave §7.3, Table 1: one of the two "consecutive reduction"
 * subgraphs, where iterative tiling and memory planning matter).  The
 * [Lq, L_b] intermediate exists one key tile at a time, in registers (§5.1 /
 * §5.3 iterative tiling), rounded to bf16 as the second product's operand.
 * Same problem description, layouts (strides, kv_lens, packed and paged K/V,
 * packed ragged queries) and causal rule as attn_prefill; a key that is not
 * visible contributes nothing, and a row with no visible key gives O = 0.
 * tau = problem->scale, or 1/sqrt(head_dim_qk) when scale <= 0.
 * Supported: bf16 Q/K/V with head_dim_qk = head_dim_v = 128 on the MFMA path
 * (the layouts attn_prefill's MFMA kernel accepts); anything else returns
 * ATTN_ERR_UNSUPPORTED before any launch.  o in problem->o_dtype.
 */
int attn_matmul_matmul(const attn_problem* problem, const void* q, const void* k,
                       const void* v, void* o, void* stream);

/* Static description of a status code; never NULL. */
const char* attn_status_str(int status);

/* Message for the calling thread's most recent failed call ("" if none). */
const char* attn_last_error(void);

/* ATTN_MI355X_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */

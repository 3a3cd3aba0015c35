// Host-side internals shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_mi355x.h"
#include "fastdiv.hpp"

namespace attn {

// Everything a kernel needs, passed by value.  Strides are in elements.
struct KParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;              // final output (prefill / combine)
  float* ws_o;          // split partials [s_max, B, Lq, Hq, Dv]
  float* ws_lse;        // split log-sum-exp [s_max, B, Lq, Hq]
  float* lse_out;       // optional [B, Lq, Hq]
  int32_t* counters;    // split arrivals per (request, KV head), zero between calls (mode 2)
  const int32_t* kv_lens;  // device, may be null
  // Variable-length and paged layouts (device, each may be null).
  const int32_t* q_indptr;    // [B + 1] packed query rows (prefill)
  const int32_t* kv_indptr;   // [B + 1] packed keys
  const int32_t* page_table;  // [B, ppr] page ids; ks_b / vs_b are then page strides
  int32_t page_size;          // rows per page
  int32_t ppr;                // page-table row length
  int32_t num_pages;          // page ids are clamped to [0, num_pages)
  int32_t page_shift;         // log2(page_size) when it is a power of two, else -1
  int64_t n_items;      // (request, KV head, split) work items of the 1-D decode grid;
                        // split_mode 3: 128-key rounds of all units laid end to end
  int32_t stream_grid;  // split_mode 3: workgroups, each taking an equal run of rounds
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int32_t B, Hq, Hkv, G, Dqk, Dv, Lq, Lcap;
  int32_t causal;
  int32_t in_bf16;      // Q/K/V element type
  int32_t o_bf16;       // O element type
  int32_t chunk;        // keys per split
  int32_t s_max;        // split slots
  int32_t rows;         // G * Lq rows per (request, KV head)
  int32_t row_tile;     // rows per workgroup (generic kernel)
  int32_t split_mode;   // 0: write o (+ lse_out); 1: write ws_o/ws_lse; 2: 1 + in-kernel merge;
                        // 3 (GQA): runs of rounds per workgroup, cut units merged in-kernel
  float scale_log2;     // tau * log2(e): scores are kept in base-2 units (tau itself when no_softmax)
  int32_t no_softmax;   // prefill only: 1 = MatMul+MatMul, O = (tau Q K^T) V
  FastDiv div_dqk, div_dv, div_g;  // divisions by Dqk, Dv and G (generic kernel)
  int32_t kv_vec;       // generic kernel: K/V rows load as 16-byte chunks (set at launch)
};

// RMSNorm followed by a MatMul: X [M, K], g [K], W [N, K], Y [M, N] (bf16
// inputs); row strides in elements.
struct RmsParams {
  const void* x;
  const void* g;
  const void* w;
  void* y;
  float* ws_u;          // split partials [s, M, N] (s > 1)
  float* ws_ssq;        // split sums of squares [s, M] (s > 1)
  int64_t x_row, w_row, y_row;
  int32_t M, K, N;
  int32_t s;            // K splits
  int32_t k_chunk;      // columns per split, a multiple of 32
  int32_t tile_n;       // weight rows per workgroup, a multiple of 4 in [4, 64]
  int32_t y_bf16;
  float eps;
};
hipError_t launch_rmsnorm_matmul(const RmsParams& p, hipStream_t s);

// SwiGLU: X [M, K], W_gate and W_up [N, K], H [M, N] (bf16 inputs); row
// strides in elements.
struct SwigluParams {
  const void* x;
  const void* wg;
  const void* wu;
  void* y;
  float* ws_g;          // gate partials [s, M, N] (s > 1)
  float* ws_u;          // up partials [s, M, N] (s > 1)
  int64_t x_row, wg_row, wu_row, y_row;
  int32_t M, K, N;
  int32_t s;            // K splits
  int32_t k_chunk;      // columns per split, a multiple of 32
  int32_t tile_n;       // output columns per workgroup, a multiple of 4 in [4, 64]
  int32_t y_bf16;
};
hipError_t launch_swiglu(const SwigluParams& p, hipStream_t s);

// Tiled bf16 GEMM of the prefill setting: A [M, K], B0 (and B1) [N, K], row
// strides in elements, K a multiple of 32.  mode 0: Y = row_scale[m] *
// (A B0^T)[m, n] (RMSNorm + MatMul, A = X * g); mode 1: Y = silu(A B0^T) *
// (A B1^T) (SwiGLU).
struct GemmParams {
  const void* a;
  const void* b0;
  const void* b1;
  void* y;
  const float* row_scale;
  int64_t a_row, b0_row, b1_row, y_row;
  int32_t M, N, K;   // K: columns of A (a multiple of kGemmKStep)
  int32_t y_bf16;
  int32_t mode;      // 0: Y = row_scale * (A B0^T); 1: Y = silu(A B0^T) * (A B1^T)
  int32_t b_shift;   // A step t (kGemmKStep columns) meets B step t >> b_shift
};
hipError_t launch_gemm_nt(const GemmParams& p, hipStream_t s);

// Prefill RMSNorm's first pass: X * g as bf16 pairs [M, 2K] (per 64-column
// step: the step's hi parts, then its lo parts) and row_scale [M].
struct RmsPrepParams {
  const void* x;
  const void* g;
  void* xg;
  float* row_scale;
  int64_t x_row, xg_row;
  int32_t M, K;
  float eps;
};
hipError_t launch_rms_prep(const RmsPrepParams& p, hipStream_t s);
constexpr int kGemmMinTokens = 256;   // token count from which the tiled GEMM is planned
constexpr int kGemmKStep = 64;        // the tiled GEMM's K step: k must be a multiple
// Largest row stride (elements) of a GEMM operand: a workgroup's 256 rows
// then span under 2^32 bytes, the reach of one buffer resource.
constexpr int64_t kGemmMaxStride = int64_t(1) << 22;

// Per-thread error reporting of the C ABI (attn_last_error): clear_error()
// at the start of an entry point, report_error(code, fmt, ...) on failure
// (returns code).
void clear_error();
int report_error(int code, const char* fmt, ...);

// Device-resident workspace of attn_decode_noalloc: arrival counters first,
// then the split partials.
constexpr uint64_t kScratchBytes = 96ull << 20;
constexpr uint64_t kScratchCntBytes = 1ull << 20;

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per (device, kernel); thread-safe.  Launchers call it before every launch.
hipError_t set_lds_limit_once(const void* kernel, int bytes);

// Launchers (one per kernel family).  Each returns a hipError_t.
hipError_t launch_generic(const KParams& p, dim3 grid, dim3 block, hipStream_t s);
hipError_t launch_combine(const KParams& p, hipStream_t s);
hipError_t launch_decode_gqa_d128(const KParams& p, hipStream_t s);  // 1-D item grid
hipError_t launch_decode_mla(const KParams& p, dim3 grid, hipStream_t s);
hipError_t launch_prefill_d128(const KParams& p, hipStream_t s);

// Tile geometry of the kernels, used by the planner.
constexpr int kGenericRowTile = 16;    // rows per generic workgroup
constexpr int kGenericTileN = 64;      // keys per generic tile
constexpr int kGenericBlock = 256;
constexpr int kGqaTileN = 128;         // keys per GQA-D128 workgroup round (4 waves x 32)
constexpr int kGqaItemsPerCu = 4;      // planner target: work items per compute unit
constexpr int kGqaStreamWgsPerCu = 2;  // attn_decode when units are cut: runs per compute unit
constexpr int kGqaMinChunk = 256;      // planner floor on keys per split
constexpr int kGqaBlock = 256;
constexpr int kGqaMaxRows = 16;
// Prefill K/V rings: contiguous caches take 64-key tiles (two 32-key blocks)
// in a 4-stage ring with a barrier per tile; paged pools 32-key tiles in a
// 6-stage ring with a barrier per two tiles (their per-lane copy moves one
// block per wave).
constexpr int kPrefillKeyBlocks = 2;      // contiguous: 32-key blocks per tile
constexpr int kPrefillStages = 4;         // contiguous: ring depth (tiles)
constexpr int kPrefillBarrierTiles = 1;   // contiguous: tiles per workgroup barrier
constexpr int kPrefillPagedStages = 6;    // paged: ring depth (32-key tiles)
constexpr int kPrefillPagedBarrierTiles = 2;  // paged: tiles per workgroup barrier
constexpr int kMlaTileN = 32;          // keys per MLA tile
constexpr int kMlaBlock = 512;         // 8 waves of 16 query rows
constexpr int kMlaRows = 128;          // query rows per MLA workgroup
constexpr int kGqaPageIds = 8448;      // page ids one paged GQA work item stages in LDS
constexpr int kPrefillPageIds = 4096;  // page ids one paged prefill workgroup stages in LDS
constexpr int kMlaPageIds = 4096;      // page ids one paged MLA split stages in LDS

}  // namespace attn

// Row addressing shared by the kernels: plain strided, packed (indptr) and
// paged layouts of Q, K, V and O, as the C ABI header defines them.
#pragma once

#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {

__device__ __forceinline__ int clamp_len(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

// Key count L_b of request b.
__device__ __forceinline__ int kv_len_b(const KParams& p, int b) {
  if (p.kv_indptr) return clamp_len(p.kv_indptr[b + 1] - p.kv_indptr[b], p.Lcap);
  return kv_len_of(p.kv_lens, b, p.Lcap);
}

// Query row count Lq_b of request b.
__device__ __forceinline__ int q_len_b(const KParams& p, int b) {
  if (p.q_indptr) return clamp_len(p.q_indptr[b + 1] - p.q_indptr[b], p.Lq);
  return p.Lq;
}

// Element offsets of query row i of request b (head 0) in Q and in O, and
// the row index of (b, i) in lse_out ([B, Lq, Hq] or, packed, [T, Hq]).
__device__ __forceinline__ int64_t q_row_off(const KParams& p, int b, int i) {
  if (p.q_indptr) return ((int64_t)p.q_indptr[b] + i) * p.qs_t;
  return (int64_t)b * p.qs_b + (int64_t)i * p.qs_t;
}
__device__ __forceinline__ int64_t o_row_off(const KParams& p, int b, int i) {
  if (p.q_indptr) return ((int64_t)p.q_indptr[b] + i) * p.os_t;
  return (int64_t)b * p.os_b + (int64_t)i * p.os_t;
}
__device__ __forceinline__ int64_t lse_row(const KParams& p, int b, int i) {
  if (p.q_indptr) return (int64_t)p.q_indptr[b] + i;
  return (int64_t)b * p.Lq + i;
}

// Page of key t of request b, clamped into the pool.
__device__ __forceinline__ int page_of(const KParams& p, int b, int t) {
  const int pg = p.page_table[(int64_t)b * p.ppr + t / p.page_size];
  return pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
}

// Element offset of key t of request b (head 0) in K or V, whose (batch or
// page, token) strides are s0 and s1.
__device__ __forceinline__ int64_t kv_row_off(const KParams& p, int b, int t, int64_t s0,
                                              int64_t s1) {
  if (p.page_table) return (int64_t)page_of(p, b, t) * s0 + (int64_t)(t % p.page_size) * s1;
  if (p.kv_indptr) return ((int64_t)p.kv_indptr[b] + t) * s1;
  return (int64_t)b * s0 + (int64_t)t * s1;
}

// Offset of request b's key 0 when its keys are contiguous rows (plain or
// packed layout, not paged).
__device__ __forceinline__ int64_t kv_base_off(const KParams& p, int b, int64_t s0, int64_t s1) {
  if (p.kv_indptr) return (int64_t)p.kv_indptr[b] * s1;
  return (int64_t)b * s0;
}

// Wave-uniform copies of a value every lane computed the same way (for a
// request index that is the same in every lane): they keep buffer
// descriptors and loop bounds in scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace attn

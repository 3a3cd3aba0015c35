// Vector-ALU attention kernel for any head dimension, f32 or bf16 inputs.
//
// It serves the fp32 problems (true fp32 end to end: fp32 products, fp32
// accumulation, 2^x on the transcendental unit) and every shape the MFMA
// kernels do not cover.  One workgroup computes one row tile of one
// (request, KV head) over one key range: the whole key axis (unsplit), or
// split j's keys [j*chunk, min((j+1)*chunk, L_b)) (Cleave §2.2 "Split-K").
// Keys are streamed in tiles of kGenericTileN; per tile the kernel forms the
// score tile, updates the running row max and row sum, and folds the exp tile
// into the output accumulator (the row sum and the V-matmul share the exp
// tile: Cleave §5.1, Listing 1 walk-through; the division comes last: §2.2).
#include "../attn_internal.hpp"
#include "common.hpp"
#include "layout.hpp"

namespace attn {
namespace {

constexpr int RT = kGenericRowTile;
constexpr int TN = kGenericTileN;
constexpr int NT = kGenericBlock;
constexpr int NB = 8;     // elements per thread and operand loaded before any is stored

__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  return (int)((__umulhi(f.m, (uint32_t)n) + (uint32_t)n) >> f.l);
}

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void* base, int64_t idx) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  } else {
    return reinterpret_cast<const float*>(base)[idx];
  }
}

// VE consecutive elements of a row (VE = 1, or 16 bytes: 4 fp32 / 8 bf16) as
// fp32; `idx` is a multiple of VE when VE > 1.
template <bool BF16, int VE>
__device__ __forceinline__ void ld_chunk(const void* base, int64_t idx, float* out) {
  if constexpr (VE == 1) {
    out[0] = ld_elem<BF16>(base, idx);
  } else if constexpr (BF16) {
    static_assert(VE == 8, "16-byte bf16 chunks");
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = bf16_bits_to_f32((uint16_t)(w[e] & 0xffff));
      out[2 * e + 1] = bf16_bits_to_f32((uint16_t)(w[e] >> 16));
    }
  } else {
    static_assert(VE == 4, "16-byte fp32 chunks");
    const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    out[0] = v.x;
    out[1] = v.y;
    out[2] = v.z;
    out[3] = v.w;
  }
}

// Copies a tile of nk rows of `wk` elements (row jj of `ka` at element offset
// rk(jj)) into LDS rows of stride `sk`, and likewise a tile of `wv`-element
// rows of `va` into rows of stride `sv`, in chunks of VE elements (16-byte
// loads when VE > 1: every row offset and width is then a multiple of VE).
// Thread t takes chunks t, t + NT, ... of each tile (consecutive threads,
// consecutive chunks: coalesced); each round issues NC loads of each tile
// before it stores any of them, so their latencies overlap instead of adding
// up.
template <bool BF16, int VE, class RowK, class RowV>
__device__ __forceinline__ void stage_kv(const void* ka, RowK rk, int wk, float* dk_s, int sk,
                                         const void* va, RowV rv, int wv, float* dv_s, int sv,
                                         int nk, int t) {
  constexpr int NC = VE == 1 ? NB : 16 / VE;  // chunks per round and tile
  const int nck = wk / VE, ncv = wv / VE;      // chunks per row
  const int djk = NT / nck, ddk = NT - djk * nck;
  const int djv = NT / ncv, ddv = NT - djv * ncv;
  int jk = t / nck, ck = t - jk * nck;
  int jv = t / ncv, cv = t - jv * ncv;
  while (jk < nk || jv < nk) {
    float xk[NC][VE], xv[NC][VE];
    int ok[NC], ov[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      // Past the tile: the first chunk of row 0 is read (it exists) and dropped.
      ok[u] = jk < nk ? jk * sk + ck * VE : -1;
      ld_chunk<BF16, VE>(ka, jk < nk ? rk(jk) + ck * VE : rk(0), xk[u]);
      ov[u] = jv < nk ? jv * sv + cv * VE : -1;
      ld_chunk<BF16, VE>(va, jv < nk ? rv(jv) + cv * VE : rv(0), xv[u]);
      jk += djk;
      ck += ddk;
      if (ck >= nck) {
        ck -= nck;
        ++jk;
      }
      jv += djv;
      cv += ddv;
      if (cv >= ncv) {
        cv -= ncv;
        ++jv;
      }
    }
#pragma unroll
    for (int u = 0; u < NC; ++u) {
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        if (ok[u] >= 0) dk_s[ok[u] + e] = xk[u][e];
        if (ov[u] >= 0) dv_s[ov[u] + e] = xv[u][e];
      }
    }
  }
}

// STAGE: each key tile's K and V rows are first copied into LDS by all
// threads (stage_kv), and the scores and the V-matmul read them from there;
// without it (head dims too large for the LDS) every thread reads its K and V
// elements from memory itself.  CP: output (row, d) pairs per thread, a power
// of two with RT * Dv <= NT * CP.
template <bool BF16, bool STAGE, int CP>
__global__ __launch_bounds__(NT) void generic_attn_kernel(KParams p) {
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  extern __shared__ float smem[];
  float* q_s = smem;                 // [RT][Dqk]
  float* s_s = q_s + RT * p.Dqk;     // [RT][TN]  scores, then exp tile
  float* m_s = s_s + RT * TN;        // [RT] running max (base-2 units)
  float* l_s = m_s + RT;             // [RT] running sum
  float* a_s = l_s + RT;             // [RT] rescale factor of this tile
  const int ks_row = p.Dqk + 1;      // staged K row stride: an odd number of words, so
                                     // the lanes' different keys fall in different banks
  float* k_s = a_s + RT;             // [TN][Dqk + 1] staged K rows (STAGE)
  float* v_s = k_s + TN * ks_row;    // [TN][Dv] staged V rows (STAGE)
  __shared__ int64_t row_k[TN], row_v[TN];  // element offsets of the tile's K and V rows

  const int t = threadIdx.x;
  const int j = blockIdx.x;
  const int rt = blockIdx.y;
  const int b = blockIdx.z / p.Hkv;
  const int kvh = blockIdx.z % p.Hkv;
  const int L = kv_len_b(p, b);
  const int Lqb = q_len_b(p, b);  // query rows of this request (packed queries: ragged)

  const int r0 = rt * RT;
  const int nrows = min(RT, p.G * Lqb - r0);
  if (nrows <= 0) return;  // row tile past this request's queries

  // Q tile (hoisted out of the key loop: Cleave §6.1, loop-invariant input);
  // NB loads per thread in flight before their stores, issued before the
  // key count is first used so that the two reads overlap.  The request's first
  // query row (an offset-array read when packed) is looked up once, so no
  // wait for it separates the loads.
  const int64_t q0 = q_row_off(p, b, 0);
  for (int e0 = t; e0 < RT * p.Dqk; e0 += NB * NT) {
    float qv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      // Every load is issued; one past the tile or its rows reads element 0
      // of row 0 (which exists) and is dropped, so no branch holds the
      // loads apart.
      const int e = e0 + u * NT;
      const bool ok = e < nrows * p.Dqk;  // rows past the tile's read as zero
      const int ec = ok ? e : 0;
      const int r = fdiv(ec, p.div_dqk), d = ec - r * p.Dqk;
      const int rr = r0 + r, i = fdiv(rr, p.div_g), h = kvh * p.G + rr - i * p.G;
      const float x = ld_elem<BF16>(p.q, q0 + (int64_t)i * p.qs_t + (int64_t)h * p.qs_h + d);
      qv[u] = ok ? x : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (e0 + u * NT < RT * p.Dqk) q_s[e0 + u * NT] = qv[u];
  }
  if (t < RT) {
    m_s[t] = kNegInf;
    l_s[t] = 0.f;
  }
  const int sb_all = (L + p.chunk - 1) / p.chunk;  // splits of this request
  if (p.split_mode == 2 && (L == 0 || sb_all > p.s_max)) {
    // Single launch: split 0 answers for a request with no key (O = 0, LSE =
    // -inf) and for one longer than the plan covers (NaN rather than a
    // truncated result); no split of such a request counts an arrival.
    if (j == 0) {
      const float val = L == 0 ? 0.f : __builtin_nanf("");
      const float lse = L == 0 ? kNegInf : __builtin_nanf("");
      for (int e = t; e < nrows * p.Dv; e += NT) {
        const int r = fdiv(e, p.div_dv), d = e - r * p.Dv;
        const int rr = r0 + r, i = fdiv(rr, p.div_g), h = kvh * p.G + rr - i * p.G;
        const int64_t oi = o_row_off(p, b, i) + (int64_t)h * p.os_h + d;
        if (p.o_bf16)
          reinterpret_cast<uint16_t*>(p.o)[oi] = (uint16_t)f32_to_bf16_bits(val);
        else
          reinterpret_cast<float*>(p.o)[oi] = val;
        if (d == 0 && p.lse_out) p.lse_out[lse_row(p, b, i) * p.Hq + h] = lse;
      }
    }
    return;
  }
  int lo = 0, hi = L;
  if (p.split_mode) {
    lo = j * p.chunk;
    if (lo >= L) return;  // split j does not exist for this request
    hi = min(lo + p.chunk, L);
  }

  // Causal: rows of this tile see keys j <= i + L - Lq; the tile needs keys
  // up to the largest such bound.
  if (p.causal) {
    const int i_last = fdiv(r0 + nrows - 1, p.div_g);
    hi = min(hi, i_last + L - Lqb + 1);
  }


  float acc[CP];
#pragma unroll
  for (int c = 0; c < CP; ++c) acc[c] = 0.f;
  const int npairs = RT * p.Dv;

  const int64_t khead = (int64_t)kvh * p.ks_h;
  const int64_t vhead = (int64_t)kvh * p.vs_h;
  // Contiguous (plain or packed) K/V: key 0 of this request and KV head.
  const int64_t kbase = p.page_table ? 0 : kv_base_off(p, b, p.ks_b, p.ks_t) + khead;
  const int64_t vbase = p.page_table ? 0 : kv_base_off(p, b, p.vs_b, p.vs_t) + vhead;
  __syncthreads();

  for (int k0 = lo; k0 < hi; k0 += TN) {
    const int nk = min(TN, hi - k0);  // keys of this tile that exist in the range
    if constexpr (STAGE) {
      // The previous tile's readers are past the barrier that ends its loop.
      // Paged: each key's row offsets once (a page-table read), through LDS;
      // contiguous layouts compute them where they are used.  16-byte
      // chunks when the layout allows (p.kv_vec), else single elements.
      if (p.page_table) {
        if (t < nk) {
          const int key = k0 + t;
          const int64_t pg = page_of(p, b, key), kr = key % p.page_size;
          row_k[t] = pg * p.ks_b + kr * p.ks_t + khead;
          row_v[t] = pg * p.vs_b + kr * p.vs_t + vhead;
        }
        __syncthreads();
        auto rk = [&](int jj) { return row_k[jj]; };
        auto rv = [&](int jj) { return row_v[jj]; };
        if (p.kv_vec)
          stage_kv<BF16, VEC>(p.k, rk, p.Dqk, k_s, ks_row, p.v, rv, p.Dv, v_s, p.Dv, nk, t);
        else
          stage_kv<BF16, 1>(p.k, rk, p.Dqk, k_s, ks_row, p.v, rv, p.Dv, v_s, p.Dv, nk, t);
      } else {
        const int64_t kb0 = kbase + (int64_t)k0 * p.ks_t, vb0 = vbase + (int64_t)k0 * p.vs_t;
        auto rk = [&](int jj) { return kb0 + (int64_t)jj * p.ks_t; };
        auto rv = [&](int jj) { return vb0 + (int64_t)jj * p.vs_t; };
        if (p.kv_vec)
          stage_kv<BF16, VEC>(p.k, rk, p.Dqk, k_s, ks_row, p.v, rv, p.Dv, v_s, p.Dv, nk, t);
        else
          stage_kv<BF16, 1>(p.k, rk, p.Dqk, k_s, ks_row, p.v, rv, p.Dv, v_s, p.Dv, nk, t);
      }
      __syncthreads();
    }
    // Scores: thread t -> key k0 + t % TN, rows 4*(t / TN) .. +3 (a wave
    // whose rows are all past the tile's rows skips the dot products).
    {
      const int jj = t % TN;
      const int rb = (t / TN) * 4;
      float dot[4] = {0.f, 0.f, 0.f, 0.f};
      if (jj < nk && rb < nrows) {
        if constexpr (STAGE) {
          const float* kr = k_s + jj * ks_row;
#pragma unroll 8
          for (int d = 0; d < p.Dqk; ++d) {
            const float kv = kr[d];
#pragma unroll
            for (int u = 0; u < 4; ++u) dot[u] = fmaf(q_s[(rb + u) * p.Dqk + d], kv, dot[u]);
          }
        } else {
          const int64_t krow = kv_row_off(p, b, k0 + jj, p.ks_b, p.ks_t) + khead;
          for (int d = 0; d < p.Dqk; ++d) {
            const float kv = ld_elem<BF16>(p.k, krow + d);
#pragma unroll
            for (int u = 0; u < 4; ++u) dot[u] = fmaf(q_s[(rb + u) * p.Dqk + d], kv, dot[u]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = rb + u;
        const int key = k0 + jj;
        bool vis = (jj < nk) && (r < nrows);
        if (vis && p.causal) {
          const int i = fdiv(r0 + r, p.div_g);
          vis = key <= i + L - Lqb;
        }
        s_s[r * TN + jj] = vis ? dot[u] * p.scale_log2 : kNegInf;
      }
    }
    __syncthreads();
    // Online softmax: 16 threads per row, 4 keys each; rows past the tile's
    // rows are never read.
    if (t / 16 < nrows) {
      const int r = t / 16;
      const int c0 = (t % 16) * 4;
      float sv[4];
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sv[u] = s_s[r * TN + c0 + u];
        mx = fmaxf(mx, sv[u]);
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
      const float m_old = m_s[r];
      const float m_new = fmaxf(m_old, mx);
      float alpha = 1.f, psum = 0.f;
      if (m_new != kNegInf) {
        alpha = fast_exp2(m_old - m_new);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float pv = fast_exp2(sv[u] - m_new);
          s_s[r * TN + c0 + u] = pv;
          psum += pv;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) s_s[r * TN + c0 + u] = 0.f;
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) psum += __shfl_xor(psum, o, 16);
      if ((t % 16) == 0) {
        l_s[r] = l_s[r] * alpha + psum;
        m_s[r] = m_new;
        a_s[r] = alpha;
      }
    }
    __syncthreads();
    // Output accumulator: thread t owns pairs e = t + NT*c -> (r = e / Dv, d = e % Dv).
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const int e = t + NT * c;
      if (e < nrows * p.Dv) {  // rows of the tile only
        const int r = fdiv(e, p.div_dv), d = e - r * p.Dv;
        float a = acc[c] * a_s[r];
        if constexpr (STAGE) {
          // Eight independent partial sums keep eight LDS reads in flight.
          float part[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          int jj = 0;
          for (; jj + 8 <= nk; jj += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
              part[u] = fmaf(s_s[r * TN + jj + u], v_s[(jj + u) * p.Dv + d], part[u]);
          }
          for (; jj < nk; ++jj) part[0] = fmaf(s_s[r * TN + jj], v_s[jj * p.Dv + d], part[0]);
          a += ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
        } else {
          for (int jj = 0; jj < nk; ++jj)
            a = fmaf(s_s[r * TN + jj],
                     ld_elem<BF16>(p.v, kv_row_off(p, b, k0 + jj, p.vs_b, p.vs_t) + vhead + d), a);
        }
        acc[c] = a;
      }
    }
    __syncthreads();
  }

  // Single launch with several splits: the splits of this (request, KV head,
  // row tile) take tickets (low 16 bits of its counter); all but the last
  // publish their partial and count it (high 16 bits); the last one, knowing
  // every other split is resident and has only its stores left, waits for
  // that count and merges the partials in split order (its own from
  // registers, computed exactly as a stored one), then resets the counter.
  // Partials use sc1 (device-coherent) stores and loads, each wave waiting
  // for its stores before the barrier that precedes the counting atomic, so
  // no partial is left dirty in, or read stale from, one XCD's L2.
  if (p.split_mode == 2 && sb_all > 1) {
    int* cnt = p.counters + ((int64_t)b * p.Hkv + kvh) * gridDim.y + rt;
    __shared__ int s_ticket;
    if (t == 0)
      s_ticket = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xffff;
    __syncthreads();
    const bool last = s_ticket == sb_all - 1;
    const int64_t nrow_all = (int64_t)p.B * p.Lq * p.Hq;
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const int e = t + NT * c;
      if (e < npairs) {
        const int r = fdiv(e, p.div_dv), d = e - r * p.Dv;
        if (r < nrows && !last) {
          const int rr = r0 + r, i = fdiv(rr, p.div_g), h = kvh * p.G + rr - i * p.G;
          const float l = l_s[r];
          const int64_t slot = (int64_t)j * nrow_all + ((int64_t)b * p.Lq + i) * p.Hq + h;
          store_dev(p.ws_o + slot * p.Dv + d, l > 0.f ? acc[c] / l : 0.f);
          if (d == 0) store_dev(p.ws_lse + slot, l > 0.f ? (m_s[r] + fast_log2(l)) * kLn2 : kNegInf);
        }
      }
    }
    if (!last) {
      wait_vmem();
      __syncthreads();
      if (t == 0) __hip_atomic_fetch_add(cnt, 1 << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (t == 0) {
      while ((__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 16) < sb_all - 1)
        __builtin_amdgcn_s_sleep(2);
    }
    __syncthreads();
    if (sb_all <= TN) {
      // Merge through a table in the (now free) score tile: tab[jj][r] holds
      // split jj's LSE of row r, then its weight 2^(LSE log2 e - M).  Every
      // partial is fetched in batches of NB loads (not one dependent load at
      // a time); the sums run in split order, as below.
      // Entry e = jj * RT + r; rows past the tile's are not loaded.
      float* tab = s_s;
      const int nent = sb_all * RT;
      for (int e0 = t; e0 < nent; e0 += NB * NT) {
        float lv[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int e = e0 + u * NT;
          const int jj = e / RT, r = e % RT;
          const bool ok = e < nent && r < nrows;
          const int rr = r0 + (ok ? r : 0), i = fdiv(rr, p.div_g), h = kvh * p.G + rr - i * p.G;
          const int64_t slot = (int64_t)(ok ? jj : 0) * nrow_all + ((int64_t)b * p.Lq + i) * p.Hq + h;
          const float x = load_dev(p.ws_lse + slot);  // split j's own slot is unused
          const float l = l_s[r];
          lv[u] = jj == j ? (l > 0.f ? (m_s[r] + fast_log2(l)) * kLn2 : kNegInf) : x;
        }
#pragma unroll
        for (int u = 0; u < NB; ++u)
          if (e0 + u * NT < nent) tab[e0 + u * NT] = lv[u];
      }
      __syncthreads();
      // Per row: M (base 2), the weights and their sum (a_s), M itself (m_s;
      // the row's own m and l are no longer needed but l_s is).
      if (t < nrows) {
        float M2 = kNegInf;
        for (int jj = 0; jj < sb_all; ++jj) M2 = fmaxf(M2, tab[jj * RT + t] * kLog2e);
        float den = 0.f;
        for (int jj = 0; jj < sb_all; ++jj) {
          const float wj = M2 == kNegInf ? 0.f : fast_exp2(tab[jj * RT + t] * kLog2e - M2);
          tab[jj * RT + t] = wj;
          den += wj;
        }
        a_s[t] = den;
        m_s[t] = M2;
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        const int e = t + NT * c;
        if (e < npairs) {
          const int r = fdiv(e, p.div_dv), d = e - r * p.Dv;
          if (r < nrows) {
            const int rr = r0 + r, i = fdiv(rr, p.div_g), h = kvh * p.G + rr - i * p.G;
            const int64_t row = ((int64_t)b * p.Lq + i) * p.Hq + h;
            const float l = l_s[r];
            const float o_own = l > 0.f ? acc[c] / l : 0.f;
            float num = 0.f;
            for (int jj0 = 0; jj0 < sb_all; jj0 += NB) {
              float ov[NB];
#pragma unroll
              for (int u = 0; u < NB; ++u) {
                const int jj = jj0 + u < sb_all ? jj0 + u : 0;
                ov[u] = load_dev(p.ws_o + ((int64_t)jj * nrow_all + row) * p.Dv + d);
              }
#pragma unroll
              for (int u = 0; u < NB; ++u) {
                const int jj = jj0 + u;
                if (jj < sb_all) num += tab[jj * RT + r] * (jj == j ? o_own : ov[u]);
              }
            }
            const float den = a_s[r], M2 = m_s[r];
            const float o = den > 0.f ? num / den : 0.f;
            const int64_t oi = o_row_off(p, b, i) + (int64_t)h * p.os_h + d;
            if (p.o_bf16)
              reinterpret_cast<uint16_t*>(p.o)[oi] = (uint16_t)f32_to_bf16_bits(o);
            else
              reinterpret_cast<float*>(p.o)[oi] = o;
            if (d == 0 && p.lse_out)
              p.lse_out[lse_row(p, b, i) * p.Hq + h] =
                  M2 == kNegInf ? kNegInf : (M2 + fast_log2(den)) * kLn2;
          }
        }
      }
      if (t == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const int e = t + NT * c;
      if (e < npairs) {
        const int r = fdiv(e, p.div_dv), d = e - r * p.Dv;
        if (r < nrows) {
          const int rr = r0 + r, i = fdiv(rr, p.div_g), h = kvh * p.G + rr - i * p.G;
          const int64_t row = ((int64_t)b * p.Lq + i) * p.Hq + h;
          const float l = l_s[r];
          const float o_own = l > 0.f ? acc[c] / l : 0.f;
          const float lse_own = l > 0.f ? (m_s[r] + fast_log2(l)) * kLn2 : kNegInf;
          float M2 = kNegInf;
          for (int jj = 0; jj < sb_all; ++jj) {
            const float lj = jj == j ? lse_own : load_dev(p.ws_lse + (int64_t)jj * nrow_all + row);
            M2 = fmaxf(M2, lj * kLog2e);
          }
          float num = 0.f, den = 0.f;
          if (M2 != kNegInf) {
            for (int jj = 0; jj < sb_all; ++jj) {
              const int64_t slot = (int64_t)jj * nrow_all + row;
              const float lj = jj == j ? lse_own : load_dev(p.ws_lse + slot);
              const float oj = jj == j ? o_own : load_dev(p.ws_o + slot * p.Dv + d);
              const float wj = fast_exp2(lj * kLog2e - M2);
              num += wj * oj;
              den += wj;
            }
          }
          const float o = den > 0.f ? num / den : 0.f;
          const int64_t oi = o_row_off(p, b, i) + (int64_t)h * p.os_h + d;
          if (p.o_bf16)
            reinterpret_cast<uint16_t*>(p.o)[oi] = (uint16_t)f32_to_bf16_bits(o);
          else
            reinterpret_cast<float*>(p.o)[oi] = o;
          if (d == 0 && p.lse_out)
            p.lse_out[lse_row(p, b, i) * p.Hq + h] =
                M2 == kNegInf ? kNegInf : (M2 + fast_log2(den)) * kLn2;
        }
      }
    }
    if (t == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // Epilogue: divide by the row sum after the V-matmul (Cleave §2.2, Fig. 2).
#pragma unroll
  for (int c = 0; c < CP; ++c) {
    const int e = t + NT * c;
    if (e < npairs) {
      const int r = fdiv(e, p.div_dv), d = e - r * p.Dv;
      if (r < nrows) {
        const int rr = r0 + r, i = fdiv(rr, p.div_g), h = kvh * p.G + rr - i * p.G;
        const float l = l_s[r];
        const float o = l > 0.f ? acc[c] / l : 0.f;
        const float lse = l > 0.f ? (m_s[r] + fast_log2(l)) * kLn2 : kNegInf;
        if (p.split_mode == 1) {
          const int64_t row = ((int64_t)b * p.Lq + i) * p.Hq + h;
          const int64_t slot = (int64_t)j * p.B * p.Lq * p.Hq + row;
          p.ws_o[slot * p.Dv + d] = o;
          if (d == 0) p.ws_lse[slot] = lse;
        } else {
          const int64_t oi = o_row_off(p, b, i) + (int64_t)h * p.os_h + d;
          if (p.o_bf16)
            reinterpret_cast<uint16_t*>(p.o)[oi] = (uint16_t)f32_to_bf16_bits(o);
          else
            reinterpret_cast<float*>(p.o)[oi] = o;
          if (d == 0 && p.lse_out) p.lse_out[lse_row(p, b, i) * p.Hq + h] = lse;
        }
      }
    }
  }
}

template <bool BF16, bool STAGE, int CP>
hipError_t launch_generic_variant(const KParams& p, dim3 grid, dim3 block, size_t shmem, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&generic_attn_kernel<BF16, STAGE, CP>);
  if (STAGE)
    if (hipError_t e = set_lds_limit_once(fn, (int)shmem)) return e;
  hipLaunchKernelGGL((generic_attn_kernel<BF16, STAGE, CP>), grid, block, shmem, s, p);
  return hipGetLastError();
}

template <bool BF16, bool STAGE>
hipError_t launch_generic_cp(const KParams& p, dim3 grid, dim3 block, size_t shmem, hipStream_t s) {
  const int pairs = RT * p.Dv;  // output (row, d) pairs of a workgroup
  if (pairs <= NT * 4) return launch_generic_variant<BF16, STAGE, 4>(p, grid, block, shmem, s);
  if (pairs <= NT * 8) return launch_generic_variant<BF16, STAGE, 8>(p, grid, block, shmem, s);
  if (pairs <= NT * 16) return launch_generic_variant<BF16, STAGE, 16>(p, grid, block, shmem, s);
  return launch_generic_variant<BF16, STAGE, 32>(p, grid, block, shmem, s);
}

}  // namespace

hipError_t launch_generic(const KParams& kp, dim3 grid, dim3 block, hipStream_t s) {
  if (RT * kp.Dv > NT * 32) return hipErrorInvalidValue;  // Dv <= 512
  // K/V staging in 16-byte chunks when every row offset and row width is a
  // whole number of chunks and the base pointers are 16-byte aligned.
  KParams p = kp;
  const int64_t ve = p.in_bf16 ? 8 : 4;
  const auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
  p.kv_vec = al16(p.k) && al16(p.v) && p.Dqk % ve == 0 && p.Dv % ve == 0 && p.ks_b % ve == 0 &&
             p.ks_t % ve == 0 && p.ks_h % ve == 0 && p.vs_b % ve == 0 && p.vs_t % ve == 0 &&
             p.vs_h % ve == 0;
  const size_t base = sizeof(float) * ((size_t)RT * p.Dqk + RT * TN + 3 * RT);
  // Stage K/V tiles when they fit in 64 KiB (head dims Dqk + Dv < 256).
  const size_t tiles = sizeof(float) * (size_t)TN * (p.Dqk + 1 + p.Dv);
  const bool stage = tiles <= (64u << 10);
  const size_t shmem = base + (stage ? tiles : 0);
  if (p.in_bf16)
    return stage ? launch_generic_cp<true, true>(p, grid, block, shmem, s)
                 : launch_generic_cp<true, false>(p, grid, block, shmem, s);
  return stage ? launch_generic_cp<false, true>(p, grid, block, shmem, s)
               : launch_generic_cp<false, false>(p, grid, block, shmem, s);
}

}  // namespace attn

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
constexpr int MAXC = 32;  // output (row, d) pairs per thread: RT * Dv <= NT * MAXC, Dv <= 512

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void* base, int64_t idx) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  } else {
    return reinterpret_cast<const float*>(base)[idx];
  }
}

template <bool BF16>
__global__ __launch_bounds__(NT) void generic_attn_kernel(KParams p) {
  extern __shared__ float smem[];
  float* q_s = smem;                 // [RT][Dqk]
  float* s_s = q_s + RT * p.Dqk;     // [RT][TN]  scores, then exp tile
  float* m_s = s_s + RT * TN;        // [RT] running max (base-2 units)
  float* l_s = m_s + RT;             // [RT] running sum
  float* a_s = l_s + RT;             // [RT] rescale factor of this tile

  const int t = threadIdx.x;
  const int j = blockIdx.x;
  const int rt = blockIdx.y;
  const int b = blockIdx.z / p.Hkv;
  const int kvh = blockIdx.z % p.Hkv;
  const int L = kv_len_b(p, b);
  const int Lqb = q_len_b(p, b);  // query rows of this request (packed queries: ragged)

  int lo = 0, hi = L;
  if (p.split_mode) {
    lo = j * p.chunk;
    if (lo >= L) return;  // split j does not exist for this request
    hi = min(lo + p.chunk, L);
  }
  const int r0 = rt * RT;
  const int nrows = min(RT, p.G * Lqb - r0);
  if (nrows <= 0) return;  // row tile past this request's queries

  // Causal: rows of this tile see keys j <= i + L - Lq; the tile needs keys
  // up to the largest such bound.
  if (p.causal) {
    const int i_last = (r0 + nrows - 1) / p.G;
    hi = min(hi, i_last + L - Lqb + 1);
  }

  // Q tile (hoisted out of the key loop: Cleave §6.1, loop-invariant input).
  for (int e = t; e < RT * p.Dqk; e += NT) {
    const int r = e / p.Dqk, d = e % p.Dqk;
    float val = 0.f;
    if (r < nrows) {
      const int rr = r0 + r, i = rr / p.G, h = kvh * p.G + rr % p.G;
      val = ld_elem<BF16>(p.q, q_row_off(p, b, i) + (int64_t)h * p.qs_h + d);
    }
    q_s[e] = val;
  }
  if (t < RT) {
    m_s[t] = kNegInf;
    l_s[t] = 0.f;
  }

  float acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = 0.f;
  const int npairs = RT * p.Dv;

  const int64_t khead = (int64_t)kvh * p.ks_h;
  const int64_t vhead = (int64_t)kvh * p.vs_h;
  __syncthreads();

  for (int k0 = lo; k0 < hi; k0 += TN) {
    const int nk = min(TN, hi - k0);  // keys of this tile that exist in the range
    // Scores: thread t -> key k0 + t % TN, rows 4*(t / TN) .. +3.
    {
      const int jj = t % TN;
      const int rb = (t / TN) * 4;
      float dot[4] = {0.f, 0.f, 0.f, 0.f};
      if (jj < nk) {
        const int64_t krow = kv_row_off(p, b, k0 + jj, p.ks_b, p.ks_t) + khead;
        for (int d = 0; d < p.Dqk; ++d) {
          const float kv = ld_elem<BF16>(p.k, krow + d);
#pragma unroll
          for (int u = 0; u < 4; ++u) dot[u] = fmaf(q_s[(rb + u) * p.Dqk + d], kv, dot[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = rb + u;
        const int key = k0 + jj;
        bool vis = (jj < nk) && (r < nrows);
        if (vis && p.causal) {
          const int i = (r0 + r) / p.G;
          vis = key <= i + L - Lqb;
        }
        s_s[r * TN + jj] = vis ? dot[u] * p.scale_log2 : kNegInf;
      }
    }
    __syncthreads();
    // Online softmax: 16 threads per row, 4 keys each.
    {
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
    for (int c = 0; c < MAXC; ++c) {
      const int e = t + NT * c;
      if (e < npairs) {
        const int r = e / p.Dv, d = e % p.Dv;
        float a = acc[c] * a_s[r];
        for (int jj = 0; jj < nk; ++jj)
          a = fmaf(s_s[r * TN + jj],
                   ld_elem<BF16>(p.v, kv_row_off(p, b, k0 + jj, p.vs_b, p.vs_t) + vhead + d), a);
        acc[c] = a;
      }
    }
    __syncthreads();
  }

  // Epilogue: divide by the row sum after the V-matmul (Cleave §2.2, Fig. 2).
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = t + NT * c;
    if (e < npairs) {
      const int r = e / p.Dv, d = e % p.Dv;
      if (r < nrows) {
        const int rr = r0 + r, i = rr / p.G, h = kvh * p.G + rr % p.G;
        const float l = l_s[r];
        const float o = l > 0.f ? acc[c] / l : 0.f;
        const float lse = l > 0.f ? (m_s[r] + fast_log2(l)) * kLn2 : kNegInf;
        if (p.split_mode) {
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

}  // namespace

hipError_t launch_generic(const KParams& p, dim3 grid, dim3 block, hipStream_t s) {
  const size_t shmem = sizeof(float) * ((size_t)RT * p.Dqk + RT * TN + 3 * RT);
  if (p.in_bf16)
    hipLaunchKernelGGL(generic_attn_kernel<true>, grid, block, shmem, s, p);
  else
    hipLaunchKernelGGL(generic_attn_kernel<false>, grid, block, shmem, s, p);
  return hipGetLastError();
}

}  // namespace attn

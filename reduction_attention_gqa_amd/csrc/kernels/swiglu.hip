// SwiGLU, H = silu(X W_gate^T) * (X W_up^T): two MatMuls that reduce over K
// and read the same X, fused horizontally (Cleave §7.3), so every X fragment
// feeds both reductions in the same loop and each weight matrix is streamed
// once.  With few output tiles (decode: a
// few tokens) the K axis is split (Cleave §2.2 "Split-K"); the gate is
// nonlinear, so the parts of both MatMuls are added up (combine kernel)
// before silu is applied.
//
// Layout: X [M, K], W_gate and W_up [N, K] (linear-layer weights), H [M, N],
// row strides in elements, bf16 inputs.  A workgroup is four waves and owns
// up to 64 output columns (the planner narrows the tile, in steps of 4, so
// that the tiles fill the compute units) and up to 32 tokens on the MFMA
// columns; waves 2c and
// 2c + 1 share columns 32c .. 32c + 31 (two 16-row blocks of each weight
// matrix, the same rows in both) and take alternate super-steps of the part's
// K range (a second, on-chip level of the same split-K; alternating, rather
// than a half each, keeps the pair's reads of a weight row contiguous:
// 6 % faster):
//   G^T[16 x 16] += W_gate[16 x 32] X^T[32 x 16],  U^T likewise   16x16x32 MFMA
// The weights move a super-step (two 32-column k-steps, 128 contiguous
// bytes per row: one line) ahead of use, double-buffered; X (a few KB, through the
// caches) is issued first so in-order completion never holds it behind W.
// The two halves are added through LDS and each wave of the pair finishes
// one row block: with the whole K range in one part (s = 1) it applies the
// gate and writes H, so one launch does everything; otherwise it writes the
// part's sums for the combine kernel.
#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {
namespace {

constexpr int NW = 4;       // waves per workgroup
constexpr int NRB = 2;      // 16-row blocks per wave and weight matrix
constexpr int COLS = NW / 2 * NRB * 16;  // output columns per workgroup (64)
static_assert(NW == 4 && NRB == 2, "a wave pair covers one column group; each wave finishes one block");
constexpr int SS = 2;       // k-steps per super-step
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every range: loads read zero

struct WBuf {
  i32x4_t g[SS][NRB];
  i32x4_t u[SS][NRB];
};
struct XBuf {
  i32x4_t x[SS][2];
};

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// H[m, n .. n + 3] (columns past N are skipped), bf16 (round to nearest even)
// or fp32.
__device__ __forceinline__ void store_h4(const SwigluParams& p, int m, int n, const f32x4_t& v) {
  if (p.y_bf16) {
    uint16_t* yp = reinterpret_cast<uint16_t*>(p.y) + (int64_t)m * p.y_row + n;
    if (n + 3 < p.N && (reinterpret_cast<uintptr_t>(yp) & 7) == 0) {
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(yp) = pk;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < p.N) yp[i] = (uint16_t)f32_to_bf16_bits(v[i]);
    }
  } else {
    float* yp = reinterpret_cast<float*>(p.y) + (int64_t)m * p.y_row + n;
    if (n + 3 < p.N && (reinterpret_cast<uintptr_t>(yp) & 15) == 0) {
      *reinterpret_cast<f32x4_t*>(yp) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < p.N) yp[i] = v[i];
    }
  }
}

__device__ __forceinline__ void store_part4(float* base, const SwigluParams& p, int m, int n,
                                            const f32x4_t& v) {
  float* dst = base + (int64_t)m * p.N + n;
  if (n + 3 < p.N && (p.N & 3) == 0) {
    *reinterpret_cast<f32x4_t*>(dst) = v;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n + i < p.N) dst[i] = v[i];
  }
}

__global__ __launch_bounds__(NW * 64) void swiglu_split_kernel(SwigluParams p) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;   // MFMA row (weight row) / column (token) index
  const int kg = lane >> 4;  // 8-column group of a 32-column k-step
  const int n_wg = blockIdx.x * p.tile_n;  // tile_n <= COLS, a multiple of 4
  const int j = blockIdx.y;
  const int m0 = blockIdx.z * 32;
  // This wave's super-steps of the part's columns: every other one, from
  // the (w & 1)-th on.
  const int lo_j = j * p.k_chunk;
  const int hi_j = min(lo_j + p.k_chunk, p.K);
  const int lo = lo_j + (w & 1) * 32 * SS;
  const int hi = hi_j;

  // Buffer ranges end at the tile's last valid weight row and token, so rows
  // past the tile, N or M read as zero without a memory access.  Offsets stay
  // 32-bit: a workgroup's 64 rows, 32 tokens.
  const int wrows = min(p.tile_n, p.N - n_wg);
  const int xrows = min(32, p.M - m0);
  const uint16_t* gp = reinterpret_cast<const uint16_t*>(p.wg) + (int64_t)n_wg * p.wg_row;
  const uint16_t* up = reinterpret_cast<const uint16_t*>(p.wu) + (int64_t)n_wg * p.wu_row;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(p.x) + (int64_t)m0 * p.x_row;
  const uint32_t gst = (uint32_t)(p.wg_row * 2), ust = (uint32_t)(p.wu_row * 2);
  const uint32_t xst = (uint32_t)(p.x_row * 2);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(gp, (uint32_t)wrows * gst);
  const __amdgpu_buffer_rsrc_t urs = make_rsrc(up, (uint32_t)wrows * ust);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xp, (uint32_t)xrows * xst);
  const int row0 = NRB * 16 * (w >> 1) + r;  // this lane's first weight row in the workgroup
  const uint32_t x_lane0 = (uint32_t)r * xst + 16u * kg;
  const uint32_t x_lane1 = (uint32_t)(16 + r) * xst + 16u * kg;

  // Columns past the split or past K read as zero without a memory access.
  auto oob_of = [&](int k) -> uint32_t { return (k < hi && k + 8 * kg < p.K) ? 0u : kOob; };
  auto load_w = [&](WBuf& b, int k0) {
#pragma unroll
    for (int blk = 0; blk < NRB; ++blk)
#pragma unroll
      for (int t = 0; t < SS; ++t) {
        const int k = k0 + 32 * t;
        const uint32_t kb = (uint32_t)k * 2 + 16u * kg, oob = oob_of(k);
        b.g[t][blk] = buf_load16(grs, ((uint32_t)(row0 + 16 * blk) * gst + kb) | oob);
        b.u[t][blk] = buf_load16(urs, ((uint32_t)(row0 + 16 * blk) * ust + kb) | oob);
      }
  };
  auto load_x = [&](XBuf& b, int k0) {
#pragma unroll
    for (int t = 0; t < SS; ++t) {
      const int k = k0 + 32 * t;
      const uint32_t oob = oob_of(k), kb = (uint32_t)k * 2;
      b.x[t][0] = buf_load16(xrs, (x_lane0 + kb) | oob);
      b.x[t][1] = buf_load16(xrs, (x_lane1 + kb) | oob);
    }
  };

  f32x4_t acc_g[NRB][2], acc_u[NRB][2];
#pragma unroll
  for (int b = 0; b < NRB; ++b)
#pragma unroll
    for (int mg = 0; mg < 2; ++mg) acc_g[b][mg] = acc_u[b][mg] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Double-buffered super-steps; scheduling barriers keep the issue order
  // (each super-step's X first, then the next super-step's weights).  STEP:
  // from one of this wave's super-steps to its next.
  constexpr int STEP = 32 * SS * 2;
  WBuf wb[2];
  XBuf xb;
  load_w(wb[0], lo);
  __builtin_amdgcn_sched_barrier(0);
  for (int k0 = lo; k0 < hi; k0 += 2 * STEP) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kc = k0 + u * STEP;
      if (u == 1 && kc >= hi) break;
      load_x(xb, kc);
      __builtin_amdgcn_sched_barrier(0);
      load_w(wb[u ^ 1], kc + STEP);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < SS; ++t) {
        if (kc + 32 * t >= hi) continue;
#pragma unroll
        for (int mg = 0; mg < 2; ++mg) {
          const bf16x8_t xv = as_bf16x8(xb.x[t][mg]);
#pragma unroll
          for (int b = 0; b < NRB; ++b) {
            acc_g[b][mg] = mfma16x16x32(as_bf16x8(wb[u].g[t][b]), xv, acc_g[b][mg]);
            acc_u[b][mg] = mfma16x16x32(as_bf16x8(wb[u].u[t][b]), xv, acc_u[b][mg]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Add the pair's halves: lane holds G^T / U^T[weight row 16 b + 4 kg + i]
  // [token r] of each token group; wave w keeps row block w & 1 of its pair.
  __shared__ f32x4_t red[NW][2][NRB][2][64];  // [wave][gate, up][block][token group][lane]: 32 KiB
#pragma unroll
  for (int b = 0; b < NRB; ++b)
#pragma unroll
    for (int mg = 0; mg < 2; ++mg) {
      red[w][0][b][mg][lane] = acc_g[b][mg];
      red[w][1][b][mg][lane] = acc_u[b][mg];
    }
  __syncthreads();
  const int blk = w & 1, w0 = w & ~1;
  const int n_lane = n_wg + NRB * 16 * (w >> 1) + 16 * blk + 4 * kg;
#pragma unroll
  for (int mg = 0; mg < 2; ++mg) {
    const int m = m0 + 16 * mg + r;
    if (m >= p.M || n_lane - n_wg >= wrows) continue;  // columns past the tile: the next one's
    const f32x4_t g = red[w0][0][blk][mg][lane] + red[w0 + 1][0][blk][mg][lane];
    const f32x4_t u = red[w0][1][blk][mg][lane] + red[w0 + 1][1][blk][mg][lane];
    if (p.s == 1) {
      f32x4_t h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = silu(g[i]) * u[i];
      store_h4(p, m, n_lane, h);
    } else {
      const int64_t part = (int64_t)j * p.M * p.N;
      store_part4(p.ws_g + part, p, m, n_lane, g);
      store_part4(p.ws_u + part, p, m, n_lane, u);
    }
  }
}

// Combine: H[m, n] = silu(sum_j G_j[m, n]) * sum_j U_j[m, n]; thread t handles
// four consecutive n of one row.
__global__ __launch_bounds__(256) void swiglu_combine_kernel(SwigluParams p) {
  const int64_t quads = (int64_t)(p.N + 3) / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= quads * p.M) return;
  const int m = (int)(t / quads);
  const int n = (int)(t - (int64_t)m * quads) * 4;
  f32x4_t g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < p.s; ++j) {
    const int64_t off = ((int64_t)j * p.M + m) * p.N + n;
    if (n + 3 < p.N && (p.N & 3) == 0) {
      g += *reinterpret_cast<const f32x4_t*>(p.ws_g + off);
      u += *reinterpret_cast<const f32x4_t*>(p.ws_u + off);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < p.N) {
          g[i] += p.ws_g[off + i];
          u[i] += p.ws_u[off + i];
        }
    }
  }
  f32x4_t h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = silu(g[i]) * u[i];
  store_h4(p, m, n, h);
}

}  // namespace

hipError_t launch_swiglu(const SwigluParams& p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.N + p.tile_n - 1) / p.tile_n), (unsigned)p.s,
                  (unsigned)((p.M + 31) / 32));
  hipLaunchKernelGGL(swiglu_split_kernel, grid, dim3(NW * 64), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.s == 1) return e;
  const int64_t threads = (int64_t)p.M * ((p.N + 3) / 4);
  hipLaunchKernelGGL(swiglu_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace attn

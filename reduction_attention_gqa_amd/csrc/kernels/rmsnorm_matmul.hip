// RMSNorm followed by a MatMul, Y = RMSNorm(X) W^T, in the rewritten form of
// the Cleave paper (§1, Fig. 1): RMSNorm's row scale is moved after the
// Matmul, so the Matmul runs on the raw input and the rows' sums of squares
// are accumulated from the same X tiles in the same loop (the two reductions
// fused horizontally); the scale 1 / sqrt(mean(x^2) + eps) is applied to the
// finished dot products and the normalised input never exists.  With few
// output tiles (decode: a few tokens) the K axis is split (Cleave §2.2
// "Split-K"): each split writes its partial dot products and sums of squares,
// and a combine kernel adds them up and applies the row scale.
//
// Layout: X [M, K], g [K], W [N, K] (linear-layer weights), Y [M, N], row
// strides in elements, bf16 inputs.  A workgroup is four waves that share the
// workgroup's tile of up to 64 weight rows (four MFMA row blocks; the planner
// narrows the tile, in steps of 4 rows, so that the tiles fill the compute
// units: 56 rows for N = 14336 on 256 of them) and up to 32 tokens (two MFMA
// column groups) and split the part's K range four ways, wave w taking the
// w-th quarter (a second, on-chip level of the same split-K):
//   U^T[16 x 16] += W[16 x 32] (X * g)^T[32 x 16]     16x16x32 bf16 MFMA
// W streams from HBM straight into the A operand (16 bytes per lane and row
// block, four k-steps in flight); X and g come through the caches (a few KB,
// shared by all workgroups) and each fragment serves the wave's four row
// blocks.  x * g is exact in fp32 (two 8-bit significands); it enters the
// MFMA as a bf16 pair hi + lo, so the gain costs no precision.  The four
// waves' partial dot products and sums of squares are added through LDS, and
// wave w finishes row block w: with the whole K range in one part (s = 1) it
// applies the row scale and writes Y, so one launch does everything;
// otherwise it writes the part's sums for the combine kernel.
#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {
namespace {

constexpr int NW = 4;      // waves per workgroup
constexpr int NRB = 4;     // 16-row weight blocks per wave
constexpr int ROWS = NRB * 16;  // weight rows per workgroup (shared by its waves)
static_assert(NRB == NW, "wave w finishes row block w");
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every range: loads read zero

// One super-step: SS consecutive 32-column k-steps.  Its W loads for one
// weight row cover SS * 64 contiguous bytes, one 128-byte line, and are
// issued back to back, so the memory sees whole lines rather than 64-byte
// pieces spread over time.  (Two-line super-steps, or two super-steps in
// flight, measured 7 % slower: more rows in flight at once cost more than
// the deeper queue gains.)
constexpr int SS = 2;
struct WBuf {
  i32x4_t w[SS][NRB];
};
struct XBuf {
  i32x4_t x[SS][2];
  i32x4_t g[SS];
};

// Y[m, n .. n + 3] (columns past N are skipped), bf16 (round to nearest
// even) or fp32; one vector store when the address allows.
__device__ __forceinline__ void store_row4(const RmsParams& p, int m, int n, const f32x4_t& v) {
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

__global__ __launch_bounds__(NW * 64) void rmsnorm_matmul_split_kernel(RmsParams p) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;   // MFMA row (weight row) / column (token) index
  const int kg = lane >> 4;  // 8-column group of a 32-column k-step
  const int n_wg = blockIdx.x * p.tile_n;  // tile_n <= ROWS, a multiple of 4
  const int j = blockIdx.y;
  const int m0 = blockIdx.z * 32;
  // This wave's quarter of the part's columns (a multiple of 32 wide).
  const int lo_j = j * p.k_chunk;
  const int hi_j = min(lo_j + p.k_chunk, p.K);
  const int kcw = (p.k_chunk + 32 * NW - 1) / (32 * NW) * 32;
  const int lo = min(lo_j + w * kcw, hi_j);
  const int hi = min(lo + kcw, hi_j);

  // Buffer ranges end at the tile's last valid weight row and token, so rows
  // past the tile, N or M read as zero without a memory access.  Offsets stay
  // 32-bit: a workgroup's 64 rows, 32 tokens.
  const int wrows = min(p.tile_n, p.N - n_wg);
  const int xrows = min(32, p.M - m0);
  const uint16_t* wp = reinterpret_cast<const uint16_t*>(p.w) + (int64_t)n_wg * p.w_row;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(p.x) + (int64_t)m0 * p.x_row;
  const uint32_t wst = (uint32_t)(p.w_row * 2), xst = (uint32_t)(p.x_row * 2);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wp, (uint32_t)wrows * wst);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xp, (uint32_t)xrows * xst);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(p.g, (uint32_t)p.K * 2);
  const uint32_t w_lane = (uint32_t)r * wst + 16u * kg;
  const uint32_t x_lane0 = (uint32_t)r * xst + 16u * kg;
  const uint32_t x_lane1 = (uint32_t)(16 + r) * xst + 16u * kg;

  // k-step at column k: this lane's 8 columns k + 8 kg .. + 7; columns past
  // the split or past K read as zero without a memory access.
  auto oob_of = [&](int k) -> uint32_t { return (k < hi && k + 8 * kg < p.K) ? 0u : kOob; };
  auto load_w = [&](WBuf& b, int k0) {
#pragma unroll
    for (int blk = 0; blk < NRB; ++blk)
#pragma unroll
      for (int t = 0; t < SS; ++t) {
        const int k = k0 + 32 * t;
        b.w[t][blk] = buf_load16(
            wrs, (w_lane + (uint32_t)(16 * blk) * wst + (uint32_t)k * 2) | oob_of(k));
      }
  };
  auto load_x = [&](XBuf& b, int k0) {
#pragma unroll
    for (int t = 0; t < SS; ++t) {
      const int k = k0 + 32 * t;
      const uint32_t oob = oob_of(k), kb = (uint32_t)k * 2;
      b.g[t] = buf_load16(grs, (16u * kg + kb) | oob);
      b.x[t][0] = buf_load16(xrs, (x_lane0 + kb) | oob);
      b.x[t][1] = buf_load16(xrs, (x_lane1 + kb) | oob);
    }
  };

  f32x4_t acc[NRB][2];
#pragma unroll
  for (int b = 0; b < NRB; ++b) acc[b][0] = acc[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float ssq[2] = {0.f, 0.f};

  auto compute = [&](const i32x4_t* wf, const i32x4_t* xf, const i32x4_t& gf) {
    float gv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gv[2 * e] = bf16_lo((uint32_t)gf[e]);
      gv[2 * e + 1] = bf16_hi((uint32_t)gf[e]);
    }
#pragma unroll
    for (int mg = 0; mg < 2; ++mg) {
      i32x4_t h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo((uint32_t)xf[mg][e]), x1 = bf16_hi((uint32_t)xf[mg][e]);
        ssq[mg] = __builtin_fmaf(x0, x0, ssq[mg]);
        ssq[mg] = __builtin_fmaf(x1, x1, ssq[mg]);
        const float p0 = x0 * gv[2 * e], p1 = x1 * gv[2 * e + 1];  // exact
        const uint32_t hp = pack_bf16x2(p0, p1);
        h[e] = (int)hp;
        l[e] = (int)pack_bf16x2(p0 - bf16_lo(hp), p1 - bf16_hi(hp));  // exact residuals
      }
#pragma unroll
      for (int b = 0; b < NRB; ++b) {
        acc[b][mg] = mfma16x16x32(as_bf16x8(wf[b]), as_bf16x8(h), acc[b][mg]);
        acc[b][mg] = mfma16x16x32(as_bf16x8(wf[b]), as_bf16x8(l), acc[b][mg]);
      }
    }
  };

  // Double-buffered super-steps.  Loads complete in order, so each super-step
  // issues its own X and g first and then the next super-step's W; the wait
  // before computing then leaves that W in flight.  Scheduling barriers keep
  // the issue order.
  constexpr int STEP = 32 * SS;
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
      for (int t = 0; t < SS; ++t)
        if (kc + 32 * t < hi) compute(wb[u].w[t], xb.x[t], xb.g[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Sums of squares of token r over this wave's columns: add the four column groups.
#pragma unroll
  for (int mg = 0; mg < 2; ++mg) {
    ssq[mg] += __shfl_xor(ssq[mg], 16, 64);
    ssq[mg] += __shfl_xor(ssq[mg], 32, 64);
  }

  // Add the four waves' parts: wave w keeps row block w.  Lane holds
  // U^T[weight row 16 b + 4 kg + i][token r] of each column group.
  __shared__ f32x4_t red[NW][NRB * 2][64];  // 32 KiB
  __shared__ float red_ssq[NW][2][16];
#pragma unroll
  for (int b = 0; b < NRB; ++b)
#pragma unroll
    for (int mg = 0; mg < 2; ++mg) red[w][2 * b + mg][lane] = acc[b][mg];
  if (kg == 0) {
    red_ssq[w][0][r] = ssq[0];
    red_ssq[w][1][r] = ssq[1];
  }
  __syncthreads();
  f32x4_t tot[2];
  float ssq_tot[2];
#pragma unroll
  for (int mg = 0; mg < 2; ++mg) {
    tot[mg] = red[0][2 * w + mg][lane];
    ssq_tot[mg] = red_ssq[0][mg][r];
#pragma unroll
    for (int u = 1; u < NW; ++u) {
      tot[mg] += red[u][2 * w + mg][lane];
      ssq_tot[mg] += red_ssq[u][mg][r];
    }
  }

  const int n_lane = n_wg + 16 * w + 4 * kg;
#pragma unroll
  for (int mg = 0; mg < 2; ++mg) {
    const int m = m0 + 16 * mg + r;
    if (m >= p.M || 16 * w + 4 * kg >= wrows) continue;  // rows past the tile: the next one's
    if (p.s == 1) {
      // The whole K range is here: apply the row scale after the Matmul.
      const float scale = 1.0f / sqrtf(ssq_tot[mg] / (float)p.K + p.eps);
      store_row4(p, m, n_lane, tot[mg] * scale);
      continue;
    }
    float* dst = p.ws_u + ((int64_t)j * p.M + m) * p.N + n_lane;
    if (n_lane + 3 < p.N && (p.N & 3) == 0) {
      *reinterpret_cast<f32x4_t*>(dst) = tot[mg];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n_lane + i < p.N) dst[i] = tot[mg][i];
    }
    if (blockIdx.x == 0 && w == 0 && kg == 0) p.ws_ssq[(int64_t)j * p.M + m] = ssq_tot[mg];
  }
}

// Combine: Y[m, n] = (sum_j U_j[m, n]) / sqrt(sum_j SSQ_j[m] / K + eps).
// Thread t handles four consecutive n of one row.
__global__ __launch_bounds__(256) void rmsnorm_matmul_combine_kernel(RmsParams p) {
  const int64_t quads = (int64_t)(p.N + 3) / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= quads * p.M) return;
  const int m = (int)(t / quads);
  const int n = (int)(t - (int64_t)m * quads) * 4;
  float ssq = 0.f;
  for (int j = 0; j < p.s; ++j) ssq += p.ws_ssq[(int64_t)j * p.M + m];
  const float scale = 1.0f / sqrtf(ssq / (float)p.K + p.eps);
  f32x4_t u = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < p.s; ++j) {
    const float* src = p.ws_u + ((int64_t)j * p.M + m) * p.N + n;
    if (n + 3 < p.N && (p.N & 3) == 0) {
      u += *reinterpret_cast<const f32x4_t*>(src);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < p.N) u[i] += src[i];
    }
  }
  store_row4(p, m, n, u * scale);
}

}  // namespace

hipError_t launch_rmsnorm_matmul(const RmsParams& p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.N + p.tile_n - 1) / p.tile_n), (unsigned)p.s,
                  (unsigned)((p.M + 31) / 32));
  hipLaunchKernelGGL(rmsnorm_matmul_split_kernel, grid, dim3(NW * 64), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.s == 1) return e;
  const int64_t threads = (int64_t)p.M * ((p.N + 3) / 4);
  hipLaunchKernelGGL(rmsnorm_matmul_combine_kernel, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn

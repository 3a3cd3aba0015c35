// The prefill setting of RMSNorm followed by a MatMul and of SwiGLU (Cleave
// §7.3 evaluates both subgraphs in the prefill and the decode setting): with
// thousands of tokens the MatMuls are compute-bound, so they run as a tiled
// bf16 MFMA GEMM over X [M, K] and the weights [N, K] (both row-major, K
// contiguous), fp32 accumulation, with the subgraph's elementwise work in the
// epilogue.
//
// * RMSNorm + MatMul (mode 0).  A first pass over X (rms_prep_kernel) forms
//   x * g exactly, as a bf16 pair hi + lo, and each token's row scale
//   1 / sqrt(mean(x^2) + eps) from the same read of X; the GEMM then
//   multiplies the un-normalised X * g by W (A steps alternate hi and lo
//   columns against the same W step: b_shift = 1) and applies the row scale
//   to the finished dot products -- the division moved after the MatMul
//   (Cleave §1, Fig. 1).  The normalised input is never formed, and the
//   gain costs no precision (at twice the MFMA work of a rounded x * g).
// * SwiGLU (mode 1).  One workgroup computes a 256-token x 128-column tile of
//   both X W_gate^T and X W_up^T from the same X tile (horizontal fusion: both
//   reductions read X once, Cleave §7.3) and writes silu(gate) * up.
//
// Workgroup: 8 waves (two per SIMD), a 256 x 256 tile of A B^T (for SwiGLU
// the B rows are 128 gate rows and the same 128 up rows).  Wave (wm, wn) =
// (w & 1, w >> 1) computes rows 128 wm .. + 127 and B rows 64 wn .. + 63 (for
// SwiGLU: gate rows 32 wn .. + 31 and the up rows beside them) as 4 x 2 MFMA
// tiles of 32 x 32 (mfma_f32_32x32x16_bf16), 128 accumulators per lane.
// K goes in steps of 32 columns: the A and B tiles of a step (16 KiB each)
// are copied HBM -> LDS by buffer loads that write LDS directly, into a
// 4-stage ring (three steps in flight).  A tile row is 64 bytes; 16-byte chunk
// c of row r sits at chunk c ^ ((r >> 2) & 3), which keeps the fragment reads
// (32 rows, two chunks per instruction) free of bank conflicts.
// Workgroups are ordered so that the eight XCDs each own every eighth column
// tile and run through all row tiles of it: a weight tile is fetched from HBM
// once per XCD and reused from that XCD's L2 by every row tile.
#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {
namespace {

constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int BM = 256;              // A rows per workgroup
constexpr int BB = 256;              // B rows per workgroup
constexpr int BK = 32;               // columns of K per step
constexpr int ROWB = BK * 2;         // bytes per tile row
constexpr int TILE = BM * ROWB;      // 16 KiB per operand and stage
constexpr int STAGE = 2 * TILE;      // A tile then B tile
constexpr int NS = 4;                // ring stages
constexpr int LOOK = NS - 1;         // steps in flight
constexpr int LDS_BYTES = NS * STAGE;  // 128 KiB
constexpr int DMA_PER_OP = TILE / 1024;        // 16 one-KiB copies per operand and stage
constexpr int DMA_PER_WAVE = DMA_PER_OP / NW;  // 2 per operand and wave
static_assert(DMA_PER_WAVE == 2, "vmcnt values below assume 4 copies per wave and stage");

typedef __attribute__((address_space(3))) const i32x4_t lds_i32x4_t;
__device__ __forceinline__ i32x4_t ds_read16_at(uint32_t lds_addr) {
  return *reinterpret_cast<lds_i32x4_t*>((uintptr_t)lds_addr);
}
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Y[m, n] (bf16 rounded to nearest even, or fp32) when inside the matrix.
__device__ __forceinline__ void store_y(const GemmParams& p, int m, int n, float v) {
  if (m >= p.M || n >= p.N) return;
  if (p.y_bf16)
    reinterpret_cast<uint16_t*>(p.y)[(int64_t)m * p.y_row + n] = (uint16_t)f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(p.y)[(int64_t)m * p.y_row + n] = v;
}

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_nt_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w & 1, wn = w >> 1;

  // Tile order: XCD x = id % 8 takes column tiles x, x + 8, ... and all row
  // tiles of each (row tiles fastest), when the column tiles split evenly.
  constexpr int NOUT = MODE == 0 ? BB : BB / 2;  // output columns per workgroup
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + NOUT - 1) / NOUT;
  const int id = blockIdx.x;
  int mt, nt;
  if ((tiles_n & 7) == 0) {
    const int x = id & 7, k = id >> 3;
    nt = x + 8 * (k / tiles_m);
    mt = k % tiles_m;
  } else {
    nt = id / tiles_m;
    mt = id % tiles_m;
  }
  const int m0 = mt * BM, n0 = nt * NOUT;

  // Buffer resources: rows past M (or N) read as zero.
  const uint32_t ast = (uint32_t)(p.a_row * 2), b0st = (uint32_t)(p.b0_row * 2),
                 b1st = (uint32_t)(p.b1_row * 2);
  const int arows = min(BM, p.M - m0);
  const __amdgpu_buffer_rsrc_t ars =
      make_rsrc(reinterpret_cast<const uint16_t*>(p.a) + (int64_t)m0 * p.a_row, (uint32_t)arows * ast);
  const int brows = min(NOUT, p.N - n0);
  const __amdgpu_buffer_rsrc_t b0rs =
      make_rsrc(reinterpret_cast<const uint16_t*>(p.b0) + (int64_t)n0 * p.b0_row, (uint32_t)brows * b0st);
  const __amdgpu_buffer_rsrc_t b1rs = MODE == 0 ? b0rs :
      make_rsrc(reinterpret_cast<const uint16_t*>(p.b1) + (int64_t)n0 * p.b1_row, (uint32_t)brows * b1st);

  // Copies of a stage: wave w fills A slots 64 (2w + u) + lane and B slots
  // likewise (u = 0, 1): slot s holds row s / 4, physical chunk s % 4, i.e.
  // logical chunk (s % 4) ^ swz(row).  For SwiGLU, B rows 0..127 are gate rows
  // and 128..255 up rows (waves 0-3 copy the former, 4-7 the latter).
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem);
  uint32_t a_off[DMA_PER_WAVE], b_off[DMA_PER_WAVE];
#pragma unroll
  for (int u = 0; u < DMA_PER_WAVE; ++u) {
    const int slot = 64 * (DMA_PER_WAVE * w + u) + lane;
    const int row = slot >> 2, c = (slot & 3) ^ swz(row);
    a_off[u] = (uint32_t)row * ast + 16u * (uint32_t)c;
    const int brow = MODE == 0 ? row : (row & 127);
    b_off[u] = (uint32_t)brow * (MODE == 0 || row < 128 ? b0st : b1st) + 16u * (uint32_t)c;
  }
  const bool b_up = MODE == 1 && w >= NW / 2;
  auto dma = [&](int step, int stage) {
    const uint32_t kb = (uint32_t)step * BK * 2, kbb = (uint32_t)(step >> p.b_shift) * BK * 2;
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const uint32_t m0a = smem_lds + (uint32_t)(stage * STAGE + (DMA_PER_WAVE * w + u) * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(m0a), "v"(a_off[u] + kb), "s"(ars) : "memory", "m0");
      const uint32_t m0b = m0a + TILE;
      if (b_up)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m0b), "v"(b_off[u] + kbb), "s"(b1rs) : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m0b), "v"(b_off[u] + kbb), "s"(b0rs) : "memory", "m0");
    }
  };
  // All copies of a step have landed once at most `later` newer steps' copies
  // (4 instructions each) are outstanding.
  auto wait_steps_but = [&](int later) {
    switch (later) {
      case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    }
  };

  // Per-lane fragment addresses (loop invariant): A block i row 128 wm + 32 i
  // + lane % 32, B block j row (mode 0) 64 wn + 32 j + lane % 32, (mode 1)
  // 32 wn + lane % 32 + 128 j; chunk 2 * sub + lane / 32, swizzled.
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t a_rd[4][2], b_rd[2][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = 128 * wm + 32 * i + lr;
      a_rd[i][sub] = smem_lds + (uint32_t)(row * ROWB + 16 * ((2 * sub + lh) ^ swz(row)));
      asm volatile("" : "+v"(a_rd[i][sub]));
    }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = MODE == 0 ? 64 * wn + 32 * j + lr : 32 * wn + lr + 128 * j;
      b_rd[j][sub] = smem_lds + (uint32_t)(TILE + row * ROWB + 16 * ((2 * sub + lh) ^ swz(row)));
      asm volatile("" : "+v"(b_rd[j][sub]));
    }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nsteps = p.K / BK;
#pragma unroll
  for (int t = 0; t < LOOK; ++t)
    if (t < nsteps) dma(t, t);
  wait_steps_but(min(LOOK - 1, nsteps - 1));
  asm volatile("s_barrier" ::: "memory");

  // Step t reads stage t % NS; the copy of step t + LOOK refills the stage step
  // t - 1 read, which every wave left at the barrier ending step t - 1.
  for (int t = 0; t < nsteps; ++t) {
    if (t + LOOK < nsteps) dma(t + LOOK, (t + LOOK) & (NS - 1));
    const uint32_t so = (uint32_t)((t & (NS - 1)) * STAGE);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      i32x4_t a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = ds_read16_at(a_rd[i][sub] + so);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = ds_read16_at(b_rd[j][sub] + so);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma32x32x16(as_bf16x8(a[i]), as_bf16x8(b[j]), acc[i][j]);
    }
    wait_steps_but(max(0, min(LOOK - 1, nsteps - 2 - t)));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // Epilogue.  Lane holds, for A block i and B block j, rows
  // 8 (e / 4) + 4 (lane / 32) + e % 4 of the block and its column lane % 32.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * lh + (e & 3);
      if constexpr (MODE == 0) {
        const float rs = m < p.M ? p.row_scale[m] : 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) store_y(p, m, n0 + 64 * wn + 32 * j + lr, acc[i][j][e] * rs);
      } else {
        store_y(p, m, n0 + 32 * wn + lr, silu(acc[i][0][e]) * acc[i][1][e]);
      }
    }
}

// The exact product x * g (two bf16 significands fit in fp32's) as a bf16
// pair hi + lo, hi = RNE(x g) and lo = x g - hi (at most 8 significant bits,
// so exact in bf16), stored per 32-column step as [hi of the step | lo of the
// step], and the row scale 1 / sqrt(mean(x^2) + eps); one read of the row,
// one workgroup per token row.
__global__ __launch_bounds__(256) void rms_prep_kernel(RmsPrepParams p) {
  const int m = blockIdx.x;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(p.x) + (int64_t)m * p.x_row;
  const uint16_t* g = reinterpret_cast<const uint16_t*>(p.g);
  uint16_t* xg = reinterpret_cast<uint16_t*>(p.xg) + (int64_t)m * p.xg_row;
  float ssq = 0.f;
  for (int k = 8 * threadIdx.x; k < p.K; k += 8 * 256) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + k);
    const uint4 gv = *reinterpret_cast<const uint4*>(g + k);
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t gs[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(xs[e]), x1 = bf16_hi(xs[e]);
      ssq = __builtin_fmaf(x0, x0, ssq);
      ssq = __builtin_fmaf(x1, x1, ssq);
      const float p0 = x0 * bf16_lo(gs[e]), p1 = x1 * bf16_hi(gs[e]);
      hi[e] = pack_bf16x2(p0, p1);
      lo[e] = pack_bf16x2(p0 - bf16_lo(hi[e]), p1 - bf16_hi(hi[e]));
    }
    const int base = 2 * (k & ~(BK - 1)) + (k & (BK - 1));
    *reinterpret_cast<uint4*>(xg + base) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(xg + base + BK) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  ssq = wave_sum(ssq);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ssq;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    p.row_scale[m] = 1.0f / sqrtf(tot / (float)p.K + p.eps);
  }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmParams& p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const int nout = p.mode == 0 ? BB : BB / 2;
  const int64_t nwg = (int64_t)((p.M + BM - 1) / BM) * ((p.N + nout - 1) / nout);
  const void* fn = p.mode == 0 ? reinterpret_cast<const void*>(&gemm_nt_kernel<0>)
                               : reinterpret_cast<const void*>(&gemm_nt_kernel<1>);
  if (hipError_t e = set_lds_limit_once(fn, LDS_BYTES)) return e;
  if (p.mode == 0)
    hipLaunchKernelGGL(gemm_nt_kernel<0>, dim3((unsigned)nwg), dim3(NT), LDS_BYTES, s, p);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<1>, dim3((unsigned)nwg), dim3(NT), LDS_BYTES, s, p);
  return hipGetLastError();
}

hipError_t launch_rms_prep(const RmsPrepParams& p, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  hipLaunchKernelGGL(rms_prep_kernel, dim3((unsigned)p.M), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn

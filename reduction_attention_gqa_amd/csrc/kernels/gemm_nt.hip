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
//   multiplies the un-normalised X * g by W (A steps alternate the hi and
//   the lo parts of 64 columns against the same W step: b_shift = 1) and applies the row scale
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
// K goes in steps of 64 columns, so that each tile row of a step is one
// whole 128-byte line (the L2 serves whole lines at twice the rate of half
// lines): the A and B tiles of a step (32 KiB each) are copied HBM -> LDS by
// buffer loads that write LDS directly, into a 2-stage ring (the next step's
// copy in flight during a step).  16-byte chunk c of tile row r sits at chunk
// c ^ ((r / 2) % 8), which keeps the fragment reads (32 rows, two chunks per
// instruction) free of bank conflicts.
// Workgroups are ordered so that the eight XCDs each own every eighth column
// tile (a weight tile is fetched by one XCD only) and walk their tiles in
// bands of GROUP_M row tiles, so that the workgroups an XCD runs at once
// share their A and B tiles through its L2.
#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {
namespace {

constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int BM = 256;              // A rows per workgroup
constexpr int BB = 256;              // B rows per workgroup
constexpr int BK = 64;               // columns of K per step
constexpr int ROWB = BK * 2;         // bytes per tile row: one 128-byte line
constexpr int CH = ROWB / 16;        // 16-byte chunks per tile row
constexpr int SUBS = BK / 16;        // MFMA k-steps (16 columns) per step
constexpr int TILE = BM * ROWB;      // 32 KiB per operand and stage
constexpr int STAGE = 2 * TILE;      // A tile then B tile
constexpr int NS = 2;                // ring stages
constexpr int LOOK = NS - 1;         // steps in flight
constexpr int GROUP_M = 8;           // row tiles per band of the tile order
constexpr int LDS_BYTES = NS * STAGE;  // 128 KiB
constexpr int DMA_PER_OP = TILE / 1024;        // one-KiB copies per operand and stage
constexpr int DMA_PER_WAVE = DMA_PER_OP / NW;  // per operand and wave
constexpr int LOADS_PER_STEP = 2 * DMA_PER_WAVE;  // copy instructions per wave and step
static_assert(LOOK <= 2, "wait_steps_but covers at most one newer step");

typedef __attribute__((address_space(3))) const i32x4_t lds_i32x4_t;
__device__ __forceinline__ i32x4_t ds_read16_at(uint32_t lds_addr) {
  return *reinterpret_cast<lds_i32x4_t*>((uintptr_t)lds_addr);
}
// Chunk c of tile row r sits at chunk c ^ ((r / 2) % CH).  The LDS serves a
// 16-byte read sixteen lanes at a time over 64 four-byte banks (256 bytes),
// and a 128-byte tile row covers half of them, its parity choosing the half:
// sixteen consecutive rows, one chunk each, then cover all 64 banks once.
// (c ^ (r % CH) would map rows r and r + 8 onto the same banks.)
__device__ __forceinline__ int swz(int r) { return (r >> 1) & (CH - 1); }
// s_waitcnt immediate: lgkmcnt(0), vmcnt and expcnt at their maxima (no wait).
constexpr int kWaitLgkm0 = 0xC07F;
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

  // Tile order.  When the column tiles split evenly over the eight XCDs, XCD
  // x = id % 8 takes column tiles x, x + 8, ... (so each weight tile is
  // fetched by one XCD only); its k-th workgroup takes local tile k of a grid
  // of row tiles x owned column tiles walked in bands of GROUP_M row tiles,
  // down a column of the band first.  The workgroups an XCD runs at once
  // (32) then cover GROUP_M rows x 32 / GROUP_M columns, and a k-step of
  // them needs GROUP_M + 32 / GROUP_M operand tiles from outside the XCD
  // rather than one per workgroup.
  constexpr int NOUT = MODE == 0 ? BB : BB / 2;  // output columns per workgroup
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + NOUT - 1) / NOUT;
  const int id = blockIdx.x;
  int mt, nt;
  if ((tiles_n & 7) == 0) {
    const int x = id & 7, k = id >> 3;
    const int cols = tiles_n >> 3;                 // column tiles of this XCD
    const int band = k / (GROUP_M * cols);
    const int r0 = band * GROUP_M;
    const int rows = min(GROUP_M, tiles_m - r0);   // rows of this band
    const int kb = k - band * GROUP_M * cols;
    mt = r0 + kb % rows;
    nt = x + 8 * (kb / rows);
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

  // Copies of a stage: wave w fills A slots 64 (DMA_PER_WAVE w + u) + lane and
  // B slots likewise: slot s holds row s / CH, physical chunk s % CH, i.e.
  // logical chunk (s % CH) ^ swz(row); eight lanes copy one whole row (a
  // 128-byte line).  For SwiGLU, B rows 0..127 are gate rows and 128..255 up
  // rows (waves 0-3 copy the former, 4-7 the latter).
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem);
  uint32_t a_off[DMA_PER_WAVE], b_off[DMA_PER_WAVE];
#pragma unroll
  for (int u = 0; u < DMA_PER_WAVE; ++u) {
    const int slot = 64 * (DMA_PER_WAVE * w + u) + lane;
    const int row = slot / CH, c = (slot % CH) ^ swz(row);
    a_off[u] = (uint32_t)row * ast + 16u * (uint32_t)c;
    const int brow = MODE == 0 ? row : (row & 127);
    b_off[u] = (uint32_t)brow * (MODE == 0 || row < 128 ? b0st : b1st) + 16u * (uint32_t)c;
  }
  const bool b_up = MODE == 1 && w >= NW / 2;
  const __amdgpu_buffer_rsrc_t brs = b_up ? b1rs : b0rs;
  // The compiler's own buffer-to-LDS load (it sets M0 itself and knows that
  // the fragment reads do not use it, so it does not drain them first).
  typedef __attribute__((address_space(3))) void lds_void_t;
  auto dma = [&](int step, int stage) {
    const uint32_t kb = (uint32_t)step * BK * 2, kbb = (uint32_t)(step >> p.b_shift) * BK * 2;
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int slot0 = stage * STAGE + (DMA_PER_WAVE * w + u) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void_t*)(smem + slot0), 16,
                                               (int)(a_off[u] + kb), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void_t*)(smem + slot0 + TILE), 16,
                                               (int)(b_off[u] + kbb), 0, 0, 0);
    }
  };
  // All copies of a step have landed once at most `later` newer steps' copies
  // are outstanding.
  auto wait_steps_but = [&](int later) {
    if (later <= 0)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LOADS_PER_STEP) : "memory");
  };

  // Per-lane fragment addresses (loop invariant): A block i row 128 wm + 32 i
  // + lane % 32, B block j row (mode 0) 64 wn + 32 j + lane % 32, (mode 1)
  // 32 wn + lane % 32 + 128 j; chunk 2 sub + lane / 32, swizzled.
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t a_rd[4][SUBS], b_rd[2][SUBS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int sub = 0; sub < SUBS; ++sub) {
      const int row = 128 * wm + 32 * i + lr;
      a_rd[i][sub] = smem_lds + (uint32_t)(row * ROWB + 16 * ((2 * sub + lh) ^ swz(row)));
      asm volatile("" : "+v"(a_rd[i][sub]));
    }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int sub = 0; sub < SUBS; ++sub) {
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

  // Fragments of one 16-column k-step: A blocks i and B blocks j.
  struct Frags { i32x4_t a[4], b[2]; };
  auto read_frags = [&](Frags& f, uint32_t so, int sub) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = ds_read16_at(a_rd[i][sub] + so);
#pragma unroll
    for (int j = 0; j < 2; ++j) f.b[j] = ds_read16_at(b_rd[j][sub] + so);
  };
  auto mfmas = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = mfma32x32x16(as_bf16x8(f.a[i]), as_bf16x8(f.b[j]), acc[i][j]);
  };

  // Step t reads stage t % NS, SUBS k-steps of 16 columns; the fragments of
  // k-step s + 1 are read while the MFMAs of k-step s run.  The first
  // k-step's fragments are read right after the barrier that makes the
  // stage visible, and that barrier comes before the last k-step's MFMAs of
  // the step before, which then cover the reads.  The copy of step t + LOOK,
  // issued at the start of step t, refills the stage of step t - 1, which
  // every wave finished reading before the barrier that ended step t - 1.
  Frags f[2];
  read_frags(f[0], 0u, 0);
  for (int t = 0; t < nsteps; ++t) {
    if (t + LOOK < nsteps) dma(t + LOOK, (t + LOOK) % NS);
    const uint32_t so = (uint32_t)((t % NS) * STAGE);
#pragma unroll
    for (int sub = 0; sub + 1 < SUBS; ++sub) {
      // Scheduling barriers keep the next k-step's reads ahead of this
      // k-step's MFMAs (left alone, the compiler sinks each read to its use).
      read_frags(f[(sub + 1) & 1], so, sub + 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(f[sub & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_steps_but(max(0, min(LOOK - 1, nsteps - 2 - t)));
    // The compiler's own wait and barrier: it then knows that the fragments
    // read before the barrier have arrived.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");   // no LDS access moves across the barrier
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nsteps) read_frags(f[0], (uint32_t)(((t + 1) % NS) * STAGE), 0);
    mfmas(f[(SUBS - 1) & 1]);
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
// so exact in bf16), stored per 64-column step as [hi of the step | lo of the
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

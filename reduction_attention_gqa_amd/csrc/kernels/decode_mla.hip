// Split-K MLA-style decode for bf16: one latent KV head, Dqk = 576, Dv = 512,
// V = the first 512 columns of K, up to 128 query rows (heads x queries) per
// KV head.
//
// One workgroup (8 waves) owns one (split, KV head, request) unit, so every
// latent K row is read from HBM once per split and serves both contractions:
// the 576-wide QK^T and, through its first 512 columns, the PV.  Waves come in
// pairs per 32-row group: wave (rg, half) holds Q^T for half of the 576-wide
// contraction (18 k-steps) and the fp32 accumulator for half of the 512 output
// columns.  Per 32-key tile:
//   partial S^T[32 x 32] = K[32 x 288-half] Q^T[288-half x 32]   18 MFMA 32x32x16
//   the pair adds its two partials through LDS (a + b == b + a bit for bit, so
//     both waves hold the same scores and take the same softmax decisions)
//   O^T[256 x 32] += V^T[256-half x 32] P^T[32 x 32]             8 x 2 MFMA 32x32x16
// Q^T stays in VGPRs for the whole split (loop-invariant, Cleave §6.1).
// Rescaling the accumulator on every tile would cost more VALU time than the
// tile's MFMAs, so the running max is updated lazily: a row's reference max
// moves (and its accumulator and row sum are rescaled) only when the row's max
// grows by more than 2^8; otherwise P = 2^(s - m_ref) <= 256 is used as is.
// Row sum and accumulator always share one reference, so O = U / l is
// unchanged.
//
// The K tile is copied HBM -> LDS by buffer loads that write LDS directly (no
// staging registers).  Rows are padded to 73 16-byte chunks, so the A-operand
// reads of K (8 consecutive keys per pass) hit distinct banks and every LDS
// offset in the loop is a compile-time immediate.
#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {
namespace {

constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int TK = kMlaTileN;          // 32 keys per tile
constexpr int DQK = 576, DV = 512;
constexpr int KS_HALF = DQK / 16 / 2;  // 18 k-steps per wave
constexpr int DB_HALF = DV / 32 / 2;   // 8 output d-blocks per wave
constexpr int CHUNKS = DQK / 8;        // 72 16-byte chunks of data per key row
constexpr int SLOTS = CHUNKS + 1;      // + 1 pad chunk
constexpr int ROW_BYTES = SLOTS * 16;  // 1168
constexpr int STAGE = TK * ROW_BYTES;  // 37,376
constexpr int XBUF = NW * 64 * 16 * 4; // partial-score exchange, 32 KiB
constexpr int NSTAGE = 3;              // tiles it, it + 1, it + 2 resident
constexpr int LDS_BYTES = NSTAGE * STAGE + XBUF;  // 144,896
constexpr int NSLOT = TK * SLOTS;      // 2336 16-byte slots per stage
constexpr int NBLK = (NSLOT + 63) / 64;  // 37 one-KiB DMA blocks
constexpr float kRescaleThreshold = 8.0f;  // log2 units

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Byte offset of (key, 16-byte chunk c) in a stage.
__device__ __forceinline__ int chunk_off(int key, int c) { return key * ROW_BYTES + 16 * c; }

__device__ __forceinline__ i32x2_t ds_read_tr(const char* lds) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds));
  return __builtin_bit_cast(i32x2_t, v);
}

__global__ __launch_bounds__(NT) void decode_mla_kernel(KParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = threadIdx.x;
  const int j = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int L = kv_len_of(p.kv_lens, b, p.Lcap);
  const int lo = j * p.chunk;
  if (lo >= L) return;
  const int hi = min(lo + p.chunk, L);

  const int rg = w >> 1;      // 32-row group
  const int half = w & 1;     // contraction half for QK, column half for PV
  const int G = p.G;
  const int R = p.rows;
  const int c = lane & 31;
  const int h = lane >> 5;
  const int r = 32 * rg + c;
  const int qi = r / G;
  const int qh = kvh * G + r % G;
  const bool row_ok = r < R;
  const int qlim = qi + L - p.Lq;

  // Q^T (this wave's 18 k-steps) as the B operand: Q[row r][16*ks + 8*h .. +7].
  bf16x8_t qf[KS_HALF];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.qs_b +
                         (int64_t)qi * p.qs_t + (int64_t)qh * p.qs_h + 16 * KS_HALF * half;
#pragma unroll
    for (int ks = 0; ks < KS_HALF; ++ks) {
      i32x4_t v = {0, 0, 0, 0};
      if (row_ok) v = *reinterpret_cast<const i32x4_t*>(qp + 16 * ks + 8 * h);
      qf[ks] = as_bf16x8(v);
    }
    // Wait for Q here, once: otherwise the wait lands at the loop head and also
    // drains the K/V DMA in flight on every tile.
#pragma unroll
    for (int ks = 0; ks < KS_HALF; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const uint32_t kst = (uint32_t)(p.ks_t * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)L * kst);

  // Tile copy, HBM -> LDS without registers (buffer_load ... lds): each wave
  // instruction fills one KiB of the stage, lane l the 16-byte slot 64*blk + l.
  // Slot P holds chunk P % 73 of key P / 73; pad slots and slots past the stage
  // are left to inactive lanes.  Waves 0-4 issue 5 instructions per tile, waves
  // 5-7 issue 4 (37 blocks).
  // The DMA is issued from inline asm so the compiler does not pair it with
  // conservative vmcnt waits before unrelated LDS reads; completion is awaited
  // explicitly (wait_older_tile) before each barrier that publishes a tile.
  const int w_s = __builtin_amdgcn_readfirstlane(w);  // wave index in an SGPR
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem);
  auto gload_lds = [&](int k0, int stage) {
    const uint32_t base = smem_lds + (uint32_t)(stage * STAGE);
    const uint32_t soff = (uint32_t)k0 * kst;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recompute the slot offsets per tile (no spills)
#pragma unroll
    for (int u = 0; u < (NBLK + NW - 1) / NW; ++u) {
      const int blk = u * NW + w_s;
      if (blk < NBLK) {
        const int P = blk * 64 + ln;
        const int key = P / SLOTS, cc = P % SLOTS;
        const uint32_t m0v = base + (uint32_t)(blk * 1024);
        const uint32_t voff = (uint32_t)key * kst + 16 * cc;
        if (P < NSLOT && cc < CHUNKS) {
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                       :: "s"(m0v), "v"(voff), "s"(krs), "s"(soff) : "memory", "m0");
        }
      }
    }
  };
  // All DMA of the older tile has landed once at most the newer tile's
  // instructions are outstanding (loads complete in order).
  auto wait_older_tile = [&]() {
    if (w < NBLK - 4 * NW)
      asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  };
  float* xbuf = reinterpret_cast<float*>(smem + NSTAGE * STAGE);   // [NW][16][64] floats
  float* xmine = xbuf + w * 1024;
  const float* xpeer = xbuf + (w ^ 1) * 1024;

  f32x16_t oacc[DB_HALF];
#pragma unroll
  for (int db = 0; db < DB_HALF; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_ref = kNegInf;   // reference max of this lane's row (base-2 units)
  float l_part = 0.f;
  const float sl2 = p.scale_log2;

  // Transposed V read: 16-lane group gq reads keys 4*(gq>>1) + li/4 (+8), element
  // columns 32*db + 16*(gq&1) + 4*(li&3) .. +3 of this wave's 256-column half.
  const int gq = lane >> 4, li = lane & 15;
  const int vkey = 4 * (gq >> 1) + (li >> 2);
  const int vcol = 256 * half + 16 * (gq & 1) + 4 * (li & 3);

  const int ntiles = (hi - lo + TK - 1) / TK;
  // Barriers are written as s_barrier after an LDS-only wait: a plain
  // __syncthreads() would also wait for the LDS DMA of the tiles in flight.
  gload_lds(lo, 0);
  if (ntiles > 1) {
    gload_lds(lo + TK, 1);
    wait_older_tile();
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  int st_cur = 0, st_pre = 2;  // stage of tile it, stage for tile it + 2
  for (int it = 0; it < ntiles; ++it) {
    const int k0 = lo + it * TK;
    const bool prefetch = it + 2 < ntiles;
    if (prefetch) gload_lds(k0 + 2 * TK, st_pre);
    const char* kl = smem + st_cur * STAGE;

    // Partial S^T over this wave's half of the contraction.
    f32x16_t s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS_HALF; ++ks) {
      const int chunk = 2 * (KS_HALF * half + ks) + h;
      const i32x4_t kf = *reinterpret_cast<const i32x4_t*>(kl + chunk_off(c, chunk));
      s = mfma32x32x16(as_bf16x8(kf), qf[ks], s);
    }
    // Exchange partials with the peer wave (column-major [e][lane]: no bank conflicts).
#pragma unroll
    for (int e = 0; e < 16; ++e) xmine[e * 64 + lane] = s[e];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] += xpeer[e * 64 + lane];

    const bool need_mask = (k0 + TK > hi) || (p.causal && k0 + TK - 1 > qlim) || !row_ok;
    float mt = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = s[e] * sl2;
      if (need_mask) {
        const int key = k0 + 8 * (e >> 2) + 4 * h + (e & 3);
        const bool vis = key < hi && (!p.causal || key <= qlim) && row_ok;
        v = vis ? v : kNegInf;
      }
      s[e] = v;
      mt = fmaxf(mt, v);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // Lazy rescale: move the reference only when some row's max outgrows it.
    const bool grow = mt > m_ref + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_ref, mt);
      // On a row's first update the accumulator and sum are still zero.
      const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB_HALF; ++db) oacc[db] *= alpha;
      m_ref = m_new;
    }
    const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = fast_exp2(s[e] - m_use);
      s[e] = pv;
      ps += pv;
    }
    l_part += ps;

    // O^T += V^T P^T over two 16-key steps.
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      const int i0 = 2 * ts;
      i32x4_t pk;
      pk[0] = (int)pack_bf16x2(s[4 * i0 + 0], s[4 * i0 + 1]);
      pk[1] = (int)pack_bf16x2(s[4 * i0 + 2], s[4 * i0 + 3]);
      pk[2] = (int)pack_bf16x2(s[4 * i0 + 4], s[4 * i0 + 5]);
      pk[3] = (int)pack_bf16x2(s[4 * i0 + 6], s[4 * i0 + 7]);
      const bf16x8_t pb = as_bf16x8(pk);
      const int key_a = 16 * ts + vkey;
      const int key_b = key_a + 8;
#pragma unroll
      for (int db = 0; db < DB_HALF; ++db) {
        const int col = 32 * db + vcol;   // element column, multiple of 4
        const int ch = col >> 3, within = (col & 7) * 2;
        const i32x2_t lo2 = ds_read_tr(kl + chunk_off(key_a, ch) + within);
        const i32x2_t hi2 = ds_read_tr(kl + chunk_off(key_b, ch) + within);
        i32x4_t va;
        va[0] = lo2[0];
        va[1] = lo2[1];
        va[2] = hi2[0];
        va[3] = hi2[1];
        oacc[db] = mfma32x32x16(as_bf16x8(va), pb, oacc[db]);
      }
    }
    // Tile it + 1 must have landed; tile it + 2 may stay in flight.
    if (prefetch)
      wait_older_tile();
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    st_cur = st_cur == NSTAGE - 1 ? 0 : st_cur + 1;
    st_pre = st_pre == NSTAGE - 1 ? 0 : st_pre + 1;
  }

  // Split epilogue: O_j = U / l (fp32), LSE_j = (m_ref + log2 l) ln 2.
  const float l_row = l_part + __shfl_xor(l_part, 32, 64);
  if (row_ok) {
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const int64_t slot = (int64_t)j * p.B * p.Lq * p.Hq + ((int64_t)b * p.Lq + qi) * p.Hq + qh;
    float* dst = p.ws_o + slot * DV + 256 * half;
#pragma unroll
    for (int db = 0; db < DB_HALF; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4_t v;
        v[0] = oacc[db][4 * i + 0] * inv;
        v[1] = oacc[db][4 * i + 1] * inv;
        v[2] = oacc[db][4 * i + 2] * inv;
        v[3] = oacc[db][4 * i + 3] * inv;
        *reinterpret_cast<f32x4_t*>(dst + 32 * db + 8 * i + 4 * h) = v;
      }
    if (h == 0 && half == 0)
      p.ws_lse[slot] = l_row > 0.f ? (m_ref + fast_log2(l_row)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_decode_mla(const KParams& p, dim3 grid, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_mla_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(decode_mla_kernel, grid, dim3(NT), LDS_BYTES, s, p);
  return hipGetLastError();
}

}  // namespace attn

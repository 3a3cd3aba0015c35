// Fused causal / non-causal GQA prefill for bf16, Dqk = Dv = 128.
//
// One workgroup (4 waves) computes one 256-row tile of one (request, KV head)
// group; a row is a (query position, head of the group) pair, so the G query
// heads that share a KV head share every K/V tile staged in LDS.  This is the
// inter-threadblock output tiling of Cleave §5.1 / §5.3 ([b_O, d] output tiles,
// one per workgroup) with GQA packing added.  Inside, the key axis is tiled in
// 32-key steps (iterative tiling, §5.1 and §5.3); the exp tile feeds both the
// row sum and the V-matmul in the same step (horizontal fusion, §5.1); the
// division by the row sum comes after the V-matmul (§2.2, Fig. 2); the Q tile
// is loaded once, outside the key loop (§6.1).
//
// Each wave owns 64 rows as two 32-row MFMA column blocks, so every K or V
// fragment read from LDS feeds two MFMAs.  Per wave and 32-key tile, keys on
// the MFMA rows:
//   S^T[32 x 64]  = K[32 x 128] Q^T[128 x 64]     2 x 8 MFMA 32x32x16 bf16
//   O^T[128 x 64] += V^T[128 x 32] P^T[32 x 64]   2 x 8 MFMA 32x32x16 bf16
// One wave per SIMD (512 registers each): the matrix cores are kept busy by
// interleaving, within the wave, the scores of tile i + 1 with the
// exponentials of tile i, and the V-matmul of tile i with the max of tile
// i + 1 (fixed interleaves pinned with scheduling barriers).
//
// The running max is updated lazily: a row's reference max moves (and its
// accumulator and row sum are rescaled) only when the row's max grows by more
// than 2^8; otherwise P = 2^(s - m_ref) <= 256 is used as is.  Row sum and
// accumulator always share one reference, so O = U / l is unchanged.
//
// K/V tiles go HBM -> LDS by buffer loads that write LDS directly, four stages
// deep (tile i + 3 is in flight while tile i is consumed).  A tile row is 256
// bytes, and the 16-byte chunk c of row r sits at chunk c ^ swz(r), which keeps
// both the K operand reads (16 keys, one chunk each) and the transposed V reads
// (4 keys, 4 chunks each) free of bank conflicts.
//
// Causal tiles beyond a tile's diagonal are never loaded; masking runs only on
// tiles that straddle the diagonal or the end of the keys.  Workgroups are
// issued heaviest first, and (when the group count allows) each XCD works
// through one (request, KV head) group at a time so its K/V stays in that
// XCD's L2.
#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {
namespace {

constexpr int ROWS = 256;             // rows per workgroup
constexpr int TK = 32;                // keys per tile
constexpr int RB = 256;               // bytes per K or V row (128 bf16)
constexpr int KT = TK * RB;           // 8 KiB: one K (or V) tile
constexpr int STAGE = 2 * KT;         // K tile then V tile
constexpr int NSTAGE = 4;
constexpr int LDS_BYTES = NSTAGE * STAGE;  // 64 KiB
constexpr float kRescaleThreshold = 8.0f;  // log2 units

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 8 bytes addressed by lanes 4e + i / 4 (e = 0..3) as its element e.
__device__ __forceinline__ i32x2_t ds_read_tr(const char* lds) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds));
  return __builtin_bit_cast(i32x2_t, v);
}

__device__ __forceinline__ i32x2_t ds_read_tr_at(uint32_t lds_addr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)lds_addr);
  return __builtin_bit_cast(i32x2_t, v);
}

// Chunk swizzle: swap the two 2-bit fields of r mod 16.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// IEEE-754 2019 maximum (v_maximum3_f32): no canonicalisation of its inputs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// Byte offset of (row, 16-byte chunk c) inside a K or V tile.
__device__ __forceinline__ int tile_off(int row, int c) { return row * RB + 16 * (c ^ swz(row)); }

// NW waves per workgroup, each owning NCB 32-row MFMA column blocks
// (NW * NCB * 32 = 256 rows); NW / 4 waves per SIMD.
template <int NW, int NCB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void prefill_d128_kernel(KParams p, int nrt) {
  constexpr int RPW = 32 * NCB;       // rows per wave
  constexpr int NDMA = 8 / NW;        // 1 KiB DMA blocks per wave per K (or V) tile
  static_assert(NW * RPW == ROWS, "a workgroup covers 256 rows");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Workgroup -> (group, row tile): heaviest row tiles first; per-XCD groups.
  const int ngroups = p.B * p.Hkv;
  const int id = blockIdx.x;
  int group, rt;
  if ((ngroups & 7) == 0) {
    const int xcd = id & 7, k = id >> 3;
    group = xcd + 8 * (k / nrt);
    rt = nrt - 1 - (k % nrt);
  } else {
    group = id / nrt;
    rt = nrt - 1 - (id % nrt);
  }
  const int b = group / p.Hkv;
  const int kvh = group % p.Hkv;
  const int L = kv_len_of(p.kv_lens, b, p.Lcap);
  const int G = p.G;
  const int R = p.rows;            // Lq * G
  const int r0 = rt * ROWS;
  const int off = L - p.Lq;        // causal: row position i sees keys <= i + off

  // This wave's rows: lane (c, h) holds row rw0 + 32*cb + c of column block cb.
  const int c = lane & 31;
  const int h = lane >> 5;
  const int rw0 = r0 + RPW * w;
  int qi[NCB], qlim[NCB];
  bool row_ok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int r = rw0 + 32 * cb + c;
    qi[cb] = r / G;
    row_ok[cb] = r < R;
    qlim[cb] = qi[cb] + off;       // last visible key of this row (causal)
  }
  const int wg_rows = max(0, min(ROWS, R - r0));
  int kend = L;                    // keys [0, kend) are visible to some row of the workgroup
  if (p.causal) kend = min(L, (r0 + wg_rows - 1) / G + off + 1);
  kend = max(kend, 0);
  // Keys below kfull_w are visible to every row of this wave.
  const int kfull_w = p.causal ? max(0, min(L, rw0 / G + off + 1)) : L;

  // Q^T as the B operand (hoisted): lane holds Q[row][16*ks + 8*h .. +7].
  bf16x8_t qf[NCB][8];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int r = rw0 + 32 * cb + c;
      const int qh = kvh * G + (r % G);
      const int64_t qoff = (int64_t)b * p.qs_b + (int64_t)qi[cb] * p.qs_t + (int64_t)qh * p.qs_h;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        i32x4_t v = {0, 0, 0, 0};
        if (row_ok[cb]) v = *reinterpret_cast<const i32x4_t*>(qp + qoff + 16 * ks + 8 * h);
        qf[cb][ks] = as_bf16x8(v);
      }
    }
    // Wait for Q here, once, rather than at the loop head on every tile.
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[cb][ks]));
  }

  // Tile copy HBM -> LDS without registers: each wave fills rows
  // 4*(NDMA*w + u) .. + 3 (u < NDMA) of the K tile and of the V tile; lane l
  // writes the 16-byte slot (row 4*(NDMA*w+u) + l/16, position l%16), which
  // holds chunk (l%16) ^ swz(row).
  // The buffer ranges end at the last key, so rows past it are zero.
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;
  const uint32_t kst = (uint32_t)(p.ks_t * 2), vst = (uint32_t)(p.vs_t * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)L * kst);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (uint32_t)L * vst);
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem);
  uint32_t k_voff[NDMA], v_voff[NDMA];
#pragma unroll
  for (int u = 0; u < NDMA; ++u) {
    const int row = 4 * (NDMA * w + u) + (lane >> 4);
    const int chunk = (lane & 15) ^ swz(row);
    k_voff[u] = (uint32_t)row * kst + 16 * chunk;
    v_voff[u] = (uint32_t)row * vst + 16 * chunk;
  }
  // The whole byte offset goes in the per-lane offset, which the buffer range
  // check covers.  The DMA is issued from inline asm so the compiler does not
  // pair it with conservative waits; its completion is awaited explicitly
  // before each barrier that publishes a tile.
  auto dma_tile = [&](int k0, int stage) {
    const uint32_t base = smem_lds + (uint32_t)(stage * STAGE);
    const uint32_t ksoff = (uint32_t)k0 * kst, vsoff = (uint32_t)k0 * vst;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
      const uint32_t m0k = base + (uint32_t)((NDMA * w + u) * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(m0k), "v"(k_voff[u] + ksoff), "s"(krs) : "memory", "m0");
      const uint32_t m0v = m0k + KT;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(m0v), "v"(v_voff[u] + vsoff), "s"(vrs) : "memory", "m0");
    }
  };

  // s_waitcnt vmcnt(n * 2 * NDMA): all but the last n tiles' DMA has landed
  // (loads complete in order; 2 * NDMA instructions per tile and wave).
  auto wait_tiles_but = [&](int n) {
    if (n >= 2) {
      if constexpr (NDMA == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else if (n == 1) {
      if constexpr (NDMA == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  // Transposed V read: 16-lane group gq reads keys 4*(gq>>1) + li/4 (+8), element
  // columns 32*db + 16*(gq&1) + 4*(li&3) .. +3.
  const int gq = lane >> 4, li = lane & 15;
  const int vkey = 4 * (gq >> 1) + (li >> 2);
  const int vcol = 16 * (gq & 1) + 4 * (li & 3);

  f32x16_t oacc[NCB][4];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[cb][db][e] = 0.f;
  float m_ref[NCB], l_part[NCB];   // reference max per row (base-2 units), row sum
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    m_ref[cb] = kNegInf;
    l_part[cb] = 0.f;
  }
  const float sl2 = p.scale_log2;

  const int ntiles = (kend + TK - 1) / TK;
  // Leading tiles that need no mask for any row of this wave; the remaining
  // ones (the diagonal, the ragged end, rows past R) are masked.
  const int n_clean = (rw0 + RPW <= R) ? min(kfull_w, L) / TK : 0;

  // Per-lane LDS byte offsets inside a tile (loop invariant, kept in
  // registers, opaque to the compiler so that every read is a base register
  // plus an immediate stage / key-step offset):
  //   K fragment of k-step ks: key c, chunk 2*ks + h;
  //   V fragments of d-block db: keys vkey (j = 0) and vkey + 8 (j = 1) of a
  //   16-key step, element columns 32*db + vcol .. + 3.
  // The offsets include the LDS address of the ring.
  uint32_t koff[8], voff[4][2];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    koff[ks] = smem_lds + (uint32_t)tile_off(c, 2 * ks + h);
    asm volatile("" : "+v"(koff[ks]));
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 32 * db + vcol;
      voff[db][j] = smem_lds + (uint32_t)(KT + tile_off(vkey + 8 * j, col >> 3) + (col & 7) * 2);
      asm volatile("" : "+v"(voff[db][j]));
    }
  typedef __attribute__((address_space(3))) const i32x4_t lds_i32x4_t;
  auto kread = [&](int stage, int ks) {  // K fragment: key c, 16-wide k-step ks
    return *reinterpret_cast<lds_i32x4_t*>((uintptr_t)(koff[ks] + (uint32_t)(stage * STAGE)));
  };
  // Masked scores are set to -inf.
  auto mask_scores = [&](f32x16_t* sc, int k0) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * h + (e & 3);
        const bool vis = key < L && (!p.causal || key <= qlim[cb]) && row_ok[cb];
        sc[cb][e] = vis ? sc[cb][e] : kNegInf;
      }
  };

  f32x16_t s_cur[NCB], s_nxt[NCB];
  float mt_cur[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) mt_cur[cb] = kNegInf;
  // Row max of a score tile in base-2 units (both lane halves hold the row);
  // IEEE maximum needs no NaN canonicalisation of the MFMA results.
  auto tile_max = [&](const f32x16_t& sc) {
    float m = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; e += 2) m = vmax(m, vmax(sc[e], sc[e + 1]));
    return m;
  };
  if (ntiles > 0) {
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (t < ntiles) dma_tile(t * TK, t);
    // Tiles 0 and 1 landed (step 0 reads K of tile 1); tile 2 may stay in flight.
    wait_tiles_but(ntiles >= 3 ? 1 : 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_cur[cb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s_cur[cb] = mfma32x32x16(as_bf16x8(kread(0, ks)), qf[cb][ks], s_cur[cb]);
    }
    if (n_clean == 0) mask_scores(s_cur, 0);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float m = tile_max(s_cur[cb]);
      mt_cur[cb] = vmax(m, __shfl_xor(m, 32, 64)) * sl2;
    }
  }

  // One key tile it (ring stage st = it & 3, a constant at every call site, so
  // all LDS addresses are a lane base plus an immediate), whose scores s_cur
  // are already masked and whose row maxes are mt_cur.  next: tile it + 1
  // exists; mask_next: it needs the mask.  Two phases, each a fixed
  // interleave pinned with scheduling barriers:
  //   1. the 8 * NCB MFMAs of S(it + 1) = K Q^T, each with the exponentials
  //      and bf16 packing of two scores of tile it; K fragments are read two
  //      k-steps ahead;
  //   2. the 8 * NCB MFMAs of O += V P(it), each with part of the max of tile
  //      it + 1; V fragments are read one pair ahead.
  auto step = [&](const int it, const int st, const bool next, const bool mask_next)
      __attribute__((always_inline)) {
    const int k0 = it * TK;
    if (it + 3 < ntiles) dma_tile(k0 + 3 * TK, (st + 3) & 3);

    // Lazy rescale: a row's reference max moves (and its accumulator and row
    // sum are rescaled) only when the row's max outgrows it by more than 2^8.
    bool grow = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) grow = grow || (mt_cur[cb] > m_ref[cb] + kRescaleThreshold);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float m_new = fmaxf(m_ref[cb], mt_cur[cb]);
        const float alpha = (m_ref[cb] == kNegInf) ? 0.f : fast_exp2(m_ref[cb] - m_new);
        l_part[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[cb][db] *= alpha;
        m_ref[cb] = m_new;
      }
    }
    float m_use[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) m_use[cb] = (m_ref[cb] == kNegInf) ? 0.f : m_ref[cb];

    // Phase 1: 8 * NCB MFMAs, 16 * NCB exponentials.
    constexpr int NG = 8 * NCB;
    uint32_t pk[NCB][8];
    const int kst_next = (st + 1) & 3;
    i32x4_t kf[3];
    if (next) {
      kf[0] = kread(kst_next, 0);
      kf[1] = kread(kst_next, 1);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_nxt[cb][e] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int ks = g / NCB, cb = g % NCB;
      if (next) {
        if (cb == 0 && ks + 2 < 8) kf[(ks + 2) % 3] = kread(kst_next, ks + 2);
        s_nxt[cb] = mfma32x32x16(as_bf16x8(kf[ks % 3]), qf[cb][ks], s_nxt[cb]);
      }
      const int pc = g >> 3, e = (2 * g) & 15;
      const float p0 = fast_exp2(__builtin_fmaf(s_cur[pc][e], sl2, -m_use[pc]));
      const float p1 = fast_exp2(__builtin_fmaf(s_cur[pc][e + 1], sl2, -m_use[pc]));
      pk[pc][e >> 1] = pack_bf16x2(p0, p1);
      // Row sum in fp32 from the unrounded exponentials (exact LSE).
      l_part[pc] += p0 + p1;
      __builtin_amdgcn_sched_barrier(0);
    }

    // Phase 2.
    // V fragments of (16-key step ts = pair >> 2, d-block pair & 3); a 16-key
    // step moves 16 rows, which the swizzle (a function of row mod 16) leaves alone.
    auto vread = [&](int pair, i32x2_t* out) {
      const int ts = pair >> 2, db = pair & 3;
      const uint32_t add = (uint32_t)(st * STAGE + 16 * ts * RB);
      out[0] = ds_read_tr_at(voff[db][0] + add);
      out[1] = ds_read_tr_at(voff[db][1] + add);
    };
    i32x2_t vf[2][2];
    vread(0, vf[0]);
    if (next && mask_next) mask_scores(s_nxt, k0 + TK);
    float mx[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) mx[cb] = kNegInf;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int pair = g / NCB, cb = g % NCB;
      const int ts = pair >> 2, db = pair & 3;
      if (cb == 0 && pair + 1 < 8) vread(pair + 1, vf[(pair + 1) & 1]);
      i32x4_t pb;
      pb[0] = (int)pk[cb][4 * ts + 0];
      pb[1] = (int)pk[cb][4 * ts + 1];
      pb[2] = (int)pk[cb][4 * ts + 2];
      pb[3] = (int)pk[cb][4 * ts + 3];
      i32x4_t va;
      va[0] = vf[pair & 1][0][0];
      va[1] = vf[pair & 1][0][1];
      va[2] = vf[pair & 1][1][0];
      va[3] = vf[pair & 1][1][1];
      oacc[cb][db] = mfma32x32x16(as_bf16x8(va), as_bf16x8(pb), oacc[cb][db]);
      const int sc = g >> 3;
      if (next) {
        const int ne = (2 * g) & 15;
        mx[sc] = vmax(mx[sc], vmax(s_nxt[sc][ne], s_nxt[sc][ne + 1]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (next) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        mt_cur[cb] = vmax(mx[cb], __shfl_xor(mx[cb], 32, 64)) * sl2;
        s_cur[cb] = s_nxt[cb];
      }
    }

    // Tile it + 2 must have landed before the next step reads its K; tile
    // it + 3 may stay in flight.  The barrier also frees stage st.
    wait_tiles_but(it + 3 < ntiles ? 1 : 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // A step whose ring stage is only known at run time.
  auto step_any = [&](const int it, const bool next, const bool mask_next)
      __attribute__((always_inline)) {
    switch (it & 3) {
      case 0: step(it, 0, next, mask_next); break;
      case 1: step(it, 1, next, mask_next); break;
      case 2: step(it, 2, next, mask_next); break;
      default: step(it, 3, next, mask_next); break;
    }
  };

  // Tiles below n_clean need no mask; step it masks tile it + 1 when that
  // tile needs it.  Every wave runs ntiles steps (one barrier each).  The
  // unmasked run starts at tile 0 and goes in groups of four (stages 0..3),
  // then a remainder of at most three with known stages.
  const int n1 = max(0, min(n_clean, ntiles - 1));
  const int clean_end = max(0, n1 - 1);
  int it = 0;
  for (; it + 4 <= clean_end; it += 4) {
    step(it, 0, true, false);
    step(it + 1, 1, true, false);
    step(it + 2, 2, true, false);
    step(it + 3, 3, true, false);
  }
  if (it < clean_end) step(it++, 0, true, false);
  if (it < clean_end) step(it++, 1, true, false);
  if (it < clean_end) step(it++, 2, true, false);
  for (; it < ntiles - 1; ++it) step_any(it, true, true);
  if (ntiles > 0) step_any(ntiles - 1, false, false);

  // Epilogue: O = U / l (division after the V-matmul), LSE = m + log l.
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float l_row = l_part[cb] + __shfl_xor(l_part[cb], 32, 64);
    if (!row_ok[cb]) continue;
    const int r = rw0 + 32 * cb + c;
    const int qh = kvh * G + (r % G);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const int64_t obase = (int64_t)b * p.os_b + (int64_t)qi[cb] * p.os_t + (int64_t)qh * p.os_h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * h;
        const float o0 = oacc[cb][db][4 * i + 0] * inv, o1 = oacc[cb][db][4 * i + 1] * inv;
        const float o2 = oacc[cb][db][4 * i + 2] * inv, o3 = oacc[cb][db][4 * i + 3] * inv;
        if (p.o_bf16) {
          uint2 pk2;
          pk2.x = pack_bf16x2(o0, o1);
          pk2.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.o) + obase + d) = pk2;
        } else {
          float4 v = make_float4(o0, o1, o2, o3);
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.o) + obase + d) = v;
        }
      }
    if (h == 0 && p.lse_out)
      p.lse_out[((int64_t)b * p.Lq + qi[cb]) * p.Hq + qh] =
          l_row > 0.f ? (m_ref[cb] + fast_log2(l_row)) * kLn2 : kNegInf;
  }
}

}  // namespace

template <int NW, int NCB>
hipError_t launch_variant(const KParams& p, int nrt, int64_t nwg, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_d128_kernel<NW, NCB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((prefill_d128_kernel<NW, NCB>), dim3((unsigned)nwg), dim3(NW * 64), LDS_BYTES,
                     s, p, nrt);
  return hipGetLastError();
}

hipError_t launch_prefill_d128(const KParams& p, hipStream_t s) {
  const int nrt = (p.rows + ROWS - 1) / ROWS;
  const int64_t nwg = (int64_t)p.B * p.Hkv * nrt;
  if (nwg == 0) return hipSuccess;
  return launch_variant<8, 1>(p, nrt, nwg, s);
}

}  // namespace attn

// Split-K MLA-style decode for bf16: one latent KV head, Dqk = 576, Dv = 512,
// V = the first 512 columns of K, up to 128 query rows (heads x queries) per
// KV head.
//
// One workgroup (8 waves, two per SIMD) owns one (split, KV head, request)
// unit, so every latent K row is read from HBM once per split and serves both
// contractions: the 576-wide QK^T and, through its first 512 columns, the PV.
// Wave w owns query rows 16w .. 16w + 15 outright: Q^T for the whole 576-wide
// contraction stays in registers for the split (loop-invariant, Cleave §6.1)
// and so does the fp32 accumulator O^T[512 x 16].  No partial result crosses
// waves, so the only barrier per tile is the one that hands a K tile over.
// Per 32-key tile and wave (16x16x32 bf16 MFMA, keys on the MFMA rows):
//   S^T[32 x 16]  = K[32 x 576] Q^T[576 x 16]      2 x 18 MFMA (two chains)
//   O^T[512 x 16] += V^T[512 x 32] P^T[32 x 16]    32 MFMA (32 accumulators)
// The two waves of a SIMD overlap one's softmax with the other's MFMAs.
//
// The running max is updated lazily: a row's reference max moves (and its
// accumulator and row sum are rescaled) only when the row's max grows by more
// than 2^8; otherwise P = 2^(s - m_ref) <= 256 is used as is.  Row sum and
// accumulator always share one reference, so O = U / l is unchanged.
//
// The K tile is copied HBM -> LDS by buffer loads that write LDS directly (no
// staging registers), four stages deep (three tiles in flight).  Key rows are
// stored unpadded (72 16-byte chunks) with the chunk index XOR-ed by the low
// bits of the key, which keeps both the 16-key A-operand reads of K and the
// transposed 4-key reads of V free of LDS bank conflicts.
#include "../attn_internal.hpp"
#include "common.hpp"
#include "layout.hpp"

namespace attn {
namespace {

constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int TK = kMlaTileN;          // 32 keys per tile
constexpr int DQK = 576, DV = 512;
constexpr int KSTEPS = DQK / 32;       // 18 k-steps of the QK contraction
constexpr int CBLK = DV / 16;          // 32 output column blocks
constexpr int CHUNKS = DQK / 8;        // 72 16-byte chunks per key row
constexpr int ROW_BYTES = CHUNKS * 16; // 1152
constexpr int HALF = 16 * ROW_BYTES;   // byte offset of key 16 in a stage
constexpr int STAGE = TK * ROW_BYTES;  // 36,864
constexpr int NSTAGE = 4;              // tiles it .. it + 3 resident
constexpr int LDS_BYTES = NSTAGE * STAGE;  // 147,456
constexpr int NBLK = TK * CHUNKS / 64;     // 36 one-KiB DMA blocks per tile
constexpr int BLK_ROUNDS = (NBLK + NW - 1) / NW;  // 5: waves 0-3 issue 5, waves 4-7 issue 4
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr int kFastMerge = 4;          // split counts the pipelined merge takes
static_assert(NBLK * 64 == TK * CHUNKS, "a tile is a whole number of DMA blocks");
static_assert(NBLK - (BLK_ROUNDS - 1) * NW == 4, "waves 0-3 own the last round");

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) const i32x4_t lds_i32x4_t;

// Physical 16-byte chunk of logical chunk c of key row `key` (within its row):
// c XOR (key & 7).  The XOR only touches the low three bits, so a chunk stays
// inside its aligned group of 8.  Measured on gfx950 with the exact per-lane
// address lists of both read patterns below, this layout runs the 16-key K
// fragment reads at the rate of lane-contiguous 16-byte reads and the
// transposed V reads at the rate of lane-contiguous transposed reads, while an
// unswizzled 1152-byte row runs both about 3x slower.
__device__ __forceinline__ int chunk_xor(int key) { return key & 7; }

__device__ __forceinline__ i32x2_t ds_read_tr_at(uint32_t lds_addr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)lds_addr);
  return __builtin_bit_cast(i32x2_t, v);
}
__device__ __forceinline__ i32x4_t ds_read16_at(uint32_t lds_addr) {
  return *reinterpret_cast<lds_i32x4_t*>((uintptr_t)lds_addr);
}
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Four consecutive output values of one row to O (bf16 or f32).
__device__ __forceinline__ void store_o4(const KParams& p, int64_t off, const f32x4_t& a) {
  if (p.o_bf16) {
    uint2 pk;
    pk.x = pack_bf16x2(a[0], a[1]);
    pk.y = pack_bf16x2(a[2], a[3]);
    uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + off;
    if ((reinterpret_cast<uintptr_t>(op) & 7) == 0) {
      *reinterpret_cast<uint2*>(op) = pk;
    } else {
      op[0] = (uint16_t)(pk.x & 0xffff);
      op[1] = (uint16_t)(pk.x >> 16);
      op[2] = (uint16_t)(pk.y & 0xffff);
      op[3] = (uint16_t)(pk.y >> 16);
    }
  } else {
    float* op = reinterpret_cast<float*>(p.o) + off;
    if ((reinterpret_cast<uintptr_t>(op) & 15) == 0) {
      *reinterpret_cast<f32x4_t*>(op) = a;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) op[e] = a[e];
    }
  }
}

// Every output row of (request b, KV head kvh) set to `val`, its LSE to `lse`.
__device__ void write_rows(const KParams& p, int b, int kvh, float val, float lse) {
  const f32x4_t v = {val, val, val, val};
  for (int e = threadIdx.x; e < p.rows * (DV / 4); e += NT) {
    const int r = e / (DV / 4), c = 4 * (e % (DV / 4));
    const int qi = r / p.G, qh = kvh * p.G + r % p.G;
    store_o4(p, (int64_t)b * p.os_b + (int64_t)qi * p.os_t + (int64_t)qh * p.os_h + c, v);
    if (c == 0 && p.lse_out) p.lse_out[((int64_t)b * p.Lq + qi) * p.Hq + qh] = lse;
  }
}

// PAGED: K rows come from a page pool (power-of-two page size).  The split's
// page ids are staged in LDS after the stages, and each lane copies its
// 16-byte slot with a 64-bit-addressed global load into LDS (same slot layout).
template <bool PAGED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mla_kernel(KParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int L = uniform(kv_len_b(p, b));
  const int lo = j * p.chunk;
  if (p.split_mode == 2) {
    // Single launch: split 0 answers for a request with no key (O = 0, LSE =
    // -inf), and for one longer than the plan covers (NaN rather than a
    // truncated result); no split of such a request counts an arrival.
    const int sb_all = (L + p.chunk - 1) / p.chunk;
    if (L == 0 || sb_all > p.s_max) {
      if (j == 0) write_rows(p, b, kvh, L == 0 ? 0.f : __builtin_nanf(""),
                             L == 0 ? kNegInf : __builtin_nanf(""));
      return;
    }
  }
  if (lo >= L) return;
  const int hi = min(lo + p.chunk, L);

  const int G = p.G;
  const int R = p.rows;
  const int li = lane & 15;   // query row within the wave (MFMA column)
  const int g = lane >> 4;    // 16-lane group
  const int r = 16 * w + li;
  const int qi = r / G;
  const int qh = kvh * G + r % G;
  const bool row_ok = r < R;
  const int qlim = qi + L - p.Lq;

  // Q^T as the B operand: lane holds Q[row r][32*ks + 8*g .. +7], ks = 0..17.
  bf16x8_t qf[KSTEPS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.qs_b +
                         (int64_t)qi * p.qs_t + (int64_t)qh * p.qs_h;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      i32x4_t v = {0, 0, 0, 0};
      if (row_ok) v = *reinterpret_cast<const i32x4_t*>(qp + 32 * ks + 8 * g);
      qf[ks] = as_bf16x8(v);
    }
    // Wait for Q here, once: otherwise the wait lands inside the loop and also
    // drains the K DMA in flight.
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)kvh * p.ks_h;
  if constexpr (!PAGED) kp += uniform(kv_base_off(p, b, p.ks_b, p.ks_t));
  const uint32_t kst = (uint32_t)(p.ks_t * 2);
  // The buffer range ends at this split's last key: rows past it read as zero.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, PAGED ? 0u : (uint32_t)hi * kst);
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem);

  // Paged: the ids of the pages holding keys [lo, hi) (lo < hi here), clamped
  // into the pool.  Slots past the split re-read key hi - 1 (masked).
  const int psh = PAGED ? p.page_shift : 0;
  const int pmask = (1 << psh) - 1;
  const int pg0 = lo >> psh;
  const int64_t kpage = p.ks_b * 2;  // bytes between pages
  int* page_ids = reinterpret_cast<int*>(smem + LDS_BYTES);
  if constexpr (PAGED) {
    const int n_ids = min(((hi - 1) >> psh) - pg0 + 1, kMlaPageIds);
    const int32_t* trow = p.page_table + (int64_t)b * p.ppr + pg0;
    for (int e = threadIdx.x; e < n_ids; e += NT) {
      const int pg = trow[e];
      page_ids[e] = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
    }
    __syncthreads();
  }

  // Tile copy, HBM -> LDS without registers (buffer_load ... lds): one wave
  // instruction fills one KiB of the stage, lane l the 16-byte slot 64*blk + l,
  // which holds physical chunk P % 72 of key P / 72 (P = the slot).  The whole
  // byte offset goes in the per-lane offset, which the buffer range check
  // covers.  The per-lane offsets are recomputed per tile (a few integer
  // instructions) rather than held in registers across the loop.
  const int nb = w < NBLK - (BLK_ROUNDS - 1) * NW ? BLK_ROUNDS : BLK_ROUNDS - 1;
  auto dma_tile = [&](int t, int stage) {
    const uint32_t base = smem_lds + (uint32_t)(stage * STAGE);
    const uint32_t toff = (uint32_t)(lo + t * TK) * kst;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if constexpr (PAGED) {
#pragma unroll
      for (int u = 0; u < BLK_ROUNDS; ++u) {
        if (u < BLK_ROUNDS - 1 || nb == BLK_ROUNDS) {
          const int P = 64 * (u * NW + w) + ln;
          const int key = P / CHUNKS;
          const int c = (P - key * CHUNKS) ^ chunk_xor(key);
          const int ka = min(lo + t * TK + key, hi - 1);
          const int pg = page_ids[(ka >> psh) - pg0];
          const char* src = reinterpret_cast<const char*>(kp) + (int64_t)pg * kpage +
                            (int64_t)(ka & pmask) * kst + 16 * c;
          const uint32_t m0v =
              __builtin_amdgcn_readfirstlane(base + (uint32_t)((u * NW + w) * 1024));
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                       :: "s"(m0v), "v"(src) : "memory", "m0");
        }
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < BLK_ROUNDS; ++u) {
      if (u < BLK_ROUNDS - 1 || nb == BLK_ROUNDS) {
        const int P = 64 * (u * NW + w) + ln;
        const int key = P / CHUNKS;
        const int c = (P - key * CHUNKS) ^ chunk_xor(key);
        const uint32_t m0v = base + (uint32_t)((u * NW + w) * 1024);
        const uint32_t voff = toff + (uint32_t)key * kst + 16u * (uint32_t)c;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m0v), "v"(voff), "s"(krs) : "memory", "m0");
      }
    }
  };
  // All DMA of a tile has landed once at most the `later` newer tiles'
  // instructions are outstanding (loads complete in order).
  auto wait_tiles_but = [&](int later) {
    if (later >= 2) {
      if (nb == 5) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else if (later == 1) {
      if (nb == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  // Per-lane LDS addresses (opaque to the compiler, so every read is one of
  // these plus an immediate).
  //   K fragment (key block kb, k-step ks): key 16*kb + li, logical chunk
  //   4*ks + g -> physical 4*(ks ^ x2) + (g ^ x01), x = chunk_xor(li) (the
  //   same for key 16 + li).
  //   Even ks: 64*ks + 64*x2; odd ks: 64*ks - 64*x2.
  const int xk = chunk_xor(li);
  const uint32_t k_lane = smem_lds + (uint32_t)(li * ROW_BYTES + 16 * (g ^ (xk & 3)));
  uint32_t k_even = k_lane + 64u * (uint32_t)(xk >> 2);
  uint32_t k_odd = k_lane - 64u * (uint32_t)(xk >> 2);
  //   V^T fragment (column block cb, key half kh): the 16-lane group g reads
  //   keys 16*kh + 4*g + (li >> 2), columns 16*cb + 4*(li & 3) .. + 3, i.e.
  //   logical chunk 2*cb + ((li >> 1) & 1), bytes 8*(li & 1) .. + 7; after the
  //   transpose lane li holds column 16*cb + li of keys 16*kh + 4*g + 0..3.
  //   Physical chunk 2*(cb ^ y1) + (((li >> 1) & 1) ^ y0), y = chunk_xor(key):
  //   one base per cb & 3, plus 128*(cb >> 2).
  const int vkey = 4 * g + (li >> 2);
  const int xv = chunk_xor(vkey);
  const uint32_t v_lane = smem_lds + (uint32_t)(vkey * ROW_BYTES + 16 * (((li >> 1) & 1) ^ (xv & 1)) +
                                                8 * (li & 1));
  uint32_t v_base[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) v_base[n] = v_lane + 32u * (uint32_t)(n ^ (xv >> 1));

  f32x4_t oacc[CBLK];
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;   // reference max of this lane's row (base-2 units)
  float l_part = 0.f;      // this lane's share of the row sum
  const float sl2 = p.scale_log2;
  const bool row_causal = p.causal != 0;
  const int ntiles = (hi - lo + TK - 1) / TK;

  // Operand fetches of a tile, in MFMA order: f = 0..35 the K fragments
  // (f = 2*ks + kb), f = 36..67 the V^T fragments (column block f - 36).  One
  // rolling window of FD fetches runs across the tile, so V is already in
  // flight during the softmax.  It stops at the tile's end: a window running
  // on into the next tile would need that tile landed one barrier earlier,
  // which leaves one tile fewer in flight (measured 2 % slower).
  constexpr int NF = 2 * KSTEPS + CBLK;  // 68
  constexpr int FD = 4;                  // fetches in flight (5 spills)
  auto fetch = [&](int f, uint32_t soff) -> i32x4_t {
    if (f < 2 * KSTEPS) {
      const int ks = f >> 1, kb = f & 1;
      return ds_read16_at((ks & 1 ? k_odd : k_even) + soff + (uint32_t)(kb * HALF + 64 * ks));
    }
    const int cb = f - 2 * KSTEPS;
    const uint32_t a = v_base[cb & 3] + soff + (uint32_t)(128 * (cb >> 2));
    const i32x2_t v0 = ds_read_tr_at(a);
    const i32x2_t v1 = ds_read_tr_at(a + HALF);
    i32x4_t va;
    va[0] = v0[0];
    va[1] = v0[1];
    va[2] = v1[0];
    va[3] = v1[1];
    return va;
  };

  // Prologue: tiles 0..2 in flight.
#pragma unroll
  for (int t = 0; t < NSTAGE - 1; ++t)
    if (t < ntiles) dma_tile(t, t);
  i32x4_t fr[NF];

  for (int it = 0; it < ntiles; ++it) {
    const int st = it & (NSTAGE - 1);
    const uint32_t soff = (uint32_t)(st * STAGE);
    // Hand-over: tile it has landed for every wave, and every wave has
    // finished tile it - 1 (its last reads fed the previous V-matmul), whose
    // stage the DMA of tile it + 3 now refills: three tiles stay in flight.
    wait_tiles_but(min(ntiles - it - 1, NSTAGE - 2));
    asm volatile("s_barrier" ::: "memory");
    if (it + NSTAGE - 1 < ntiles) dma_tile(it + NSTAGE - 1, (it + NSTAGE - 1) & (NSTAGE - 1));
#pragma unroll
    for (int f = 0; f < FD; ++f) fr[f] = fetch(f, soff);

    // S^T = K Q^T: two chains (key blocks).
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < 2 * KSTEPS; ++f) {
      fr[f + FD] = fetch(f + FD, soff);
      if (f & 1)
        s1 = mfma16x16x32(as_bf16x8(fr[f]), qf[f >> 1], s1);
      else
        s0 = mfma16x16x32(as_bf16x8(fr[f]), qf[f >> 1], s0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Softmax: lane holds keys k0 + 4*g + e (s0) and k0 + 16 + 4*g + e (s1).
    const int k0 = lo + it * TK;
    float sc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = s0[e];
      sc[4 + e] = s1[e];
    }
    const bool need_mask = (k0 + TK > hi) || (row_causal && k0 + TK - 1 > qlim) || !row_ok;
    if (__builtin_amdgcn_ballot_w64(need_mask) != 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = k0 + 16 * (e >> 2) + 4 * g + (e & 3);
        const bool vis = key < hi && (!row_causal || key <= qlim) && row_ok;
        sc[e] = vis ? sc[e] : kNegInf;
      }
    }
    float mx = vmax(vmax(vmax(sc[0], sc[1]), vmax(sc[2], sc[3])),
                    vmax(vmax(sc[4], sc[5]), vmax(sc[6], sc[7])));
    mx *= sl2;
    // Lazy rescale: move the reference only when some row's max outgrows it.
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleThreshold) != 0) {
      mx = vmax(mx, __shfl_xor(mx, 16, 64));
      mx = vmax(mx, __shfl_xor(mx, 32, 64));
      const float m_new = vmax(m_ref, mx);
      // On a row's first update the accumulator and sum are still zero.
      const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
      m_ref = m_new;
    }
    const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(__builtin_fmaf(sc[e], sl2, -m_use));
    l_part += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    // P^T as the B operand: k-slot 8*g + t <-> key 4*g + t (t < 4), 16 + 4*g + t - 4.
    i32x4_t pk;
    pk[0] = (int)pack_bf16x2(pv[0], pv[1]);
    pk[1] = (int)pack_bf16x2(pv[2], pv[3]);
    pk[2] = (int)pack_bf16x2(pv[4], pv[5]);
    pk[3] = (int)pack_bf16x2(pv[6], pv[7]);
    const bf16x8_t pb = as_bf16x8(pk);

    // O^T += V^T P^T.
#pragma unroll
    for (int f = 2 * KSTEPS; f < NF; ++f) {
      if (f + FD < NF) fr[f + FD] = fetch(f + FD, soff);
      const int cb = f - 2 * KSTEPS;
      oacc[cb] = mfma16x16x32(as_bf16x8(fr[f]), pb, oacc[cb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Split epilogue: O_j = U / l (fp32), LSE_j = (m_ref + log2 l) ln 2.  Lane
  // holds columns 16*cb + 4*g .. + 3 of row r.  The row's indices are
  // recomputed here rather than kept live across the loop.
  float l_row = l_part + __shfl_xor(l_part, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  int e_lane = threadIdx.x;
  asm volatile("" : "+v"(e_lane));
  const int e_r = 16 * w + (e_lane & 15), e_g = (e_lane >> 4) & 3;
  const bool e_ok = e_r < R;
  const int e_qi = e_r / G, e_qh = kvh * G + e_r % G;
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  const float lse_own = l_row > 0.f ? (m_ref + fast_log2(l_row)) * kLn2 : kNegInf;
  const int64_t nrows = (int64_t)p.B * p.Lq * p.Hq;
  const int64_t row = ((int64_t)b * p.Lq + e_qi) * p.Hq + e_qh;
  const int64_t obase = (int64_t)b * p.os_b + (int64_t)e_qi * p.os_t + (int64_t)e_qh * p.os_h + 4 * e_g;
  const int sb = (L + p.chunk - 1) / p.chunk;  // splits of this request (>= 1 here)

  if (p.split_mode == 1) {  // partial for the combine kernel
    if (e_ok) {
      float* dst = p.ws_o + ((int64_t)j * nrows + row) * DV + 4 * e_g;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb)
        *reinterpret_cast<f32x4_t*>(dst + 16 * cb) = oacc[cb] * inv;
      if (e_g == 0) p.ws_lse[(int64_t)j * nrows + row] = lse_own;
    }
    return;
  }
  if (sb == 1) {  // the whole request in one split: O directly
    if (e_ok) {
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) store_o4(p, obase + 16 * cb, oacc[cb] * inv);
      if (e_g == 0 && p.lse_out) p.lse_out[row] = lse_own;
    }
    return;
  }

  // Single-launch merge (the combine of Cleave §4 inside the split kernel).
  // The (request, KV head) counter holds tickets in its low 16 bits and
  // published partials in its high 16 bits.  Every split takes a ticket when
  // its keys are done; all but the last publish their partial and count it;
  // the last one (whose ticket is sb - 1) knows that every other split has
  // already taken its ticket, so it is resident and only has its stores left:
  // it waits for their count, then merges all sb partials in split order
  // (its own from registers, with the same arithmetic as a stored one, so the
  // result is the same bits whichever split comes last) and resets the
  // counter.
  //
  // The partials of this mode are private to the kernel and kept in its lane
  // order: split j of unit u is a block of ceil(R / 16) wave slabs, slab w
  // holding for each column block cb the 64 lanes' four values (1 KiB, one
  // store or load instruction of whole cache lines), plus one LSE per row.
  // With at most kFastMerge splits they are stored as bf16 (round to nearest
  // even), the lane's values of column blocks 2q and 2q + 1 side by side in
  // one 16-byte slot of 1 KiB row q: the splits of every request finish
  // together, so the partial traffic (written, then read back by the merging
  // split) is not hidden behind other work and halving it shortens the
  // launch's tail.  The merging split rounds its own partial the same way.
  //
  // Ordering on gfx950: partials are written with sc1 (device-coherent)
  // stores, which write through the XCD's L2 instead of leaving dirty lines
  // there, and each wave waits for them (vmcnt(0)) before the workgroup
  // barrier that precedes the counting atomic; the reader's loads are sc1
  // too, so they are served from the device-coherent level, never from a
  // stale line of its own L2.  Because no data is left dirty in an L2, the
  // whole-L2 write-back a device-scope release fence would add is not
  // needed.
  int* s_ticket = reinterpret_cast<int*>(smem);
  const int unit = b * p.Hkv + kvh;
  int* cnt = p.counters + unit;
  __syncthreads();
  if (threadIdx.x == 0)
    *s_ticket = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xffff;
  __syncthreads();
  const int ticket = *s_ticket;
  const int nslab = (R + 15) >> 4;                       // wave slabs per block
  const int64_t nunits = (int64_t)p.B * p.Hkv;
  const uint32_t slab_bytes = CBLK * 64 * 16;            // 32 KiB
  const uint32_t block_bytes = (uint32_t)nslab * slab_bytes;
  // Buffer over the whole partial area; byte offset of (split jj, this lane, cb).
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.ws_o, 0xffffffffu);
  const uint32_t lane_off = (uint32_t)w * slab_bytes + (uint32_t)lane * 16;
  auto part_off = [&](int jj, int cb) {
    return (uint32_t)(((int64_t)jj * nunits + unit) * block_bytes) + lane_off +
           (uint32_t)(cb * 64 * 16);
  };
  auto lse_ptr = [&](int jj) { return p.ws_lse + ((int64_t)jj * nunits + unit) * (nslab * 16) + e_r; };
  // bf16 partials: byte offset of (split jj, this lane, column blocks 2q,
  // 2q + 1).  They fill the first half of the same per-(split, unit) blocks
  // as fp32 ones, since requests with more splits share the area in fp32.
  const bool half_parts = sb <= kFastMerge;
  const uint32_t lane_off16 = (uint32_t)w * (slab_bytes / 2) + (uint32_t)lane * 16;
  auto part16_off = [&](int jj, int q) {
    return (uint32_t)(((int64_t)jj * nunits + unit) * block_bytes) + lane_off16 +
           (uint32_t)(q * 64 * 16);
  };
  // Column blocks 2q and 2q + 1 of this split's O_j, rounded to bf16 and packed.
  auto own16 = [&](int q) {
    const f32x4_t a = oacc[2 * q] * inv, c = oacc[2 * q + 1] * inv;
    i32x4_t v;
    v[0] = (int)pack_bf16x2(a[0], a[1]);
    v[1] = (int)pack_bf16x2(a[2], a[3]);
    v[2] = (int)pack_bf16x2(c[0], c[1]);
    v[3] = (int)pack_bf16x2(c[2], c[3]);
    return v;
  };
  if (ticket < sb - 1) {
    if (w < nslab) {
      if (half_parts) {
#pragma unroll
        for (int q = 0; q < CBLK / 2; ++q)
          store16_dev(wrs, part16_off(j, q), __builtin_bit_cast(f32x4_t, own16(q)));
      } else {
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) store16_dev(wrs, part_off(j, cb), oacc[cb] * inv);
      }
      if (e_g == 0) store_dev(lse_ptr(j), lse_own);
    }
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(cnt, 1 << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (threadIdx.x == 0) {
    while ((__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 16) < sb - 1)
      __builtin_amdgcn_s_sleep(2);
  }
  __syncthreads();
  if (w < nslab && half_parts) {
    // Up to four splits: every load of the merge is issued ahead of its use.
    // The LSEs first (one round trip; a split index past sb is clamped to a
    // slot inside the area and its value dropped), then the other splits'
    // bf16 partials, MD steps of two column blocks ahead.
    float lb[kFastMerge];
#pragma unroll
    for (int jj = 0; jj < kFastMerge; ++jj) lb[jj] = load_dev(lse_ptr(min(jj, sb - 1)));
    int jo[kFastMerge - 1];  // the other splits in split order
#pragma unroll
    for (int k = 0; k < kFastMerge - 1; ++k) jo[k] = min(k < j ? k : k + 1, sb - 1);
    constexpr int MCB = 2, MD = 4, NSTEP = CBLK / MCB;
    i32x4_t xb[MD][kFastMerge - 1];
    auto issue = [&](int step, int slot) {
#pragma unroll
      for (int k = 0; k < kFastMerge - 1; ++k)
        xb[slot][k] = __builtin_bit_cast(i32x4_t, load16_dev(wrs, part16_off(jo[k], step)));
    };
    // Values 4u .. 4u + 3 of a packed slot (column block 2q + u) as fp32.
    auto unpack = [](const i32x4_t& v, int u) {
      f32x4_t r;
      r[0] = __builtin_bit_cast(float, (uint32_t)v[2 * u] << 16);
      r[1] = __builtin_bit_cast(float, (uint32_t)v[2 * u] & 0xffff0000u);
      r[2] = __builtin_bit_cast(float, (uint32_t)v[2 * u + 1] << 16);
      r[3] = __builtin_bit_cast(float, (uint32_t)v[2 * u + 1] & 0xffff0000u);
      return r;
    };
#pragma unroll
    for (int st = 0; st < MD; ++st) issue(st, st);
    // Pass 1: the common reference M (base 2), the weights and their sum in
    // split order.
#pragma unroll
    for (int jj = 0; jj < kFastMerge; ++jj)
      lb[jj] = jj >= sb ? kNegInf : (jj == j ? lse_own : lb[jj]) * kLog2e;
    float M2 = kNegInf;
#pragma unroll
    for (int jj = 0; jj < kFastMerge; ++jj) M2 = vmax(M2, lb[jj]);
    float wt[kFastMerge];
    float wsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < kFastMerge; ++jj) {
      wt[jj] = M2 == kNegInf ? 0.f : fast_exp2(lb[jj] - M2);
      wsum += wt[jj];
    }
    const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
    // Pass 2: two column blocks per step, the splits in order (this split's
    // own partial from registers, rounded as a stored one).
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      const int slot = step % MD;
      const i32x4_t own_pk = own16(step);
#pragma unroll
      for (int u = 0; u < MCB; ++u) {
        const int cb = MCB * step + u;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < kFastMerge; ++jj) {
          const i32x4_t xp = jj == j ? own_pk
                                     : (jj < j ? xb[slot][jj < kFastMerge - 1 ? jj : 0]
                                               : xb[slot][jj > 0 ? jj - 1 : 0]);
          const f32x4_t xv = unpack(xp, u);
          const f32x4_t t = acc + wt[jj] * xv;
          acc = jj < sb ? t : acc;
        }
        if (e_ok) store_o4(p, obase + 16 * cb, acc * winv);
      }
      if (step + MD < NSTEP) issue(step + MD, slot);
    }
    if (e_ok && e_g == 0 && p.lse_out)
      p.lse_out[row] = M2 == kNegInf ? kNegInf : (M2 + fast_log2(wsum)) * kLn2;
  } else if (w < nslab) {
    // Pass 1: the common reference M (base 2) and the weight sum, split order.
    float M2 = kNegInf;
    for (int jj = 0; jj < sb; ++jj) {
      const float lj = jj == j ? lse_own : load_dev(lse_ptr(jj));
      M2 = vmax(M2, lj * kLog2e);
    }
    float wsum = 0.f;
    if (M2 != kNegInf) {
      for (int jj = 0; jj < sb; ++jj) {
        const float lj = jj == j ? lse_own : load_dev(lse_ptr(jj));
        wsum += fast_exp2(lj * kLog2e - M2);
      }
    }
    const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
    // Pass 2: four column blocks at a time, the splits in order; the loads of
    // up to four splits are issued together.
    constexpr int CB = 4, MB = 4;
#pragma unroll
    for (int c0 = 0; c0 < CBLK; c0 += CB) {
      f32x4_t acc[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (M2 != kNegInf) {
        for (int j0 = 0; j0 < sb; j0 += MB) {
          f32x4_t x[MB][CB];
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int u = 0; u < CB; ++u)
              x[m][u] = (j0 + m < sb && j0 + m != j) ? load16_dev(wrs, part_off(j0 + m, c0 + u))
                                                     : oacc[c0 + u] * inv;
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            if (j0 + m < sb) {
              const float lj = j0 + m == j ? lse_own : load_dev(lse_ptr(j0 + m));
              const float wj = fast_exp2(lj * kLog2e - M2);
#pragma unroll
              for (int u = 0; u < CB; ++u) acc[u] += wj * x[m][u];
            }
          }
        }
      }
      if (e_ok) {
#pragma unroll
        for (int u = 0; u < CB; ++u) store_o4(p, obase + 16 * (c0 + u), acc[u] * winv);
      }
    }
    if (e_ok && e_g == 0 && p.lse_out)
      p.lse_out[row] = M2 == kNegInf ? kNegInf : (M2 + fast_log2(wsum)) * kLn2;
  }
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool PAGED>
hipError_t launch_mla_variant(const KParams& p, dim3 grid, hipStream_t s) {
  constexpr int lds = LDS_BYTES + (PAGED ? 4 * kMlaPageIds : 0);
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&decode_mla_kernel<PAGED>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_mla_kernel<PAGED>, grid, dim3(NT), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mla(const KParams& p, dim3 grid, hipStream_t s) {
  if (p.page_table) return launch_mla_variant<true>(p, grid, s);
  return launch_mla_variant<false>(p, grid, s);
}

}  // namespace attn

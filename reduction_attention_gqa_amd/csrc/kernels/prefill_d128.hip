// Fused causal / non-causal GQA prefill for bf16, Dqk = Dv = 128.
//
// One workgroup (8 waves) computes one 256-row tile of one (request, KV head)
// group; a row is a (query position, head of the group) pair, so the G query
// heads that share a KV head share every K/V tile staged in LDS.  This is the
// inter-threadblock output tiling of Cleave §5.1 / §5.3 ([b_O, d] output tiles,
// one per workgroup) with GQA packing added.  Inside, the key axis is tiled
// (iterative tiling, §5.1 and §5.3); the exp tile feeds both the row sum and
// the V-matmul in the same step (horizontal fusion, §5.1); the division by the
// row sum comes after the V-matmul (§2.2, Fig. 2); the Q tile is loaded once,
// outside the key loop (§6.1).
//
// Each wave owns 32 rows (one MFMA column block); two waves share a SIMD.
// Per wave and tile of TK = 32 * KB keys, keys on the MFMA rows:
//   S^T[TK x 32]  = K[TK x 128] Q^T[128 x 32]     KB x 8 MFMA 32x32x16 bf16
//   O^T[128 x 32] += V^T[128 x TK] P^T[TK x 32]   KB x 8 MFMA 32x32x16 bf16
// Within a wave, the scores of tile i + 1 are computed under the
// exponentials of tile i, and the V-matmul of tile i under the max of tile
// i + 1 (fixed interleaves pinned with scheduling barriers).
//
// The running max is updated lazily: a row's reference max moves (and its
// accumulator and row sum are rescaled) only when the row's max grows by more
// than 2^8; otherwise P = 2^(s - m_ref) <= 256 is used as is.  Row sum and
// accumulator always share one reference, so O = U / l is unchanged.
//
// K/V tiles go HBM -> LDS by buffer loads that write LDS directly, into an
// NS-stage K ring and an NS-stage V ring; the workgroup meets at a barrier
// once per group of BAR tiles, which publishes the next group's tiles and
// frees the group's stages.  Contiguous caches: 64-key tiles (KB = 2), NS =
// 4, a barrier per tile (the tile, the next one and two in flight); against
// 32-key tiles with NS = 6 and a barrier per two tiles (the same keys per
// barrier, 128 keys in flight instead of 192) this measured about 2 %
// faster on both causal attention and MatMul+MatMul, and NS = 5 (all of the
// LDS) slower.  Paged pools keep the 32-key tiles, NS = 6, BAR = 2: their
// per-lane copy moves one block per wave.  A tile row is 256 bytes, and the 16-byte chunk c of
// row r sits at chunk c ^ swz(r), which keeps both the K operand reads (16
// keys, one chunk each) and the transposed V reads (4 keys, 4 chunks each)
// free of bank conflicts.  Every LDS read is a per-lane base register plus an
// immediate (stage, key block, key step).
//
// SOFTMAX = false gives MatMul+MatMul (Cleave §7.3 subgraph list, the two
// consecutive reductions without the softmax between them): the scores times
// tau (KParams::scale_log2 then carries tau itself) are the intermediate, a
// hidden key contributes 0, and O = U; the intermediate still lives one key
// tile at a time in registers (iterative tiling, §5.1 / §5.3).
//
// Causal tiles beyond a tile's diagonal are never loaded; masking runs only on
// tiles that straddle the diagonal or the end of the keys.  Workgroups are
// issued heaviest first: when the group count allows, each XCD owns a fixed
// set of (request, KV head) groups and works through them two at a time
// (their K/V, 4 MB at D = 128 and 4096 keys, stays in that XCD's L2), taking
// the pair's row tiles in order of decreasing key count; the causal row
// tiles then balance over its compute units better than one group at a
// time (about 1 % on the causal workload; interleaving all four groups of
// an XCD gains a little more but doubles the K/V fetched from HBM).
#include "../attn_internal.hpp"
#include "common.hpp"
#include "layout.hpp"

namespace attn {
namespace {

constexpr int NW = 8;                 // waves per workgroup
constexpr int NT = NW * 64;
constexpr int ROWS = NW * 32;         // rows per workgroup
constexpr int RB = 256;               // bytes per K or V row (128 bf16)
constexpr float kRescaleThreshold = 8.0f;  // log2 units

constexpr int lds_bytes(int kb, int ns) { return 2 * ns * 32 * kb * RB; }

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) const i32x4_t lds_i32x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 8 bytes addressed by lanes 4e + i / 4 (e = 0..3) as its element e.
__device__ __forceinline__ i32x2_t ds_read_tr_at(uint32_t lds_addr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)lds_addr);
  return __builtin_bit_cast(i32x2_t, v);
}
__device__ __forceinline__ i32x4_t ds_read16_at(uint32_t lds_addr) {
  return *reinterpret_cast<lds_i32x4_t*>((uintptr_t)lds_addr);
}

// Chunk swizzle: swap the two 2-bit fields of r mod 16.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// IEEE-754 2019 maximum (v_maximum3_f32): no canonicalisation of its inputs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// Combine lane l with lane l ^ 32 (the two lanes of a row) with gfx950's
// v_permlane32_swap: a VALU exchange instead of an LDS-unit permute.  With both
// operands equal, the two results are the lower and the upper lane's value.
__device__ __forceinline__ f32x2_t row_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2_t{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float row_max(float v) { const f32x2_t h = row_halves(v); return vmax(h[0], h[1]); }
__device__ __forceinline__ float row_sum(float v) { const f32x2_t h = row_halves(v); return h[0] + h[1]; }
// Byte offset of (row, 16-byte chunk c) inside a K or V tile.
__device__ __forceinline__ int tile_off(int row, int c) { return row * RB + 16 * (c ^ swz(row)); }

// KB key blocks of 32 per tile; NS ring stages; BAR tiles per barrier group,
// whose successors' copies are issued when the group starts.  PAGED: K/V rows come from a page pool (power-of-two
// page size); the request's page ids are staged in LDS after the rings and
// each lane copies its row with a 64-bit-addressed global load into LDS.
template <int KB, int NS, int BAR, bool PAGED, bool SOFTMAX>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_d128_kernel(KParams p, int nrt) {
  constexpr int TK = 32 * KB;         // keys per tile
  constexpr int KT = TK * RB;         // bytes of one K (or V) tile
  constexpr int VRING = NS * KT;      // the V ring follows the K ring
  constexpr int LOOK = NS - BAR;      // DMA lookahead in tiles
  // A group reads tiles g .. g + BAR and the next one up to g + 2 BAR; stage
  // arithmetic is compile-time only when groups tile the ring.
  static_assert(BAR >= 1 && NS % BAR == 0 && NS >= 2 * BAR + 1, "ring stages per barrier group");
  constexpr int NDMA = KB;            // 1 KiB DMA blocks per wave per K (or V) tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Workgroup -> (group, row tile): heaviest row tiles first, over pairs of
  // an XCD's groups.
  const int ngroups = p.B * p.Hkv;
  const int id = blockIdx.x;
  int group, rt;
  if ((ngroups & 7) == 0) {
    const int xcd = id & 7, k = id >> 3;
    const int gpx = ngroups >> 3;  // groups per XCD
    if ((gpx & 1) == 0) {
      // Two groups at a time, their row tiles interleaved heaviest first.
      const int pr = k / (2 * nrt), kk = k - pr * 2 * nrt;
      group = xcd + 8 * (2 * pr + (kk & 1));
      rt = nrt - 1 - (kk >> 1);
    } else {
      group = xcd + 8 * (k / nrt);
      rt = nrt - 1 - (k % nrt);
    }
  } else {
    group = id / nrt;
    rt = nrt - 1 - (id % nrt);
  }
  const int b = group / p.Hkv;
  const int kvh = group % p.Hkv;
  const int L = uniform(kv_len_b(p, b));
  const int Lqb = uniform(q_len_b(p, b));  // query rows of this request (packed queries: ragged)
  const int G = p.G;
  const int R = Lqb * G;           // rows of this request
  const int r0 = rt * ROWS;
  if (r0 >= R) return;             // a row tile past this request's queries
  const int off = L - Lqb;         // causal: row position i sees keys <= i + off

  // This wave's rows: lane (c, h) holds row rw0 + c.
  const int c = lane & 31;
  const int h = lane >> 5;
  const int rw0 = r0 + 32 * w;
  const int r = rw0 + c;
  const int qi = r / G;
  const bool row_ok = r < R;
  const int qlim = qi + off;       // last visible key of this row (causal)
  const int wg_rows = max(0, min(ROWS, R - r0));
  int kend = L;                    // keys [0, kend) are visible to some row of the workgroup
  if (p.causal) kend = min(L, (r0 + wg_rows - 1) / G + off + 1);
  kend = max(kend, 0);
  // Keys below kfull_w are visible to every row of this wave.
  const int kfull_w = p.causal ? max(0, min(L, rw0 / G + off + 1)) : L;

  // Q^T as the B operand (hoisted): lane holds Q[row r][16*ks + 8*h .. +7].
  bf16x8_t qf[8];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
    const int qh = kvh * G + (r % G);
    const int64_t qoff = q_row_off(p, b, qi) + (int64_t)qh * p.qs_h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      i32x4_t v = {0, 0, 0, 0};
      if (row_ok) v = *reinterpret_cast<const i32x4_t*>(qp + qoff + 16 * ks + 8 * h);
      qf[ks] = as_bf16x8(v);
    }
    // Wait for Q here, once, rather than at the loop head on every tile.
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  // Tile copy HBM -> LDS without registers: each wave fills rows
  // 4*(NDMA*w + u) .. + 3 (u < NDMA) of the K tile and of the V tile; lane l
  // writes the 16-byte slot (row 4*(NDMA*w+u) + l/16, position l%16), which
  // holds chunk (l%16) ^ swz(row).  The buffer ranges end at the last key, so
  // rows past it are zero.
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)kvh * p.ks_h;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)kvh * p.vs_h;
  if constexpr (!PAGED) {
    kp += uniform(kv_base_off(p, b, p.ks_b, p.ks_t));
    vp += uniform(kv_base_off(p, b, p.vs_b, p.vs_t));
  }
  const uint32_t kst = (uint32_t)(p.ks_t * 2), vst = (uint32_t)(p.vs_t * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, PAGED ? 0u : (uint32_t)L * kst);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, PAGED ? 0u : (uint32_t)L * vst);

  // Paged: keys [0, kload) are the ones any tile copy reads; tile rows past
  // kload re-read key kload - 1 (masked, zero probability).  The ids of their
  // pages go to LDS after the K/V rings, clamped into the pool.
  const int ntiles = (kend + TK - 1) / TK;
  const int kload = min(L, ntiles * TK);
  const int psh = PAGED ? p.page_shift : 0;
  const int pmask = (1 << psh) - 1;
  int* page_ids = reinterpret_cast<int*>(smem + 2 * NS * KT);
  if constexpr (PAGED) {
    const int n_ids = kload > 0 ? min(((kload - 1) >> psh) + 1, kPrefillPageIds) : 0;
    const int32_t* trow = p.page_table + (int64_t)b * p.ppr;
    for (int e = threadIdx.x; e < n_ids; e += NT) {
      const int pg = trow[e];
      page_ids[e] = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
    }
    __syncthreads();
  }
  const int dma_row = 4 * w + (lane >> 4);  // this lane's row of a tile copy (NDMA == 1)
  const int dma_chunk = (lane & 15) ^ swz(dma_row);
  const int64_t kpage = p.ks_b * 2, vpage = p.vs_b * 2;  // bytes between pages
  auto page_of_tile = [&](int k0) { return page_ids[min(k0 + dma_row, kload - 1) >> psh]; };
  int pg_next = (PAGED && ntiles > 0) ? page_of_tile(0) : 0;
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
    if constexpr (PAGED) {
      // Tiles are copied in order; the page of this one was read from LDS
      // when the previous copy was issued.
      const int key = min(k0 + dma_row, kload - 1);
      const int64_t in_page = (int64_t)(key & pmask);
      const char* ka = reinterpret_cast<const char*>(kp) + (int64_t)pg_next * kpage +
                       in_page * kst + 16 * dma_chunk;
      const char* va = reinterpret_cast<const char*>(vp) + (int64_t)pg_next * vpage +
                       in_page * vst + 16 * dma_chunk;
      const uint32_t m0k = __builtin_amdgcn_readfirstlane(smem_lds + (uint32_t)(stage * KT + w * 1024));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(m0k), "v"(ka) : "memory", "m0");
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(m0k + VRING), "v"(va) : "memory", "m0");
      pg_next = page_of_tile(k0 + TK);
      return;
    }
    const uint32_t ksoff = (uint32_t)k0 * kst, vsoff = (uint32_t)k0 * vst;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
      const uint32_t m0k = smem_lds + (uint32_t)(stage * KT + (NDMA * w + u) * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(m0k), "v"(k_voff[u] + ksoff), "s"(krs) : "memory", "m0");
      const uint32_t m0v = m0k + VRING;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(m0v), "v"(v_voff[u] + vsoff), "s"(vrs) : "memory", "m0");
    }
  };
  // s_waitcnt: all but the newest n tiles' DMA has landed (loads complete in
  // order; 2 * NDMA instructions per tile and wave).
  static_assert(NDMA == 1 || !PAGED, "a paged copy moves one block per wave and tensor");
  static_assert(12 * NDMA <= 63, "vmcnt range");
  auto wait_tiles_but = [&](int n) {
    switch (n) {
      case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * NDMA) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(4 * NDMA) : "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(6 * NDMA) : "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(8 * NDMA) : "memory"); break;
      case 5: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(10 * NDMA) : "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(12 * NDMA) : "memory"); break;
    }
  };

  // Per-lane LDS addresses (loop invariant, kept in registers, opaque to the
  // compiler so that every read is this base plus an immediate):
  //   K fragment of k-step ks: key c of a 32-key block, chunk 2*ks + h;
  //   V fragments of d-block db: 16-lane group gq reads keys vkey (j = 0) and
  //   vkey + 8 (j = 1) of a 16-key step, element columns 32*db + vcol .. + 3.
  // Key blocks and 16-key steps move whole multiples of 16 rows, which the
  // swizzle (a function of row mod 16) leaves alone.
  const int gq = lane >> 4, li = lane & 15;
  const int vkey = 4 * (gq >> 1) + (li >> 2);
  const int vcol = 16 * (gq & 1) + 4 * (li & 3);
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
      voff[db][j] = smem_lds + (uint32_t)(VRING + tile_off(vkey + 8 * j, col >> 3) + (col & 7) * 2);
      asm volatile("" : "+v"(voff[db][j]));
    }
  auto kread = [&](int stage, int kb, int ks) {
    return ds_read16_at(koff[ks] + (uint32_t)(stage * KT + kb * 32 * RB));
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_ref = kNegInf;   // reference max of this lane's row (base-2 units)
  float l_part = 0.f;
  const float sl2 = p.scale_log2;

  // Leading tiles that need no mask for any row of this wave; the remaining
  // ones (the diagonal, the ragged end, rows past R) are masked.
  const int n_clean = (rw0 + 32 <= R) ? min(kfull_w, L) / TK : 0;

  // Masked scores are set to -inf (0 without the softmax).  Lane element e of key block kb is key
  // k0 + 32*kb + 8*(e/4) + 4*h + e%4.
  auto mask_scores = [&](f32x16_t* sc, int k0) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3);
        const bool vis = key < L && (!p.causal || key <= qlim) && row_ok;
        sc[kb][e] = vis ? sc[kb][e] : (SOFTMAX ? kNegInf : 0.f);
      }
  };
  // Row max of a score tile in base-2 units (both lane halves hold the row);
  // IEEE maximum needs no NaN canonicalisation of the MFMA results.
  auto tile_max = [&](const f32x16_t* sc) {
    float m = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) m = vmax(m, vmax(sc[kb][e], sc[kb][e + 1]));
    return row_max(m) * sl2;
  };

  f32x16_t s_cur[KB], s_nxt[KB];
  float mt_cur = kNegInf;
  if (ntiles > 0) {
#pragma unroll
    for (int t = 0; t < LOOK; ++t)
      if (t < ntiles) dma_tile(t * TK, t);
    // Tiles 0 .. BAR landed (steps 0 .. BAR - 1 read K of tiles 1 .. BAR);
    // later ones may stay in flight.
    wait_tiles_but(max(0, min(LOOK - 1, ntiles - 1) - BAR));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_cur[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s_cur[kb] = mfma32x32x16(as_bf16x8(kread(0, kb, ks)), qf[ks], s_cur[kb]);
    }
    if (n_clean == 0) mask_scores(s_cur, 0);
    if constexpr (SOFTMAX) mt_cur = tile_max(s_cur);
  }

  // One key tile it (ring stage st = it % NS, a constant at every call site),
  // whose scores s_cur are already masked and whose row max is mt_cur.  next:
  // tile it + 1 exists; mask_next: it needs the mask.  Two phases, each a
  // fixed interleave pinned with scheduling barriers:
  //   1. the 8 * KB MFMAs of S(it + 1) = K Q^T (key blocks alternate, so
  //      consecutive MFMAs are independent), each with the exponentials, bf16
  //      packing and row sum of two scores of tile it; K fragments are read
  //      three MFMAs ahead;
  //   2. the 8 * KB MFMAs of O += V P(it), each with part of the max of tile
  //      it + 1; V fragments are read two MFMAs ahead (one fewer ahead in
  //      either phase measured about 1 % slower).
  auto step = [&](const int it, const int st, const bool next, const bool mask_next)
      __attribute__((always_inline)) {
    const int k0 = it * TK;
    // A group of BAR steps starts: copy its successors' tiles it + LOOK ..
    // it + LOOK + BAR - 1 into the stages of tiles it - BAR .. it - 1, which
    // every wave finished with before the barrier that ended the last group.
    if (st % BAR == 0) {
#pragma unroll
      for (int j = 0; j < BAR; ++j)
        if (it + LOOK + j < ntiles) dma_tile(k0 + (LOOK + j) * TK, (st + LOOK + j) % NS);
    }

    // Lazy rescale (rare).
    if (SOFTMAX && __builtin_amdgcn_ballot_w64(mt_cur > m_ref + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m_ref, mt_cur);
      const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      m_ref = m_new;
    }
    const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;

    // Phase 1.
    constexpr int NG = 8 * KB;
    uint32_t pk[KB][8];
    const int kst_next = (st + 1) % NS;
    i32x4_t kf[4];
    if (next) {
      kf[0] = kread(kst_next, 0 % KB, 0 / KB);
      kf[1] = kread(kst_next, 1 % KB, 1 / KB);
      kf[2] = kread(kst_next, 2 % KB, 2 / KB);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_nxt[kb][e] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (next) {
        if (g + 3 < NG) kf[(g + 3) % 4] = kread(kst_next, (g + 3) % KB, (g + 3) / KB);
        s_nxt[g % KB] = mfma32x32x16(as_bf16x8(kf[g % 4]), qf[g / KB], s_nxt[g % KB]);
      }
      const int pc = g >> 3, e = (2 * g) & 15;
      if constexpr (SOFTMAX) {
        const float p0 = fast_exp2(__builtin_fmaf(s_cur[pc][e], sl2, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s_cur[pc][e + 1], sl2, -m_use));
        pk[pc][e >> 1] = pack_bf16x2(p0, p1);
        l_part += p0 + p1;  // row sum from the unrounded exponentials (exact LSE)
      } else {
        pk[pc][e >> 1] = pack_bf16x2(s_cur[pc][e] * sl2, s_cur[pc][e + 1] * sl2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Phase 2: MFMA g is 16-key step ts = g / 4 and d-block db = g % 4.
    auto vread = [&](int g, i32x2_t* out) {
      const uint32_t add = (uint32_t)(st * KT + 16 * (g >> 2) * RB);
      out[0] = ds_read_tr_at(voff[g & 3][0] + add);
      out[1] = ds_read_tr_at(voff[g & 3][1] + add);
    };
    i32x2_t vf[3][2];
    vread(0, vf[0]);
    vread(1, vf[1]);
    if (next && mask_next) mask_scores(s_nxt, k0 + TK);
    float mx = kNegInf;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int ts = g >> 2, db = g & 3;
      if (g + 2 < NG) vread(g + 2, vf[(g + 2) % 3]);
      i32x4_t pb;
      pb[0] = (int)pk[ts >> 1][4 * (ts & 1) + 0];
      pb[1] = (int)pk[ts >> 1][4 * (ts & 1) + 1];
      pb[2] = (int)pk[ts >> 1][4 * (ts & 1) + 2];
      pb[3] = (int)pk[ts >> 1][4 * (ts & 1) + 3];
      i32x4_t va;
      va[0] = vf[g % 3][0][0];
      va[1] = vf[g % 3][0][1];
      va[2] = vf[g % 3][1][0];
      va[3] = vf[g % 3][1][1];
      oacc[db] = mfma32x32x16(as_bf16x8(va), as_bf16x8(pb), oacc[db]);
      if (SOFTMAX && next) {
        const int mc = g >> 3, ne = (2 * g) & 15;
        mx = vmax(mx, vmax(s_nxt[mc][ne], s_nxt[mc][ne + 1]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (next) {
      if constexpr (SOFTMAX) mt_cur = row_max(mx) * sl2;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s_cur[kb] = s_nxt[kb];
    }

    // The last step of a group: tiles up to it + BAR + 1 must have landed
    // before the next group reads them (K of it + 2 .. it + BAR + 1, V of
    // it + 1 .. it + BAR); later tiles may stay in flight.  The barrier also
    // frees the group's stages.  The last step waits for every copy.
    if (!next) {
      wait_tiles_but(0);
    } else if (st % BAR == BAR - 1) {
      wait_tiles_but(max(0, min(it + LOOK, ntiles - 1) - (it + BAR + 1)));
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };
  // A step whose ring stage is only known at run time.
  // A step whose ring stage is only known at run time (the masked steps near
  // the diagonal and the last one): one copy of the step, stage offsets added
  // at run time.
  auto step_any = [&](const int it, const bool next, const bool mask_next)
      __attribute__((always_inline)) {
    step(it, it % NS, next, mask_next);
  };

  // Tiles below n_clean need no mask; step it masks tile it + 1 when that
  // tile needs it.  Every wave runs ntiles steps (a barrier every BAR).  The
  // unmasked run starts at tile 0 and goes in groups of NS (stages 0..NS-1,
  // known at compile time), then a remainder of at most NS - 1 steps and the
  // masked ones with the stage known at run time (one copy of the step: six
  // unrolled masked copies spilled registers and ran 4 % slower).
  const int n1 = max(0, min(n_clean, ntiles - 1));
  const int clean_end = max(0, n1 - 1);
  int it = 0;
  for (; it + NS <= clean_end; it += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(it + u, u, true, false);
  }
  for (; it < clean_end; ++it) step_any(it, true, false);
  for (; it < ntiles - 1; ++it) step_any(it, true, true);
  if (ntiles > 0) step_any(ntiles - 1, false, false);

  // Epilogue: O = U / l (division after the V-matmul), LSE = m + log l;
  // without the softmax O = U.
  const float l_row = row_sum(l_part);
  if (row_ok) {
    const int qh = kvh * G + (r % G);
    const float inv = !SOFTMAX ? 1.f : (l_row > 0.f ? 1.f / l_row : 0.f);
    const int64_t obase = o_row_off(p, b, qi) + (int64_t)qh * p.os_h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * h;
        const float o0 = oacc[db][4 * i + 0] * inv, o1 = oacc[db][4 * i + 1] * inv;
        const float o2 = oacc[db][4 * i + 2] * inv, o3 = oacc[db][4 * i + 3] * inv;
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
    if (SOFTMAX && h == 0 && p.lse_out)
      p.lse_out[lse_row(p, b, qi) * p.Hq + qh] =
          l_row > 0.f ? (m_ref + fast_log2(l_row)) * kLn2 : kNegInf;
  }
}

template <int KB, int NS, int BAR, bool PAGED, bool SOFTMAX>
hipError_t launch_variant(const KParams& p, int nrt, int64_t nwg, hipStream_t s) {
  constexpr int lds = lds_bytes(KB, NS) + (PAGED ? 4 * kPrefillPageIds : 0);
  static_assert(lds <= 160 * 1024, "LDS per workgroup");
  hipError_t e = set_lds_limit_once(
      reinterpret_cast<const void*>(&prefill_d128_kernel<KB, NS, BAR, PAGED, SOFTMAX>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_d128_kernel<KB, NS, BAR, PAGED, SOFTMAX>), dim3((unsigned)nwg), dim3(NT), lds, s,
                     p, nrt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_d128(const KParams& p, hipStream_t s) {
  const int nrt = (p.rows + ROWS - 1) / ROWS;
  const int64_t nwg = (int64_t)p.B * p.Hkv * nrt;
  if (nwg == 0) return hipSuccess;
  constexpr int KB = kPrefillKeyBlocks, NS = kPrefillStages, BAR = kPrefillBarrierTiles;
  constexpr int NSP = kPrefillPagedStages, BARP = kPrefillPagedBarrierTiles;
  if (p.no_softmax) {
    if (p.page_table) return launch_variant<1, NSP, BARP, true, false>(p, nrt, nwg, s);
    return launch_variant<KB, NS, BAR, false, false>(p, nrt, nwg, s);
  }
  if (p.page_table) return launch_variant<1, NSP, BARP, true, true>(p, nrt, nwg, s);
  return launch_variant<KB, NS, BAR, false, true>(p, nrt, nwg, s);
}

}  // namespace attn

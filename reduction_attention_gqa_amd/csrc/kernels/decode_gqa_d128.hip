// Split-K GQA decode for bf16, Dqk = Dv = 128, up to 16 query rows per KV head.
//
// Decode has one query row per request, so output tiles are too few to fill
// the GPU; the key axis is split into pieces that run as separate workgroups
// (Cleave §2.2 "Split-K", §7.3 decode setting).  A workgroup packs the G query
// heads that share a KV head into the MFMA column dimension, so every K/V
// byte is read from HBM once.
//
// Two kernels share the key streaming below:
//
// * decode_gqa_d128_items (attn_decode_split, and attn_decode with one split
//   per request): one workgroup per work item (request, KV head, split j of
//   `chunk` keys), numbered split-fastest; XCD x (workgroups x, x + 8, ...)
//   takes one contiguous range of items, found on the device from the
//   per-request key counts, so one compiled kernel serves any mix of lengths.
//   Every split writes its partial (O_j = U_j / l_j, LSE_j) for the combine
//   kernel (Cleave §4, Fig. 5(b)); with one split per request O is written
//   directly.
// * decode_gqa_d128_stream (attn_decode when the plan splits): the keys of every
//   (request, KV head) unit, in 128-key rounds, laid end to end, and each of
//   the grid's workgroups (about one per compute unit) takes an equal run of
//   rounds, whatever the request lengths: a long contiguous stream per
//   compute unit, balanced by construction.  A unit that lies wholly inside
//   one run is written to O directly; a unit cut by run boundaries is split
//   into pieces, each piece's workgroup publishes its partial, and the last
//   one to finish merges them (the combine of Cleave §4 inside the kernel).
//
// Within a workgroup the four waves take interleaved 32-key blocks and each
// keeps its own running max / sum / output (a second, on-chip level of the
// same split); the waves are merged through LDS at the end of a piece.
//
// Per 32-key block and wave (transposed orientation, keys on the MFMA rows):
//   S^T[32 x 16] = K[32 x 128] * Q^T[128 x 16]      2 x 4 MFMA 16x16x32
//   online softmax on S^T columns (one query row per lane column)
//   O^T[128 x 16] += V^T[128 x 32] * P^T[32 x 16]   8 MFMA 16x16x32
// K arrives from HBM straight in the A-operand layout (16 bytes per lane);
// V goes row-major into a wave-private LDS tile and comes back transposed.
#include "../attn_internal.hpp"
#include "common.hpp"
#include "layout.hpp"

namespace attn {
namespace {

constexpr int KB = 32;           // keys per wave block
constexpr int D = 128;
constexpr int VROW = 288;        // bytes per V row in LDS (256 + 32 pad)
constexpr int VTILE = KB * VROW; // one wave's V tile
constexpr int NW = 4;            // waves per workgroup
constexpr int NB = 2;            // register blocks in flight per wave
constexpr int ROUND = KB * NW;   // keys per workgroup round (128)
static_assert(ROUND == kGqaTileN, "the planner's round is the kernel's");

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 8 bytes addressed by lanes 4e + i / 4 (e = 0..3) as its element e.
__device__ __forceinline__ i32x2_t ds_read_tr(const char* lds) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds));
  return __builtin_bit_cast(i32x2_t, v);
}

// One wave's 32-key block in registers: K in the MFMA A-operand layout, V rows.
struct Block {
  i32x4_t k[8];
  i32x4_t v[8];
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// The work item of this workgroup: request b, KV head kvh, split j (of sb) and
// the request's key count L.  Returns false when the workgroup has none.
// Every wave computes the same answer.
//
// `beyond_plan` is set when the device key counts need more than the plan
// provides: a request longer than s_max * chunk keys, or more work items in
// total than the grid was sized for (n_items, counted from the host lengths
// the plan was made from).  Work would then be dropped without a trace, so
// the caller writes NaN instead of a result.
__device__ __forceinline__ bool find_item(const KParams& p, int lane, int& b, int& kvh, int& j,
                                          int& sb, int& L, bool& beyond_plan) {
  beyond_plan = false;
  // One split per request: workgroup i is unit i (request i / Hkv, KV head
  // i % Hkv), every request has exactly one item, and only this request's
  // length is needed (a scalar load).
  if (p.s_max == 1) {
    if ((int64_t)blockIdx.x >= (int64_t)p.B * p.Hkv) return false;
    b = blockIdx.x / p.Hkv;
    kvh = blockIdx.x - b * p.Hkv;
    j = 0;
    sb = 1;
    L = kv_len_b(p, b);
    beyond_plan = L > p.chunk;
    return true;
  }
  const int64_t N = p.n_items;
  const int x = blockIdx.x & 7;
  const int64_t k = blockIdx.x >> 3;
  const int64_t s0 = ((int64_t)x * N) >> 3, s1 = ((int64_t)(x + 1) * N) >> 3;
  if (k >= s1 - s0) return false;
  const int64_t item = s0 + k;
  const int64_t cover = (int64_t)p.s_max * p.chunk;  // keys the plan covers per request
  // Splits per request: s_b = ceil(L_b / chunk), at least 1 (an empty request
  // still owns one item, which writes O = 0 and LSE = -inf), and at most the
  // plan's s_max (the workspace has s_max slots).
  if (p.kv_lens == nullptr && p.kv_indptr == nullptr) {
    sb = max(1, min((p.Lcap + p.chunk - 1) / p.chunk, p.s_max));
    const int64_t per = (int64_t)p.Hkv * sb;
    if (per == 0 || item >= per * p.B) return false;
    b = (int)(item / per);
    const int local = (int)(item - (int64_t)b * per);
    kvh = local / sb;
    j = local - kvh * sb;
    L = p.Lcap;
    beyond_plan = L > cover || per * p.B > N;
    return true;
  }
  // Items per request are Hkv * s_b; scan them 64 requests at a time, all the
  // way to the end (the total is checked against the grid).
  int64_t base = 0;
  bool found = false;
  for (int c = 0; c < p.B; c += 64) {
    const int bb = c + lane;
    int n = 0;
    if (bb < p.B)
      n = p.Hkv * max(1, min((kv_len_b(p, bb) + p.chunk - 1) / p.chunk, p.s_max));
    const int incl = wave_incl_scan(n, lane);
    const int total = __shfl(incl, 63, 64);
    if (!found && item < base + total) {
      const int rel = (int)(item - base);
      const int idx = __builtin_amdgcn_readfirstlane(__popcll(__ballot(incl <= rel)));
      const int excl = __builtin_amdgcn_readfirstlane(__shfl(incl - n, idx, 64));
      const int nb = __builtin_amdgcn_readfirstlane(__shfl(n, idx, 64));
      b = c + idx;
      sb = nb / p.Hkv;
      const int local = rel - excl;
      kvh = local / sb;
      j = local - kvh * sb;
      L = kv_len_b(p, b);
      found = true;
    }
    base += total;
  }
  beyond_plan = found && (L > cover || base > N);
  return found;
}


// Eight consecutive output values of one row to O (bf16 or f32), 16-byte
// stores when the address allows.
__device__ __forceinline__ void store_o8(const KParams& p, int64_t off, const f32x4_t& a,
                                         const f32x4_t& c) {
  if (p.o_bf16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + off;
    uint4 pk;
    pk.x = pack_bf16x2(a[0], a[1]);
    pk.y = pack_bf16x2(a[2], a[3]);
    pk.z = pack_bf16x2(c[0], c[1]);
    pk.w = pack_bf16x2(c[2], c[3]);
    if ((reinterpret_cast<uintptr_t>(op) & 15) == 0) {
      *reinterpret_cast<uint4*>(op) = pk;
    } else {
      const uint32_t wv[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        op[2 * e] = (uint16_t)(wv[e] & 0xffff);
        op[2 * e + 1] = (uint16_t)(wv[e] >> 16);
      }
    }
  } else {
    float* op = reinterpret_cast<float*>(p.o) + off;
    if ((reinterpret_cast<uintptr_t>(op) & 15) == 0) {
      reinterpret_cast<f32x4_t*>(op)[0] = a;
      reinterpret_cast<f32x4_t*>(op)[1] = c;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        op[e] = a[e];
        op[4 + e] = c[e];
      }
    }
  }
}

// A work item whose device key counts exceed the plan: NaN to its partial
// slot, which the combine kernel carries into O.
__device__ void write_beyond_plan(const KParams& p, int b, int kvh, int j) {
  const float nan = __builtin_nanf("");
  const f32x4_t v = {nan, nan, nan, nan};
  const int t = threadIdx.x;
  const int orow = t >> 4;
  const int oc = (t & 15) * 8;
  if (orow >= p.rows) return;
  const int i = orow / p.G;
  const int h = kvh * p.G + orow % p.G;
  const int64_t slot = (int64_t)j * p.B * p.Lq * p.Hq + ((int64_t)b * p.Lq + i) * p.Hq + h;
  float* dst = p.ws_o + slot * D + oc;
  reinterpret_cast<f32x4_t*>(dst)[0] = v;
  reinterpret_cast<f32x4_t*>(dst)[1] = v;
  if (oc == 0) p.ws_lse[slot] = nan;
}

// One wave's running state over a piece of keys.
struct WaveState {
  f32x4_t oacc[8];  // O^T[d = 16 db + 4 h4 + i][row r], relative to m_run
  float m_run;      // running max of the lane's row (base-2 units)
  float l_part;     // this lane's share of the row sum
};

// Streams keys [lo, hi) of (request b, KV head kvh), L_b = L keys, into each
// wave's state.  Wave w takes blocks lo + 32 w + 128 i (NB in flight).  Every
// thread of the workgroup calls it.  PAGED: K and V rows are found through
// the page table (power-of-two page size); the ids of a segment's pages are
// staged in LDS (at most kGqaPageIds - 1 pages a segment) and every lane forms
// the 64-bit address of each row it loads, so pages of any size, down to one
// row, are read with the same 16-byte-per-lane loads as the strided layout.
template <bool PAGED, bool ROTATE = false>
__device__ __forceinline__ void stream_keys(const KParams& p, int b, int kvh, int lo, int hi,
                                            int L, char* lds_raw, int* page_ids, WaveState& ws,
                                            int rot_rounds = 0) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;   // MFMA column: query row within the KV group
  const int h4 = lane >> 4;  // lane group
  const int R = p.rows;
  const int qi = r / p.G;    // query position of row r
  const int qh = kvh * p.G + r % p.G;

  // Q^T as the B operand: lane holds Q[row r][d = 32*db + 8*h4 .. +7].
  bf16x8_t qf[4];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
    const int64_t qoff = (int64_t)b * p.qs_b + (int64_t)qi * p.qs_t + (int64_t)qh * p.qs_h;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x4_t v = {0, 0, 0, 0};
      if (r < R) v = *reinterpret_cast<const i32x4_t*>(qp + qoff + 32 * db + 8 * h4);
      qf[db] = as_bf16x8(v);
    }
  }

  // The buffer ranges end at the piece's last key: loads past it return zero
  // without touching memory, so every load below is unconditional (which lets
  // the compiler wait only for the block about to be used).
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)kvh * p.ks_h;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)kvh * p.vs_h;
  if constexpr (!PAGED) {
    kp += kv_base_off(p, b, p.ks_b, p.ks_t);
    vp += kv_base_off(p, b, p.vs_b, p.vs_t);
  }
  const uint32_t kst = (uint32_t)(p.ks_t * 2);  // bytes between consecutive keys
  const uint32_t vst = (uint32_t)(p.vs_t * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, PAGED ? 0u : (uint32_t)hi * kst);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, PAGED ? 0u : (uint32_t)hi * vst);

  const int psh = PAGED ? p.page_shift : 0;
  const int pmask = (1 << psh) - 1;
  const int64_t kpage = p.ks_b * 2;  // bytes between pages (paged layout)
  const int64_t vpage = p.vs_b * 2;
  int seg_lo = lo, seg_hi = hi;      // the keys whose page ids are staged
  int pg0 = 0;
  // Address of key `key` in a pool; keys past the segment read its last key
  // instead (its scores are masked and its probabilities are zero).
  auto paged_row = [&](const uint16_t* pool, int64_t page_bytes, uint32_t st, int key) {
    const int kc = min(key, seg_hi - 1);
    const int pg = page_ids[(kc >> psh) - pg0];
    return reinterpret_cast<const char*>(pool) + (int64_t)pg * page_bytes +
           (int64_t)(kc & pmask) * st;
  };

  // Per-lane load offsets inside a block (bytes), independent of the block start.
  //   K: sub-block sb, d-block db -> key 16*sb + r, d = 32*db + 8*h4
  //   V: load c -> key 4*c + h4, d = 8*r
  const uint32_t k_lane = (uint32_t)r * kst + (uint32_t)(16 * h4);
  const uint32_t v_lane = (uint32_t)h4 * vst + (uint32_t)(16 * r);

  char* vt = lds_raw + w * VTILE;  // this wave's row-major V tile [32][VROW]
  // ds_read_tr addresses: lane l reads row l/4 (+16), columns 16*db + 4*(l%4).
  const char* vt_rd = vt + (lane >> 2) * VROW + 8 * (lane & 3);

  f32x4_t oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_part = 0.f;
  const float sl2 = p.scale_log2;
  const int qlim = qi + L - p.Lq;  // causal: keys <= qlim are visible

  auto load_block = [&](Block& x, int kb0) {
    if constexpr (PAGED) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const char* kr = paged_row(kp, kpage, kst, kb0 + 16 * sb + r) + 16 * h4;
#pragma unroll
        for (int db = 0; db < 4; ++db)
          x.k[sb * 4 + db] = *reinterpret_cast<const i32x4_t*>(kr + 64 * db);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c)
        x.v[c] = *reinterpret_cast<const i32x4_t*>(paged_row(vp, vpage, vst, kb0 + 4 * c + h4) +
                                                    16 * r);
      return;
    }
    const uint32_t kbc = (uint32_t)min(kb0, hi);
    const uint32_t kbase = kbc * kst;
    const uint32_t vbase = kbc * vst;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        x.k[sb * 4 + db] = buf_load16(krs, kbase + k_lane + (uint32_t)(16 * sb) * kst + 64 * db);
#pragma unroll
    for (int c = 0; c < 8; ++c) x.v[c] = buf_load16(vrs, vbase + v_lane + (uint32_t)(4 * c) * vst);
  };

  auto process_block = [&](const Block& x, int kb) {
    // V rows into the wave's LDS tile: load c is row 4c + h4, bytes 16r .. 16r + 15.
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<i32x4_t*>(vt + (4 * c + h4) * VROW + 16 * r) = x.v[c];

    // S^T = K Q^T for the two 16-key sub-blocks.
    f32x4_t s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < 4; ++db) a = mfma16x16x32(as_bf16x8(x.k[sb * 4 + db]), qf[db], a);
      s[sb] = a;
    }
    // Scale to base-2 units and mask: lane holds keys kb + 16*sb + 4*h4 + i.
    float xs[8];
    float mt = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 16 * sb + 4 * h4 + i;
        const bool vis = key < seg_hi && (!p.causal || key <= qlim);
        const float v = vis ? s[sb][i] * sl2 : kNegInf;
        xs[sb * 4 + i] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    float alpha = 1.f;
    float pv[8];
    if (m_new == kNegInf) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = 0.f;
    } else {
      alpha = fast_exp2(m_run - m_new);
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(xs[e] - m_new);
    }
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ps += pv[e];
    l_part = l_part * alpha + ps;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] *= alpha;

    // P^T as the B operand: k-slot 8*h4 + t <-> key 4*h4 + t (t < 4), 16 + 4*h4 + t - 4.
    i32x4_t pk;
    pk[0] = (int)pack_bf16x2(pv[0], pv[1]);
    pk[1] = (int)pack_bf16x2(pv[2], pv[3]);
    pk[2] = (int)pack_bf16x2(pv[4], pv[5]);
    pk[3] = (int)pack_bf16x2(pv[6], pv[7]);
    const bf16x8_t pb = as_bf16x8(pk);

    // O^T += V^T P^T.  A lane holds V^T[d = 16*db + r][the same key slots]: the
    // transposed LDS reads give keys 4*h4 + e (rows l/4) and 16 + 4*h4 + e.
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const i32x2_t v0 = ds_read_tr(vt_rd + 32 * db);
      const i32x2_t v1 = ds_read_tr(vt_rd + 16 * VROW + 32 * db);
      i32x4_t va;
      va[0] = v0[0];
      va[1] = v0[1];
      va[2] = v1[0];
      va[3] = v1[1];
      oacc[db] = mfma16x16x32(as_bf16x8(va), pb, oacc[db]);
    }
  };

  // Rotation over NB register blocks: while one block is processed, the next
  // NB - 1 are in flight.  Loads past the piece return zero without touching
  // memory.  Paged keys go segment by segment (each segment's page ids staged
  // in LDS first); a paged piece with no keys loads nothing.
  constexpr int STEP = KB * NW;
  const int seg_len = PAGED ? ((kGqaPageIds - 1) << psh) / STEP * STEP : 0;
  for (seg_lo = lo; seg_lo < hi || (!PAGED && seg_lo == lo); seg_lo += PAGED ? seg_len : hi - lo) {
    if constexpr (PAGED) {
      seg_hi = min(hi, seg_lo + seg_len);
      pg0 = seg_lo >> psh;
      const int n_ids = min(((seg_hi - 1) >> psh) - pg0 + 1, kGqaPageIds);
      const int32_t* row = p.page_table + (int64_t)b * p.ppr + pg0;
      __syncthreads();  // the previous segment's ids are no longer read
      for (int e = threadIdx.x; e < n_ids; e += NW * 64) {
        const int pg = row[e];
        page_ids[e] = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
      }
      __syncthreads();
    }
    Block X[NB];
    // The rounds of the piece in rotated order (ROTATE, non-paged):
    // position v (from seg_lo) holds round (v / STEP + rot_rounds) mod the
    // round count, so units that start together do not walk the same
    // address offsets in step.  Positions past the last round stay past it
    // (zero loads, nothing processed).
    const int span = (seg_hi - seg_lo + STEP - 1) / STEP * STEP;
    const int rot = !ROTATE || PAGED || span == 0 ? 0 : (int)((int64_t)rot_rounds * STEP % span);
    // Positions that can hold keys: the whole span when rotated (the last,
    // partial round may sit anywhere), else up to the last key.
    const int vend = ROTATE && rot ? seg_lo + span : seg_hi;
    auto key_of = [&](int v) {
      if (!ROTATE || v >= seg_lo + span) return v;
      const int o = v - seg_lo + rot;
      return seg_lo + (o >= span ? o - span : o);
    };
    int kb = seg_lo + KB * w;
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) load_block(X[i], key_of(kb + i * STEP));
    // The scheduling barriers keep each block's loads issued before the wait for
    // the block being processed.
    for (; kb < vend; kb += NB * STEP) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        load_block(X[(i + NB - 1) % NB], key_of(kb + (i + NB - 1) * STEP));
        __builtin_amdgcn_sched_barrier(0);
        if (i == 0 || kb + i * STEP < vend) process_block(X[i], key_of(kb + i * STEP));
      }
    }
    if (!PAGED) break;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) ws.oacc[db] = oacc[db];
  ws.m_run = m_run;
  ws.l_part = l_part;
}

// One row's result after the waves are merged: thread t holds row t >> 4,
// columns 8 (t & 15) .. + 7 (threads of rows >= G * Lq hold nothing useful).
struct RowOut {
  f32x4_t o0, o1;  // O = U / l, columns oc .. oc + 3 and oc + 4 .. oc + 7
  float lse;       // natural-log LSE of the piece (-inf without a key)
};

// Merges the four waves' states through LDS (all threads call it).  The
// caller must not write lds_raw again before a barrier.
__device__ __forceinline__ RowOut merge_waves(const WaveState& ws, char* lds_raw,
                                              float (*m_w)[16], float (*l_w)[16]) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, h4 = lane >> 4;
  float l_row = ws.l_part;
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  __syncthreads();  // every wave is done with its V tile
  if (h4 == 0) {
    m_w[w][r] = ws.m_run;
    l_w[w][r] = l_row;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int u = 0; u < NW; ++u) M = fmaxf(M, m_w[u][r]);
  const float fw = (ws.m_run == kNegInf) ? 0.f : fast_exp2(ws.m_run - M);
  float* osum = reinterpret_cast<float*>(lds_raw);  // [NW][16][128] floats
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      osum[(w * 16 + r) * D + 16 * db + 4 * h4 + i] = ws.oacc[db][i] * fw;
  __syncthreads();

  const int t = threadIdx.x;
  const int orow = t >> 4;
  const int oc = (t & 15) * 8;
  float Mr = kNegInf;
#pragma unroll
  for (int u = 0; u < NW; ++u) Mr = fmaxf(Mr, m_w[u][orow]);
  float Lt = 0.f;
  if (Mr != kNegInf) {
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const float mu = m_w[u][orow];
      if (mu != kNegInf) Lt += l_w[u][orow] * fast_exp2(mu - Mr);
    }
  }
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  RowOut ro;
  ro.o0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  ro.o1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    ro.o0 += *reinterpret_cast<const f32x4_t*>(osum + (u * 16 + orow) * D + oc);
    ro.o1 += *reinterpret_cast<const f32x4_t*>(osum + (u * 16 + orow) * D + oc + 4);
  }
  ro.o0 *= inv;
  ro.o1 *= inv;
  ro.lse = Lt > 0.f ? (Mr + fast_log2(Lt)) * kLn2 : kNegInf;
  return ro;
}

// Work-item kernel (attn_decode_split): every split writes its partial.
template <bool PAGED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_gqa_d128_items(KParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[NW * VTILE];  // 36 KiB
  __shared__ float m_w[NW][16];
  __shared__ float l_w[NW][16];
  __shared__ int page_ids[PAGED ? kGqaPageIds : 1];

  const int lane = threadIdx.x & 63;
  int b, kvh, j, sb, L;
  bool beyond_plan;
  if (!find_item(p, lane, b, kvh, j, sb, L, beyond_plan)) return;
  // The item is the same in every lane; saying so keeps the buffer resources
  // in scalar registers (otherwise every load is wrapped in a loop over the
  // distinct descriptor values of the wave).
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  j = __builtin_amdgcn_readfirstlane(j);
  L = __builtin_amdgcn_readfirstlane(L);
  if (__builtin_amdgcn_readfirstlane((int)beyond_plan)) {
    write_beyond_plan(p, b, kvh, j);
    return;
  }
  const int lo = j * p.chunk;
  const int hi = min(lo + p.chunk, L);
  WaveState ws;
  // Units start at different rounds of their keys (one round further per
  // unit): 2-3 % faster on the Llama decode; the stream kernel, whose runs
  // continue from one unit into the next, keeps the plain order.
  stream_keys<PAGED, !PAGED>(p, b, kvh, lo, hi, L, lds_raw, page_ids, ws, b * p.Hkv + kvh);
  const RowOut ro = merge_waves(ws, lds_raw, m_w, l_w);
  const int t = threadIdx.x;
  const int orow = t >> 4;
  const int oc = (t & 15) * 8;
  if (orow < p.rows) {
    const int i = orow / p.G;
    const int h = kvh * p.G + orow % p.G;
    if (p.split_mode == 0) {  // one split per request: O directly
      store_o8(p, (int64_t)b * p.os_b + (int64_t)i * p.os_t + (int64_t)h * p.os_h + oc, ro.o0,
               ro.o1);
      if (oc == 0 && p.lse_out) p.lse_out[((int64_t)b * p.Lq + i) * p.Hq + h] = ro.lse;
      return;
    }
    const int64_t slot = (int64_t)j * p.B * p.Lq * p.Hq + ((int64_t)b * p.Lq + i) * p.Hq + h;
    float* dst = p.ws_o + slot * D + oc;
    reinterpret_cast<f32x4_t*>(dst)[0] = ro.o0;
    reinterpret_cast<f32x4_t*>(dst)[1] = ro.o1;
    if (oc == 0) p.ws_lse[slot] = ro.lse;
  }
}

// One workgroup's run of rounds [g T / N, (g + 1) T / N) over the units laid
// end to end (unit u = (request, KV head), max(1, ceil(L_b / 128)) rounds,
// so an empty unit still has one piece, which writes O = 0).
//
// A unit covering global rounds [U0, U1) is cut into the pieces of the
// workgroups whose runs meet it: g_first = ceil((U0 + 1) N / T) - 1 to
// g_last = ceil(U1 N / T) - 1, piece index g - g_first.  Every workgroup
// computes the same numbers, so they agree on the piece count.
//
// Merge of a cut unit: the (request, KV head) counter in ws_cnt holds tickets
// in its low 16 bits and published partials in its high 16 bits.  Each piece
// takes a ticket as it starts; all but the last publish their partial when
// their keys are done and count it; the last one (ticket = pieces - 1) knows
// every other piece has already taken its ticket, so that workgroup is
// resident and has nothing left to wait for (a piece that does not merge
// never waits): it waits for their count, merges all pieces in piece
// order (its own from registers, with the same arithmetic as a stored one,
// so the bits do not depend on which piece finishes last), writes O and
// resets the counter.  A partial is an 8 KiB block in thread order (thread t's
// columns oc .. oc + 3 at 16 t, oc + 4 .. oc + 7 at 4096 + 16 t: each store
// or load instruction moves 1 KiB of whole cache lines) plus one LSE per row.
//
// Ordering on gfx950: partials are written with sc1 (device-coherent)
// stores, which write through the XCD's L2 instead of leaving dirty lines
// there, and each wave waits for them (vmcnt(0)) before the workgroup barrier
// that precedes the counting atomic; the reader's loads are sc1 too, so they
// are served from the device-coherent level, never from a stale line of its
// own L2.  Because no data is left dirty in an L2, the whole-L2 write-back of
// a device-scope release fence is not needed.
template <bool PAGED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_gqa_d128_stream(KParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[NW * VTILE];  // 36 KiB
  __shared__ float m_w[NW][16];
  __shared__ float l_w[NW][16];
  __shared__ int page_ids[PAGED ? kGqaPageIds : 1];
  __shared__ int s_ticket;

  const int lane = threadIdx.x & 63;
  const int64_t T = p.n_items;            // rounds of all units (plan)
  const int64_t N = gridDim.x;
  const int64_t g = blockIdx.x;
  const int64_t r_beg = g * T / N, r_end = (g + 1) * T / N;
  if (r_beg >= r_end) return;

  // The request holding round r_beg, and the device total of rounds (units
  // of request b have max(1, ceil(L_b / 128)) rounds each), scanned 64
  // requests at a time.
  int64_t base = 0, req_base = 0;
  int b = -1;
  for (int c = 0; c < p.B; c += 64) {
    const int bb = c + lane;
    int n = 0;
    if (bb < p.B) n = p.Hkv * max(1, (kv_len_b(p, bb) + ROUND - 1) / ROUND);
    const int incl = wave_incl_scan(n, lane);
    const int total = __shfl(incl, 63, 64);
    if (b < 0 && r_beg < base + total) {
      const int rel = (int)(r_beg - base);
      const int idx = __builtin_amdgcn_readfirstlane(__popcll(__ballot(incl <= rel)));
      b = c + idx;
      req_base = base + __builtin_amdgcn_readfirstlane(__shfl(incl - n, idx, 64));
    }
    base += total;
  }
  // More rounds on the device than the plan's T: the rounds past T belong to
  // no workgroup, so every workgroup writes NaN for the units it meets
  // instead of results (and counts nothing).
  const bool beyond_plan = base > T;
  if (b < 0) {
    // A run past the device's rounds (device lengths shorter than planned).
    return;
  }
  int L = uniform(kv_len_b(p, b));
  int nr = max(1, (L + ROUND - 1) / ROUND);
  int kvh = (int)((r_beg - req_base) / nr);
  int rin = (int)((r_beg - req_base) - (int64_t)kvh * nr);
  int64_t cur = r_beg;
  const int t = threadIdx.x;
  const int orow = t >> 4;
  const int oc = (t & 15) * 8;
  const int64_t nunits = (int64_t)p.B * p.Hkv;
  while (cur < r_end && b < p.B) {
    const int take = (int)min((int64_t)(nr - rin), r_end - cur);
    const int64_t U0 = cur - rin, U1 = U0 + nr;
    const bool whole = rin == 0 && take == nr;
    const int lo = rin * ROUND;
    const int hi = min((rin + take) * ROUND, L);
    const int qi = orow / p.G;
    const int qh = kvh * p.G + orow % p.G;
    const int64_t row = ((int64_t)b * p.Lq + qi) * p.Hq + qh;
    const int64_t obase = (int64_t)b * p.os_b + (int64_t)qi * p.os_t + (int64_t)qh * p.os_h + oc;
    if (beyond_plan) {
      const float nan = __builtin_nanf("");
      const f32x4_t v = {nan, nan, nan, nan};
      if (orow < p.rows) {
        store_o8(p, obase, v, v);
        if (oc == 0 && p.lse_out) p.lse_out[row] = nan;
      }
    } else {
      // A piece of a cut unit takes its ticket as it starts, so the atomic's
      // round trip runs under the piece's key stream.
      int early_ticket = 0;
      if (!whole && t == 0)
        early_ticket = __hip_atomic_fetch_add(p.counters + b * p.Hkv + kvh, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      WaveState ws;
      stream_keys<PAGED>(p, b, kvh, lo, hi, L, lds_raw, page_ids, ws);
      const RowOut ro = merge_waves(ws, lds_raw, m_w, l_w);
      if (whole) {
        if (orow < p.rows) {
          store_o8(p, obase, ro.o0, ro.o1);
          if (oc == 0 && p.lse_out) p.lse_out[row] = ro.lse;
        }
      } else {
        const int64_t g_first = ((U0 + 1) * N + T - 1) / T - 1;
        const int64_t g_last = (U1 * N + T - 1) / T - 1;
        const int pieces = (int)(g_last - g_first + 1);
        const int pi = (int)(g - g_first);
        const int unit = b * p.Hkv + kvh;
        int* cnt = p.counters + unit;
        if (t == 0) s_ticket = early_ticket & 0xffff;
        __syncthreads();
        const int ticket = s_ticket;
        const __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.ws_o, 0xffffffffu);
        auto blk = [&](int q) { return (uint32_t)(((int64_t)q * nunits + unit) * (16 * D * 4)); };
        auto lse_at = [&](int q) { return p.ws_lse + ((int64_t)q * nunits + unit) * 16 + orow; };
        if (ticket < pieces - 1) {
          store16_dev(wrs, blk(pi) + 16u * (uint32_t)t, ro.o0);
          store16_dev(wrs, blk(pi) + 4096u + 16u * (uint32_t)t, ro.o1);
          if (oc == 0) store_dev(lse_at(pi), ro.lse);
          wait_vmem();
          __syncthreads();
          if (t == 0)
            __hip_atomic_fetch_add(cnt, 1 << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          if (t == 0) {
            while ((__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 16) <
                   pieces - 1)
              __builtin_amdgcn_s_sleep(2);
          }
          __syncthreads();
          // Pieces in order, four at a time: one memory round trip per batch;
          // the running reference and weight sum are rescaled per batch.
          constexpr int MB = 4;
          float M = kNegInf;  // base-2 units
          f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
          float wsum = 0.f;
          for (int q0 = 0; q0 < pieces; q0 += MB) {
            float lq[MB];
            f32x4_t x0[MB], x1[MB];
#pragma unroll
            for (int u = 0; u < MB; ++u) {
              const int q = q0 + u;
              if (q < pieces && q != pi) {
                lq[u] = load_dev(lse_at(q));
                x0[u] = load16_dev(wrs, blk(q) + 16u * (uint32_t)t);
                x1[u] = load16_dev(wrs, blk(q) + 4096u + 16u * (uint32_t)t);
              } else {
                lq[u] = ro.lse;
                x0[u] = ro.o0;
                x1[u] = ro.o1;
              }
            }
            float mb = M;
#pragma unroll
            for (int u = 0; u < MB; ++u)
              if (q0 + u < pieces) mb = fmaxf(mb, lq[u] * kLog2e);
            if (mb == kNegInf) continue;
            const float sc = (M == kNegInf) ? 0.f : fast_exp2(M - mb);
            a0 *= sc;
            a1 *= sc;
            wsum *= sc;
#pragma unroll
            for (int u = 0; u < MB; ++u) {
              if (q0 + u < pieces) {
                const float wgt = fast_exp2(lq[u] * kLog2e - mb);
                a0 += wgt * x0[u];
                a1 += wgt * x1[u];
                wsum += wgt;
              }
            }
            M = mb;
          }
          if (M != kNegInf) {
            const float winv = 1.f / wsum;
            a0 *= winv;
            a1 *= winv;
          }
          if (orow < p.rows) {
            store_o8(p, obase, a0, a1);
            if (oc == 0 && p.lse_out)
              p.lse_out[row] = M == kNegInf ? kNegInf : (M + fast_log2(wsum)) * kLn2;
          }
          if (t == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();  // LDS (wave merge, ticket) is reused by the next piece
    cur += take;
    rin = 0;
    if (++kvh == p.Hkv) {
      kvh = 0;
      ++b;
      if (b < p.B) {
        L = uniform(kv_len_b(p, b));
        nr = max(1, (L + ROUND - 1) / ROUND);
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_gqa_d128(const KParams& p, hipStream_t s) {
  if (p.split_mode == 3) {
    const unsigned nwg = (unsigned)p.stream_grid;
    if (nwg == 0) return hipSuccess;
    if (p.page_table)
      hipLaunchKernelGGL(decode_gqa_d128_stream<true>, dim3(nwg), dim3(NW * 64), 0, s, p);
    else
      hipLaunchKernelGGL(decode_gqa_d128_stream<false>, dim3(nwg), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
  }
  const int64_t nwg = (p.n_items + 7) / 8 * 8;
  if (nwg == 0) return hipSuccess;
  if (p.page_table)
    hipLaunchKernelGGL(decode_gqa_d128_items<true>, dim3((unsigned)nwg), dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL(decode_gqa_d128_items<false>, dim3((unsigned)nwg), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn

// Split-K GQA decode for bf16, Dqk = Dv = 128, up to 16 query rows per KV head.
//
// Decode has one query row per request, so output tiles are too few to fill
// the GPU; the key axis is split into chunks that run as separate workgroups
// (Cleave §2.2 "Split-K", §7.3 decode setting).  A workgroup owns one work
// item (request, KV head, split) and packs the G query heads that share the KV
// head into the MFMA column dimension, so every K/V byte is read from HBM once.
//
// Work items are numbered with the split fastest, then the KV head, then the
// request.  With several splits per request, XCD x (workgroups x, x + 8, ...)
// takes one contiguous range of them, so each XCD streams a compact region of
// the K/V cache; with one split per request, workgroup i takes item i, which
// spreads the KV heads of a request over the XCDs (measured faster for that
// case, the other way round for many splits).  The item of a workgroup is
// found on the device from the per-request key counts, so one compiled kernel
// serves any mix of lengths.
//
// Within the workgroup the four waves take interleaved 32-key blocks of the
// split and each keeps its own running max / sum / output (a second, on-chip
// level of the same split); the waves are merged through LDS at the end.
//
// Per 32-key block and wave (transposed orientation, keys on the MFMA rows):
//   S^T[32 x 16] = K[32 x 128] * Q^T[128 x 16]      2 x 4 MFMA 16x16x32
//   online softmax on S^T columns (one query row per lane column)
//   O^T[128 x 16] += V^T[128 x 32] * P^T[32 x 16]   8 MFMA 16x16x32
// K arrives from HBM straight in the A-operand layout (16 bytes per lane);
// V goes row-major into a wave-private LDS tile and comes back transposed.
//
// Epilogues (KParams::split_mode):
//   0  one split per request: O = U / l straight to the output;
//   1  every split writes its partial (O_j = U_j / l_j, LSE_j) to the
//      workspace for the combine kernel (Cleave §4, Fig. 5(b));
//   2  as 1, then the last split of each (request, KV head) to finish merges
//      the partials itself (single launch); a request with one split writes
//      O directly.
#include "../attn_internal.hpp"
#include "common.hpp"
#include "layout.hpp"

namespace attn {
namespace {

constexpr int KB = 32;           // keys per wave block
constexpr int D = 128;
constexpr int VROW = 288;        // bytes per V row in LDS (256 + 32 pad)
constexpr int VTILE = KB * VROW; // one wave's V tile

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

// A work item whose device key counts exceed the plan: NaN to its rows of O
// (one split per request, or the single-launch merge) or to its partial slot
// (the two-launch split, whose NaN the combine carries into O), and no
// arrival is counted, so the counters stay zero.
__device__ void write_beyond_plan(const KParams& p, int b, int kvh, int j, int sb) {
  const float nan = __builtin_nanf("");
  const f32x4_t v = {nan, nan, nan, nan};
  const int t = threadIdx.x;
  const int orow = t >> 4;
  const int oc = (t & 15) * 8;
  if (orow >= p.rows) return;
  const int i = orow / p.G;
  const int h = kvh * p.G + orow % p.G;
  const int64_t row = ((int64_t)b * p.Lq + i) * p.Hq + h;
  if (p.split_mode == 1) {
    const int64_t slot = (int64_t)j * p.B * p.Lq * p.Hq + row;
    float* dst = p.ws_o + slot * D + oc;
    reinterpret_cast<f32x4_t*>(dst)[0] = v;
    reinterpret_cast<f32x4_t*>(dst)[1] = v;
    if (oc == 0) p.ws_lse[slot] = nan;
    return;
  }
  store_o8(p, (int64_t)b * p.os_b + (int64_t)i * p.os_t + (int64_t)h * p.os_h + oc, v, v);
  if (oc == 0 && p.lse_out) p.lse_out[row] = nan;
}

// Four waves per workgroup; a workgroup round covers KB * NW keys.  NB
// register blocks per wave are in flight (four measured slower than two, also
// with one workgroup per CU).
//
// PAGED: K and V rows are found through the page table (page size a power of
// two).  The item's page ids are staged in LDS once; each lane then forms the
// 64-bit address of every row it loads, so pages of any size, down to one
// row, are read with the same 16-byte-per-lane loads as the strided layout.
constexpr int NW = 4;
constexpr int NB = 2;
template <bool PAGED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_gqa_d128_kernel(KParams p) {
  constexpr int STEP = KB * NW;
  __shared__ __attribute__((aligned(16))) char lds_raw[NW * VTILE];  // 36 KiB
  __shared__ float m_w[NW][16];
  __shared__ float l_w[NW][16];
  __shared__ int page_ids[PAGED ? kGqaPageIds : 1];

  const int lane = threadIdx.x & 63;
  // Wave index, made visibly wave-uniform so the key loop below is a scalar loop.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b, kvh, j, sb, L;
  bool beyond_plan;
  if (!find_item(p, lane, b, kvh, j, sb, L, beyond_plan)) return;
  // The item is the same in every lane; saying so keeps the buffer resources
  // below in scalar registers (otherwise every load is wrapped in a loop over
  // the distinct descriptor values of the wave).
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  j = __builtin_amdgcn_readfirstlane(j);
  sb = __builtin_amdgcn_readfirstlane(sb);
  L = __builtin_amdgcn_readfirstlane(L);
  if (__builtin_amdgcn_readfirstlane((int)beyond_plan)) {
    write_beyond_plan(p, b, kvh, j, sb);
    return;
  }
  const int lo = j * p.chunk;
  const int hi = min(lo + p.chunk, L);

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

  // The buffer ranges end at this split's last key: loads past it return zero
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

  // Paged: the ids of the pages holding keys [lo, hi), clamped into the pool.
  const int psh = PAGED ? p.page_shift : 0;
  const int pmask = (1 << psh) - 1;
  const int pg0 = lo >> psh;
  if constexpr (PAGED) {
    const int n_ids = hi > lo ? min(((hi - 1) >> psh) - pg0 + 1, kGqaPageIds) : 0;
    const int32_t* row = p.page_table + (int64_t)b * p.ppr + pg0;
    for (int e = threadIdx.x; e < n_ids; e += NW * 64) {
      const int pg = row[e];
      page_ids[e] = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
    }
    __syncthreads();
  }
  const int64_t kpage = p.ks_b * 2;  // bytes between pages (paged layout)
  const int64_t vpage = p.vs_b * 2;
  // Address of key `key` in a pool; keys past the split read the split's last
  // key instead (its scores are masked and its probabilities are zero).
  auto paged_row = [&](const uint16_t* pool, int64_t page_bytes, uint32_t st, int key) {
    const int kc = min(key, hi - 1);
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
        const bool vis = key < hi && (!p.causal || key <= qlim);
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
  // NB - 1 are in flight.  Wave w takes blocks lo + 32*w + 128*i.  Loads past
  // the split return zero without touching memory.
  // A paged item with no keys loads nothing (there is no row to clamp to).
  Block X[NB];
  int kb = lo + KB * w;
  if (!PAGED || hi > lo) {
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) load_block(X[i], kb + i * STEP);
    // The scheduling barriers keep each block's loads issued before the wait for
    // the block being processed.
    for (; kb < hi; kb += NB * STEP) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        load_block(X[(i + NB - 1) % NB], kb + (i + NB - 1) * STEP);
        __builtin_amdgcn_sched_barrier(0);
        if (i == 0 || kb + i * STEP < hi) process_block(X[i], kb + i * STEP);
      }
    }
  }

  // Merge the four waves' partial states.
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  if (h4 == 0) {
    m_w[w][r] = m_run;
    l_w[w][r] = l_row;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int u = 0; u < NW; ++u) M = fmaxf(M, m_w[u][r]);
  const float fw = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - M);
  float* osum = reinterpret_cast<float*>(lds_raw);  // [NW][16][128] floats
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) osum[(w * 16 + r) * D + 16 * db + 4 * h4 + i] = oacc[db][i] * fw;
  __syncthreads();

  // Threads 0..255 write 16 rows x 128 columns: row t/16, columns 8*(t%16) .. +7.
  const int t = threadIdx.x;
  const int orow = t >> 4;
  const int oc = (t & 15) * 8;
  if (orow < R) {
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
    f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      o0 += *reinterpret_cast<const f32x4_t*>(osum + (u * 16 + orow) * D + oc);
      o1 += *reinterpret_cast<const f32x4_t*>(osum + (u * 16 + orow) * D + oc + 4);
    }
    o0 *= inv;
    o1 *= inv;
    const int i = orow / p.G;
    const int h = kvh * p.G + orow % p.G;
    const float lse = Lt > 0.f ? (Mr + fast_log2(Lt)) * kLn2 : kNegInf;
    if (p.split_mode == 0 || (p.split_mode == 2 && sb == 1)) {
      store_o8(p, (int64_t)b * p.os_b + (int64_t)i * p.os_t + (int64_t)h * p.os_h + oc, o0, o1);
      if (oc == 0 && p.lse_out) p.lse_out[((int64_t)b * p.Lq + i) * p.Hq + h] = lse;
    } else {
      const int64_t slot = (int64_t)j * p.B * p.Lq * p.Hq + ((int64_t)b * p.Lq + i) * p.Hq + h;
      float* dst = p.ws_o + slot * D + oc;
      if (p.split_mode == 1) {
        reinterpret_cast<f32x4_t*>(dst)[0] = o0;
        reinterpret_cast<f32x4_t*>(dst)[1] = o1;
        if (oc == 0) p.ws_lse[slot] = lse;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          store_dev(dst + e, o0[e]);
          store_dev(dst + 4 + e, o1[e]);
        }
        if (oc == 0) store_dev(p.ws_lse + slot, lse);
      }
    }
  }
  if (p.split_mode != 2 || sb == 1) return;

  // Single-launch merge: the last split of this (request, KV head) to arrive
  // reduces the sb partials (the combine of Cleave §4, done in place).  Each
  // wave waits until its device-coherent partial stores have completed, the
  // barrier gathers the waves, and thread 0 counts the arrival; the last
  // arrival reads the partials back with device-coherent loads issued after
  // its counter update returned.
  __shared__ int s_last;
  wait_vmem();
  __syncthreads();
  const int unit = b * p.Hkv + kvh;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(p.counters + unit, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == sb - 1;
  __syncthreads();
  if (!s_last) return;
  if (orow < R) {
    const int i = orow / p.G;
    const int h = kvh * p.G + orow % p.G;
    const int64_t nrows = (int64_t)p.B * p.Lq * p.Hq;
    const int64_t row = ((int64_t)b * p.Lq + i) * p.Hq + h;
    // One pass over the splits in split order, MB at a time: the loads of a
    // batch are independent (one memory round trip per batch, not two per
    // split); the running max and weight sum are rescaled per batch.
    constexpr int MB = 4;
    float M = kNegInf;  // natural-log units
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int j0 = 0; j0 < sb; j0 += MB) {
      float lse[MB];
      f32x4_t x0[MB], x1[MB];
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        const int64_t slot = (int64_t)min(j0 + u, sb - 1) * nrows + row;
        lse[u] = load_dev(p.ws_lse + slot);
        const float* src = p.ws_o + slot * D + oc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x0[u][e] = load_dev(src + e);
          x1[u][e] = load_dev(src + 4 + e);
        }
      }
      float mb = M;
#pragma unroll
      for (int u = 0; u < MB; ++u)
        if (j0 + u < sb) mb = fmaxf(mb, lse[u]);
      if (mb == kNegInf) continue;
      const float m2 = mb * kLog2e;
      const float sc = (M == kNegInf) ? 0.f : fast_exp2(M * kLog2e - m2);
      a0 *= sc;
      a1 *= sc;
      wsum *= sc;
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        if (j0 + u < sb) {
          const float wgt = fast_exp2(lse[u] * kLog2e - m2);
          a0 += wgt * x0[u];
          a1 += wgt * x1[u];
          wsum += wgt;
        }
      }
      M = mb;
    }
    if (M != kNegInf) {
      const float inv = 1.f / wsum;
      a0 *= inv;
      a1 *= inv;
    }
    store_o8(p, (int64_t)b * p.os_b + (int64_t)i * p.os_t + (int64_t)h * p.os_h + oc, a0, a1);
    if (oc == 0 && p.lse_out)
      p.lse_out[row] = M == kNegInf ? kNegInf : M + fast_log2(wsum) * kLn2;
  }
  if (threadIdx.x == 0)  // leave the counter zeroed for the next call
    __hip_atomic_store(p.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_decode_gqa_d128(const KParams& p, hipStream_t s) {
  const int64_t nwg = (p.n_items + 7) / 8 * 8;
  if (nwg == 0) return hipSuccess;
  if (p.page_table)
    hipLaunchKernelGGL(decode_gqa_d128_kernel<true>, dim3((unsigned)nwg), dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL(decode_gqa_d128_kernel<false>, dim3((unsigned)nwg), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn

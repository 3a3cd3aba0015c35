// Split-K GQA decode for bf16, Dqk = Dv = 128, up to 16 query rows per KV head.
//
// Decode has one query row per request, so output tiles are too few to fill
// the GPU; the key axis is split into chunks that run as separate workgroups
// (Cleave §2.2 "Split-K", §7.3 decode setting).  A workgroup owns one
// (split, KV head, request) unit and packs the G query heads that share the KV
// head into the MFMA column dimension, so every K/V byte is read from HBM once.
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
// V is transposed through a wave-private LDS tile.  Out-of-range keys are
// zero-filled by the buffer loads (num_records bound) and masked to -inf.
#include "../attn_internal.hpp"
#include "common.hpp"

namespace attn {
namespace {

constexpr int NW = 4;            // waves per workgroup
constexpr int KB = 32;           // keys per wave block
constexpr int STEP = KB * NW;    // keys per workgroup round
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

__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_gqa_d128_kernel(KParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[NW * VTILE];  // 36 KiB
  __shared__ float m_w[NW][16];
  __shared__ float l_w[NW][16];

  const int lane = threadIdx.x & 63;
  // Wave index, made visibly wave-uniform so the key loop below is a scalar loop.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int L = kv_len_of(p.kv_lens, b, p.Lcap);
  const int lo = j * p.chunk;
  if (lo >= L) return;
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
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;
  const uint32_t kst = (uint32_t)(p.ks_t * 2);  // bytes between consecutive keys
  const uint32_t vst = (uint32_t)(p.vs_t * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)hi * kst);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (uint32_t)hi * vst);

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

  // Ping-pong over two register blocks: while one block is processed, the
  // next one is in flight.  Wave w takes blocks lo + 32*w + 128*i.
  Block A, Bk;
  int kb = lo + KB * w;
  load_block(A, kb);
  // The scheduling barriers keep each block's loads issued before the wait for
  // the block being processed.
  for (; kb < hi; kb += 2 * STEP) {
    load_block(Bk, kb + STEP);
    __builtin_amdgcn_sched_barrier(0);
    process_block(A, kb);
    load_block(A, kb + 2 * STEP);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + STEP < hi) process_block(Bk, kb + STEP);
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
  float* osum = reinterpret_cast<float*>(lds_raw);  // [NW][16][128] floats (32 KiB)
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) osum[(w * 16 + r) * D + 16 * db + 4 * h4 + i] = oacc[db][i] * fw;
  __syncthreads();

  // 256 threads write 16 rows x 128 columns: thread -> row t/16, columns 8*(t%16) .. +7.
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
    const int64_t slot = (int64_t)j * p.B * p.Lq * p.Hq + ((int64_t)b * p.Lq + i) * p.Hq + h;
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(p.ws_o + slot * D + oc);
    dst[0] = o0;
    dst[1] = o1;
    if (oc == 0) p.ws_lse[slot] = Lt > 0.f ? (Mr + fast_log2(Lt)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_decode_gqa_d128(const KParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL(decode_gqa_d128_kernel, grid, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn

// Fused causal / non-causal GQA prefill for bf16, Dqk = Dv = 128.
//
// One workgroup (8 waves) computes one 256-row tile of one (request, KV head)
// group; a row is a (query position, head of the group) pair, so the G query
// heads that share a KV head share every K/V tile staged in LDS.  This is the
// inter-threadblock output tiling of Cleave §5.1 / §5.3 ([b_O, d] output tiles,
// one per workgroup) with GQA packing added.  Inside, the key axis is tiled in
// 64-key steps (iterative tiling, §5.1 and §5.3); the exp tile feeds both the
// row sum and the V-matmul in the same step (horizontal fusion, §5.1); the
// division by the row sum comes after the V-matmul (§2.2, Fig. 2); the Q tile
// is loaded once, outside the key loop (§6.1).  The running max rescaling is
// the online-softmax update.
//
// Per wave (32 rows) and 64-key tile, keys on the MFMA rows:
//   S^T[64 x 32]  = K[64 x 128] Q^T[128 x 32]     2 x 8 MFMA 32x32x16 bf16
//   O^T[128 x 32] += V^T[128 x 64] P^T[64 x 32]   4 x 4 MFMA 32x32x16 bf16
// K is read from LDS in the A-operand layout (16 bytes per lane); V is read
// transposed from its row-major LDS tile with ds_read_b64_tr_b16.
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

constexpr int NW = 8;                 // waves per workgroup
constexpr int NT = NW * 64;
constexpr int ROWS = NW * 32;         // rows per workgroup
constexpr int TK = 64;                // keys per tile
constexpr int D = 128;
constexpr int K_STRIDE = 272;         // bytes per K row in LDS (256 + 16 pad)
constexpr int V_STRIDE = 288;         // bytes per V row in LDS (256 + 32 pad)
constexpr int K_TILE = TK * K_STRIDE;
constexpr int V_TILE = TK * V_STRIDE;
constexpr int STAGE = K_TILE + V_TILE;
constexpr int LDS_BYTES = 2 * STAGE;  // double buffered

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 8 bytes addressed by lanes 4e + i / 4 (e = 0..3) as its element e.
__device__ __forceinline__ i32x2_t ds_read_tr(const char* lds) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds));
  return __builtin_bit_cast(i32x2_t, v);
}

__global__ __launch_bounds__(NT) void prefill_d128_kernel(KParams p, int nrt) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = threadIdx.x;

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

  // This wave's rows and key range.
  const int c = lane & 31;          // MFMA column = row of this lane
  const int h = lane >> 5;          // lane half
  const int rw0 = r0 + 32 * w;
  const int r = rw0 + c;
  const int qi = r / G;
  const int wave_rows = max(0, min(32, R - rw0));
  int kend_w = 0;                  // keys [0, kend_w) can be visible to this wave
  if (wave_rows > 0) {
    kend_w = L;
    if (p.causal) kend_w = min(L, (rw0 + wave_rows - 1) / G + off + 1);
    kend_w = max(kend_w, 0);
  }
  const int wg_rows = max(0, min(ROWS, R - r0));
  int kend = L;
  if (p.causal) kend = min(L, (r0 + wg_rows - 1) / G + off + 1);
  kend = max(kend, 0);
  // First key that some row of the wave cannot see (causal diagonal).
  const int kfull_w = p.causal ? max(0, rw0 / G + off + 1) : L;

  // Q^T as the B operand (hoisted): lane holds Q[row r][16*ks + 8*h .. +7].
  bf16x8_t qf[8];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
    const int qh = kvh * G + (r % G);
    const int64_t qoff = (int64_t)b * p.qs_b + (int64_t)qi * p.qs_t + (int64_t)qh * p.qs_h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      i32x4_t v = {0, 0, 0, 0};
      if (r < R) v = *reinterpret_cast<const i32x4_t*>(qp + qoff + 16 * ks + 8 * h);
      qf[ks] = as_bf16x8(v);
    }
  }

  // K/V global -> LDS copy: thread t moves chunks t and t + NT of each tile
  // (chunk x: key x / 16, 16-byte column x % 16).
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;
  const uint32_t kst = (uint32_t)(p.ks_t * 2), vst = (uint32_t)(p.vs_t * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)L * kst);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (uint32_t)L * vst);
  const int ck0 = t >> 4, cc = t & 15;  // chunk t: key ck0, column cc; chunk t+NT: key ck0+32
  i32x4_t stg[4];
  auto gload = [&](int k0) {
    stg[0] = buf_load16(krs, (uint32_t)(k0 + ck0) * kst + 16 * cc);
    stg[1] = buf_load16(krs, (uint32_t)(k0 + ck0 + 32) * kst + 16 * cc);
    stg[2] = buf_load16(vrs, (uint32_t)(k0 + ck0) * vst + 16 * cc);
    stg[3] = buf_load16(vrs, (uint32_t)(k0 + ck0 + 32) * vst + 16 * cc);
  };
  auto lstore = [&](int stage) {
    char* kl = smem + stage * STAGE;
    char* vl = kl + K_TILE;
    *reinterpret_cast<i32x4_t*>(kl + ck0 * K_STRIDE + 16 * cc) = stg[0];
    *reinterpret_cast<i32x4_t*>(kl + (ck0 + 32) * K_STRIDE + 16 * cc) = stg[1];
    *reinterpret_cast<i32x4_t*>(vl + ck0 * V_STRIDE + 16 * cc) = stg[2];
    *reinterpret_cast<i32x4_t*>(vl + (ck0 + 32) * V_STRIDE + 16 * cc) = stg[3];
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = kNegInf, l_part = 0.f;
  const float sl2 = p.scale_log2;
  const int qlim = qi + off;  // last visible key of this lane's row (causal)

  // Per-lane LDS byte offsets that do not depend on the tile.
  const int k_rd = c * K_STRIDE + 16 * h;                     // + 32*ks + 32*kb*K_STRIDE
  const int gq = lane >> 4, li = lane & 15;
  const int v_rd = (4 * (gq >> 1) + (li >> 2)) * V_STRIDE + 2 * (16 * (gq & 1) + 4 * (li & 3));

  const int ntiles = (kend + TK - 1) / TK;
  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * TK;
    const bool more = it + 1 < ntiles;
    if (more) gload(k0 + TK);
    if (k0 < kend_w) {
      const char* kl = smem + (it & 1) * STAGE;
      const char* vl = kl + K_TILE;
      // S^T for the two 32-key blocks.
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16_t a;
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const i32x4_t kf = *reinterpret_cast<const i32x4_t*>(kl + kb * 32 * K_STRIDE + k_rd + 32 * ks);
          a = mfma32x32x16(as_bf16x8(kf), qf[ks], a);
        }
        s[kb] = a;
      }
      // Scale to base-2 units; mask only tiles that cross the diagonal or the end.
      const bool need_mask = (k0 + TK > kfull_w) || (k0 + TK > L) || (r >= R);
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = s[kb][e] * sl2;
          if (need_mask) {
            const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3);
            const bool vis = key < L && (!p.causal || key <= qlim) && r < R;
            v = vis ? v : kNegInf;
          }
          s[kb][e] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      float alpha = 1.f;
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      if (m_new != kNegInf) alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pv = fast_exp2(s[kb][e] - m_use);
          s[kb][e] = pv;
          ps += pv;
        }
      l_part = l_part * alpha + ps;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;

      // O^T += V^T P^T, four 16-key k-steps.
#pragma unroll
      for (int ts = 0; ts < 4; ++ts) {
        const int kb = ts >> 1, i0 = 2 * (ts & 1);
        i32x4_t pk;
        pk[0] = (int)pack_bf16x2(s[kb][4 * i0 + 0], s[kb][4 * i0 + 1]);
        pk[1] = (int)pack_bf16x2(s[kb][4 * i0 + 2], s[kb][4 * i0 + 3]);
        pk[2] = (int)pack_bf16x2(s[kb][4 * i0 + 4], s[kb][4 * i0 + 5]);
        pk[3] = (int)pack_bf16x2(s[kb][4 * i0 + 6], s[kb][4 * i0 + 7]);
        const bf16x8_t pb = as_bf16x8(pk);
        const char* vrow = vl + (16 * ts) * V_STRIDE + v_rd;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const i32x2_t lo = ds_read_tr(vrow + 64 * db);
          const i32x2_t hi = ds_read_tr(vrow + 8 * V_STRIDE + 64 * db);
          i32x4_t va;
          va[0] = lo[0];
          va[1] = lo[1];
          va[2] = hi[0];
          va[3] = hi[1];
          oacc[db] = mfma32x32x16(as_bf16x8(va), pb, oacc[db]);
        }
      }
    }
    if (more) lstore((it + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = U / l (division after the V-matmul), LSE = m + log l.
  float l_row = l_part + __shfl_xor(l_part, 32, 64);
  if (r < R) {
    const int qh = kvh * G + (r % G);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const int64_t obase = (int64_t)b * p.os_b + (int64_t)qi * p.os_t + (int64_t)qh * p.os_h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * h;
        const float o0 = oacc[db][4 * i + 0] * inv, o1 = oacc[db][4 * i + 1] * inv;
        const float o2 = oacc[db][4 * i + 2] * inv, o3 = oacc[db][4 * i + 3] * inv;
        if (p.o_bf16) {
          uint2 pk;
          pk.x = pack_bf16x2(o0, o1);
          pk.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.o) + obase + d) = pk;
        } else {
          float4 v = make_float4(o0, o1, o2, o3);
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.o) + obase + d) = v;
        }
      }
    if (h == 0 && p.lse_out)
      p.lse_out[((int64_t)b * p.Lq + qi) * p.Hq + qh] =
          l_row > 0.f ? (m_run + fast_log2(l_row)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_prefill_d128(const KParams& p, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_d128_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nrt = (p.rows + ROWS - 1) / ROWS;
  const int64_t nwg = (int64_t)p.B * p.Hkv * nrt;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_d128_kernel, dim3((unsigned)nwg), dim3(NT), LDS_BYTES, s, p, nrt);
  return hipGetLastError();
}

}  // namespace attn

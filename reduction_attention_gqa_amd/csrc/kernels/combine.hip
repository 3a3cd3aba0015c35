// Combine kernel: merges the split partials of every output row.
//
// The split kernel leaves, per split j of a row, O_j (already divided by the
// split's own row sum) and LSE_j.  Cleave §4 / Fig. 5(b) reduces the per-split
// row sums and value-products over s and then divides; with each partial taken
// relative to its own max that is the log-sum-exp merge
//   M = max_j LSE_j,  w_j = 2^((LSE_j - M) log2 e),  O = sum_j w_j O_j / sum_j w_j.
// One wave per row; lanes own 4 consecutive output columns (16-byte loads).
#include "../attn_internal.hpp"
#include "common.hpp"
#include "layout.hpp"

namespace attn {
namespace {

constexpr int kRowsPerBlock = 4;

__global__ __launch_bounds__(64 * kRowsPerBlock) void combine_kernel(KParams p) {
  const int lane = threadIdx.x % 64;
  const int64_t nrows = (int64_t)p.B * p.Lq * p.Hq;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / 64;
  if (row >= nrows) return;
  const int h = (int)(row % p.Hq);
  const int i = (int)((row / p.Hq) % p.Lq);
  const int b = (int)(row / ((int64_t)p.Hq * p.Lq));
  const int L = kv_len_b(p, b);
  int sb = L == 0 ? 0 : (L + p.chunk - 1) / p.chunk;
  const int64_t obase = (int64_t)b * p.os_b + (int64_t)i * p.os_t + (int64_t)h * p.os_h;
  if (sb > p.s_max) {
    // More keys on the device than the plan split: some were never reduced.
    // NaN marks the row instead of a silently truncated result.
    const float nan = __builtin_nanf("");
    for (int d = lane; d < p.Dv; d += 64) {
      if (p.o_bf16)
        reinterpret_cast<uint16_t*>(p.o)[obase + d] = 0x7fc0;
      else
        reinterpret_cast<float*>(p.o)[obase + d] = nan;
    }
    if (lane == 0 && p.lse_out) p.lse_out[row] = nan;
    return;
  }

  float m = kNegInf;
  for (int j = lane; j < sb; j += 64) m = fmaxf(m, p.ws_lse[(int64_t)j * nrows + row]);
  m = wave_max(m);

  if (m == kNegInf) {  // no split saw a key: O = 0, LSE = -inf
    for (int d = lane; d < p.Dv; d += 64) {
      if (p.o_bf16)
        reinterpret_cast<uint16_t*>(p.o)[obase + d] = 0;
      else
        reinterpret_cast<float*>(p.o)[obase + d] = 0.f;
    }
    if (lane == 0 && p.lse_out) p.lse_out[row] = kNegInf;
    return;
  }
  const float m2 = m * kLog2e;
  float wsum = 0.f;
  for (int j = lane; j < sb; j += 64)
    wsum += fast_exp2(p.ws_lse[(int64_t)j * nrows + row] * kLog2e - m2);
  wsum = wave_sum(wsum);
  const float inv = 1.f / wsum;

  if ((p.Dv & 3) == 0) {
    for (int d = lane * 4; d < p.Dv; d += 256) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < sb; ++j) {
        const int64_t slot = (int64_t)j * nrows + row;
        const float w = fast_exp2(p.ws_lse[slot] * kLog2e - m2);
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(p.ws_o + slot * p.Dv + d);
        a += w * x;
      }
      a *= inv;
      if (p.o_bf16) {
        uint2 pk;
        pk.x = pack_bf16x2(a[0], a[1]);
        pk.y = pack_bf16x2(a[2], a[3]);
        uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + obase + d;
        if ((reinterpret_cast<uintptr_t>(op) & 7) == 0) {
          *reinterpret_cast<uint2*>(op) = pk;
        } else {
          op[0] = (uint16_t)(pk.x & 0xffff);
          op[1] = (uint16_t)(pk.x >> 16);
          op[2] = (uint16_t)(pk.y & 0xffff);
          op[3] = (uint16_t)(pk.y >> 16);
        }
      } else {
        float* op = reinterpret_cast<float*>(p.o) + obase + d;
        op[0] = a[0];
        op[1] = a[1];
        op[2] = a[2];
        op[3] = a[3];
      }
    }
  } else {
    for (int d = lane; d < p.Dv; d += 64) {
      float a = 0.f;
      for (int j = 0; j < sb; ++j) {
        const int64_t slot = (int64_t)j * nrows + row;
        a += fast_exp2(p.ws_lse[slot] * kLog2e - m2) * p.ws_o[slot * p.Dv + d];
      }
      a *= inv;
      if (p.o_bf16)
        reinterpret_cast<uint16_t*>(p.o)[obase + d] = (uint16_t)f32_to_bf16_bits(a);
      else
        reinterpret_cast<float*>(p.o)[obase + d] = a;
    }
  }
  if (lane == 0 && p.lse_out) p.lse_out[row] = m + fast_log2(wsum) * kLn2;
}

}  // namespace

hipError_t launch_combine(const KParams& p, hipStream_t s) {
  const int64_t nrows = (int64_t)p.B * p.Lq * p.Hq;
  if (nrows == 0) return hipSuccess;
  const dim3 grid((unsigned)((nrows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(64 * kRowsPerBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn

// Device helpers for gfx950 (CDNA4, wave64) kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even, on
// gfx950's v_cvt_pk_bf16_f32 (one instruction, no branches).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Raw buffer resource: out-of-range loads (offset >= num_bytes) return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
__device__ __forceinline__ i32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// D = A * B + C on 16x16x32 bf16 tiles.  Lane l holds A[row = l%16][k = 8*(l/16) .. +7],
// B[k = 8*(l/16) .. +7][col = l%16], and D/C[row = 4*(l/16) .. +3][col = l%16].
__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D = A * B + C on 32x32x16 bf16 tiles.  Lane l holds A[row = l%32][k = 8*(l/32) .. +7],
// B[k = 8*(l/32) .. +7][col = l%32], and D/C[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32]
// for i = 0..15.
__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b,
                                                 const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const i32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Device-coherent (sc1) stores and loads for single-launch merges.  They do
// not stay dirty in one XCD's L2 and do not hit stale lines there, so a
// partial published by one workgroup and read by another after an arrival
// counter needs no whole-L2 write-back or invalidate (which a device-scope
// release/acquire fence would issue for ordinary stores and loads).
__device__ __forceinline__ void store_dev(float* ptr, float v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* ptr) {
  return __hip_atomic_load(const_cast<float*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Sixteen-byte versions through a buffer resource, with the same
// device-coherent cache policy (sc1, cache-policy bit 4 of the buffer
// instructions).
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ void store16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r, (int)off, 0,
                                         kCachePolicySc1);
}
__device__ __forceinline__ f32x4_t load16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicySc1));
}
// s_waitcnt vmcnt(0): every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Key count of request b, clamped to [0, cap].
__device__ __forceinline__ int kv_len_of(const int32_t* lens, int b, int cap) {
  if (lens == nullptr) return cap;
  int n = lens[b];
  return n < 0 ? 0 : (n > cap ? cap : n);
}

}  // namespace attn

// attn_decode_noalloc: attn_decode with its workspace in a device-resident
// array of this library instead of caller memory, for callers that cannot
// allocate (code under graph capture, tight serving loops).
//
// The array `scratch` holds, from its start: kScratchCntBytes of arrival
// counters (int32, zero between calls), then ws_lse and ws_o, each aligned to
// 256 bytes.  A plan whose workspace does not fit is rejected before anything
// is enqueued.  The host never passes `scratch` itself to a kernel (in host
// code the name is a stand-in, not a device address): the device address is
// looked up once per device with hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../attn_internal.hpp"
#include "attn_mi355x.h"

namespace attn {
namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

__global__ void zero_words(int32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Device address of the current device's scratch array.  The first call on a
// device looks it up and clears the counter region (a fill kernel on the
// caller's stream, ahead of the decode that follows on that stream).
int scratch_of_current_device(char** out, hipStream_t s) {
  static std::mutex mu;
  static std::vector<char*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return report_error(ATTN_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return report_error(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s",
                          hipGetErrorString(e));
    hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, s, reinterpret_cast<int32_t*>(ptr),
                       (int64_t)(kScratchCntBytes / 4));
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess)
      return report_error(ATTN_ERR_HIP, "clearing the scratch counters failed: %s",
                          hipGetErrorString(le));
    ptrs[dev] = static_cast<char*>(ptr);
  }
  *out = ptrs[dev];
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

extern "C" int attn_decode_noalloc(const attn_problem* problem, const attn_plan* plan,
                                   const void* q, const void* k, const void* v, void* o,
                                   float* lse_out, void* stream) {
  using namespace attn;
  clear_error();
  if (!plan) return report_error(ATTN_ERR_ARG, "plan is NULL");
  const uint64_t lse_off = kScratchCntBytes;
  const uint64_t o_off = lse_off + align256(plan->ws_lse_bytes);
  if (plan->ws_cnt_bytes > kScratchCntBytes || o_off + plan->ws_o_bytes > kScratchBytes)
    return report_error(ATTN_ERR_WORKSPACE,
                        "the plan's workspace (%llu + %llu + %llu bytes) exceeds the library's "
                        "scratch (%llu bytes of partials, %llu of counters)",
                        (unsigned long long)plan->ws_o_bytes,
                        (unsigned long long)plan->ws_lse_bytes,
                        (unsigned long long)plan->ws_cnt_bytes,
                        (unsigned long long)(kScratchBytes - kScratchCntBytes),
                        (unsigned long long)kScratchCntBytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = nullptr;
  if (int st = scratch_of_current_device(&base, s)) return st;
  return attn_decode(problem, plan, q, k, v, reinterpret_cast<float*>(base + o_off),
                     kScratchBytes - o_off, reinterpret_cast<float*>(base + lse_off),
                     o_off - lse_off, reinterpret_cast<int32_t*>(base), kScratchCntBytes, o,
                     lse_out, stream);
}

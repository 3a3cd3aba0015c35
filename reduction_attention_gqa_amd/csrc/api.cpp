// C-ABI front end: argument checks, the split planner, kernel selection and launch.
// Every check runs before anything is enqueued; no exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <utility>
#include <vector>

#include "attn_internal.hpp"
#include "attn_mi355x.h"
#include "rmsnorm_matmul.h"
#include "swiglu.h"

namespace attn {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, cached per device id.
int device_cu_count(int* out) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    cache[dev] = n;
  }
  *out = cache[dev];
  return 0;
}

int check_problem(const attn_problem* p) {
  if (!p) return fail(ATTN_ERR_ARG, "problem is NULL");
  if (p->reserved0 != 0) return fail(ATTN_ERR_ARG, "reserved0 must be 0");
  if ((p->dtype != ATTN_F32 && p->dtype != ATTN_BF16) ||
      (p->o_dtype != ATTN_F32 && p->o_dtype != ATTN_BF16))
    return fail(ATTN_ERR_ARG, "dtype/o_dtype must be ATTN_F32 or ATTN_BF16");
  if (p->batch < 0) return fail(ATTN_ERR_ARG, "batch < 0");
  if (p->q_heads < 1 || p->kv_heads < 1) return fail(ATTN_ERR_ARG, "head counts must be >= 1");
  if (p->q_heads % p->kv_heads != 0)
    return fail(ATTN_ERR_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", p->q_heads,
                p->kv_heads);
  if (p->head_dim_qk < 1 || p->head_dim_v < 1) return fail(ATTN_ERR_ARG, "head dims must be >= 1");
  if (p->q_len < 1) return fail(ATTN_ERR_ARG, "q_len < 1");
  if (p->kv_len_max < 0) return fail(ATTN_ERR_ARG, "kv_len_max < 0");
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_ERR_ARG, "causal must be 0 or 1");
  if (!std::isfinite(p->scale)) return fail(ATTN_ERR_ARG, "scale is not finite");
  for (int a = 0; a < 3; ++a)
    if (p->q_stride[a] < 0 || p->k_stride[a] < 0 || p->v_stride[a] < 0 || p->o_stride[a] < 0)
      return fail(ATTN_ERR_ARG, "strides must be >= 0");
  if (p->head_dim_qk > 768 || p->head_dim_v > 512)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim_qk > 768 or head_dim_v > 512");
  if (p->reserved1 != 0) return fail(ATTN_ERR_ARG, "reserved1 must be 0");
  if (p->kv_indptr && (p->kv_lens || p->page_table))
    return fail(ATTN_ERR_ARG, "kv_indptr excludes kv_lens and page_table");
  if (p->page_table) {
    if (p->page_size < 1) return fail(ATTN_ERR_ARG, "page_size < 1");
    if (p->num_pages < 1) return fail(ATTN_ERR_ARG, "num_pages < 1");
    if ((int64_t)p->pages_per_req * p->page_size < p->kv_len_max)
      return fail(ATTN_ERR_ARG, "pages_per_req * page_size (%lld) < kv_len_max (%d)",
                  (long long)p->pages_per_req * p->page_size, p->kv_len_max);
  } else if (p->page_size != 0 || p->pages_per_req != 0 || p->num_pages != 0) {
    return fail(ATTN_ERR_ARG, "page_size, pages_per_req and num_pages must be 0 without page_table");
  }
  return ATTN_OK;
}

// Decode entry points take one query tensor of uniform Lq rows per request.
int check_decode_layout(const attn_problem* p) {
  if (p->q_indptr)
    return fail(ATTN_ERR_UNSUPPORTED, "packed queries (q_indptr) are a prefill layout");
  return ATTN_OK;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2_of(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

uint64_t problem_key(const attn_problem* p) {
  // The output dtype is not part of the key: the split partials are fp32 either way.
  // The layout kind (packed, paged and the page size) selects kernels and
  // bounds the split size, so it is part of the key; the arrays are not.
  const int32_t f[] = {p->dtype, p->batch, p->q_heads, p->kv_heads, p->head_dim_qk,
                       p->head_dim_v, p->q_len, p->kv_len_max, p->causal,
                       p->q_indptr != nullptr, p->kv_indptr != nullptr,
                       p->page_table ? p->page_size : 0};
  uint64_t h = 1469598103934665603ull;
  for (int32_t x : f) {
    for (int s = 0; s < 32; s += 8) {
      h ^= (uint64_t)((x >> s) & 0xff);
      h *= 1099511628211ull;
    }
  }
  return h | 1ull;  // never 0, so a zeroed plan is always rejected
}

float scale_of(const attn_problem* p) {
  return p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->head_dim_qk);
}

KParams base_params(const attn_problem* p) {
  KParams k;
  std::memset(&k, 0, sizeof(k));
  k.kv_lens = p->kv_lens;
  k.q_indptr = p->q_indptr;
  k.kv_indptr = p->kv_indptr;
  k.page_table = p->page_table;
  k.page_size = p->page_table ? p->page_size : 1;
  k.ppr = p->pages_per_req;
  k.num_pages = p->num_pages;
  k.page_shift = is_pow2(k.page_size) ? log2_of(k.page_size) : -1;
  k.qs_b = p->q_stride[0]; k.qs_t = p->q_stride[1]; k.qs_h = p->q_stride[2];
  k.ks_b = p->k_stride[0]; k.ks_t = p->k_stride[1]; k.ks_h = p->k_stride[2];
  k.vs_b = p->v_stride[0]; k.vs_t = p->v_stride[1]; k.vs_h = p->v_stride[2];
  k.os_b = p->o_stride[0]; k.os_t = p->o_stride[1]; k.os_h = p->o_stride[2];
  k.B = p->batch; k.Hq = p->q_heads; k.Hkv = p->kv_heads; k.G = p->q_heads / p->kv_heads;
  k.Dqk = p->head_dim_qk; k.Dv = p->head_dim_v; k.Lq = p->q_len; k.Lcap = p->kv_len_max;
  k.causal = p->causal;
  k.in_bf16 = p->dtype == ATTN_BF16;
  k.o_bf16 = p->o_dtype == ATTN_BF16;
  k.rows = k.G * k.Lq;
  k.row_tile = kGenericRowTile;
  k.scale_log2 = scale_of(p) * 1.44269504088896340736f;
  k.div_dqk = make_fastdiv(std::max(k.Dqk, 1));
  k.div_dv = make_fastdiv(std::max(k.Dv, 1));
  k.div_g = make_fastdiv(std::max(k.G, 1));
  return k;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// Shape-level kernel choice for decode (pointers are checked at launch).
// Paged K/V runs on the MFMA kernels when the page size is a power of two,
// and on the generic kernel otherwise.
int decode_family(const attn_problem* p) {
  const int rows = (p->q_heads / p->kv_heads) * p->q_len;
  if (p->dtype == ATTN_BF16 && p->head_dim_qk == 128 && p->head_dim_v == 128 &&
      rows <= kGqaMaxRows && (!p->page_table || is_pow2(p->page_size)))
    return ATTN_KERNEL_GQA_D128;
  if (p->dtype == ATTN_BF16 && p->head_dim_qk == 576 && p->head_dim_v == 512 && rows <= kMlaRows &&
      (!p->page_table || is_pow2(p->page_size)))
    return ATTN_KERNEL_MLA;
  return ATTN_KERNEL_GENERIC;
}

// Longest split a paged MFMA decode kernel accepts: its page ids fit in LDS.
int64_t paged_max_chunk(const attn_problem* p, int family) {
  if (family == ATTN_KERNEL_MLA) return (int64_t)(kMlaPageIds - 1) * p->page_size / kMlaTileN * kMlaTileN;
  return (int64_t)(kGqaPageIds - 1) * p->page_size / kGqaTileN * kGqaTileN;
}

// Workgroups per compute unit the planner aims for, by kernel family.
int target_wgs_per_cu(int family) {
  switch (family) {
    case ATTN_KERNEL_GQA_D128: return kGqaItemsPerCu;
    case ATTN_KERNEL_MLA: return 1;  // one 8-wave workgroup fills a CU (LDS ring)
    default: return 4;
  }
}

int tile_n_of(int family) {
  switch (family) {
    case ATTN_KERNEL_GQA_D128: return kGqaTileN;
    case ATTN_KERNEL_MLA: return kMlaTileN;
    default: return kGenericTileN;
  }
}

// Can the MFMA GQA kernel run on these pointers/strides?  (16-byte rows,
// 32-bit buffer offsets.)
bool gqa_d128_fits(const attn_problem* p, const void* q, const void* k, const void* v) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return false;
  for (int a = 0; a < 3; ++a)
    if ((p->q_stride[a] | p->k_stride[a] | p->v_stride[a]) & 7) return false;
  // Paged rows are addressed with 64-bit pointers, not buffer offsets.
  if (p->page_table) return true;
  // Buffer offsets reach up to 64 rows past the last key (clamped block starts).
  const int64_t kbytes = ((int64_t)p->kv_len_max + 64) * p->k_stride[1] * 2 + 256;
  const int64_t vbytes = ((int64_t)p->kv_len_max + 64) * p->v_stride[1] * 2 + 256;
  return kbytes < (1ll << 31) && vbytes < (1ll << 31);
}

// Can the MLA kernel run?  V must be the first Dv columns of K (same pointer
// and strides), with 16-byte rows and 32-bit buffer offsets.
bool mla_fits(const attn_problem* p, const void* q, const void* k, const void* v) {
  if (v != k) return false;
  for (int a = 0; a < 3; ++a)
    if (p->v_stride[a] != p->k_stride[a]) return false;
  return gqa_d128_fits(p, q, k, v);
}

// Can the MFMA prefill kernel run on these pointers/strides?
bool prefill_d128_fits(const attn_problem* p, const void* q, const void* k, const void* v,
                       const void* o) {
  if (p->dtype != ATTN_BF16 || p->head_dim_qk != 128 || p->head_dim_v != 128) return false;
  // Paged: a power-of-two page size, and the page ids of the longest request
  // fit in the workgroup's LDS table.
  if (p->page_table && (!is_pow2(p->page_size) ||
                        ceil_div(p->kv_len_max, p->page_size) > kPrefillPageIds))
    return false;
  if (!gqa_d128_fits(p, q, k, v)) return false;
  const int oal = p->o_dtype == ATTN_BF16 ? 8 : 16;
  if ((reinterpret_cast<uintptr_t>(o) & (oal - 1)) != 0) return false;
  for (int a = 0; a < 3; ++a)
    if (p->o_stride[a] & 3) return false;
  const int64_t rows = (int64_t)(p->q_heads / p->kv_heads) * p->q_len;
  return rows < (1ll << 30);
}

// The GQA kernel for a plan: pointers and strides fit, and a paged split's
// page ids fit in the kernel's LDS table.
bool gqa_d128_usable(const attn_problem* p, const attn_plan* plan, const void* q, const void* k,
                     const void* v) {
  if (p->page_table &&
      (!is_pow2(p->page_size) || plan->chunk > paged_max_chunk(p, ATTN_KERNEL_GQA_D128)))
    return false;
  return gqa_d128_fits(p, q, k, v);
}

bool mla_usable(const attn_problem* p, const attn_plan* plan, const void* q, const void* k,
                const void* v) {
  if (p->page_table &&
      (!is_pow2(p->page_size) || plan->chunk > paged_max_chunk(p, ATTN_KERNEL_MLA)))
    return false;
  return mla_fits(p, q, k, v);
}

int check_ptrs(const void* a, const char* na, const void* b, const char* nb, const void* c,
               const char* nc) {
  if (!a) return fail(ATTN_ERR_ARG, "%s is NULL", na);
  if (!b) return fail(ATTN_ERR_ARG, "%s is NULL", nb);
  if (!c) return fail(ATTN_ERR_ARG, "%s is NULL", nc);
  return ATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace

void clear_error() { g_err[0] = 0; }

int report_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

hipError_t set_lds_limit_once(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<int, const void*>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({dev, kernel})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({dev, kernel});
  return e;
}

}  // namespace attn

using namespace attn;

extern "C" {

int attn_version(void) { return ATTN_MI355X_VERSION; }

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported problem";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_err; }

int attn_decode_plan(const attn_problem* problem, int32_t s_request, const int32_t* kv_lens_host,
                     int32_t num_cus, attn_plan* out) {
  g_err[0] = 0;
  if (!out) return fail(ATTN_ERR_ARG, "plan output is NULL");
  std::memset(out, 0, sizeof(*out));
  if (int st = check_problem(problem)) return st;
  if (int st = check_decode_layout(problem)) return st;
  const attn_problem* p = problem;
  int cus = num_cus;
  if (cus <= 0 && device_cu_count(&cus) != 0)
    return fail(ATTN_ERR_HIP, "cannot query the compute-unit count of the current device");

  const int family = decode_family(p);
  int tile_n = tile_n_of(family);
  const int G = p->q_heads / p->kv_heads;
  const int rows = G * p->q_len;
  const int row_tiles = family == ATTN_KERNEL_GENERIC ? (int)ceil_div(rows, kGenericRowTile) : 1;
  const int64_t units_per_req = (int64_t)p->kv_heads * row_tiles;

  // Lengths as the kernels will see them.
  int64_t lmax = 0, tiles_total = 0, keys_total = 0;
  for (int b = 0; b < p->batch; ++b) {
    int64_t n = kv_lens_host ? kv_lens_host[b] : p->kv_len_max;
    n = std::min<int64_t>(std::max<int64_t>(n, 0), p->kv_len_max);
    lmax = std::max(lmax, n);
    keys_total += n;
    tiles_total += ceil_div(n, tile_n);
  }

  // GQA D=128: when there are at least as many (request, KV head) units as
  // compute units and no request is much longer than the mean, one split per
  // request (no partials, no merge); otherwise the key axis is split to about
  // kGqaItemsPerCu items per CU.
  bool one_split = false;
  if (family == ATTN_KERNEL_GQA_D128 && p->batch > 0) {
    const bool balanced = lmax * 4 * p->batch <= keys_total * 5;
    one_split = s_request == 1 ||
        (s_request <= 0 && (int64_t)p->batch * p->kv_heads >= cus && balanced);
  }

  int64_t s_max = 1, chunk = tile_n;
  if (lmax > 0) {
    const int64_t max_tiles = ceil_div(lmax, tile_n);
    if (one_split) {
      chunk = max_tiles * tile_n;
    } else if (s_request > 0) {
      s_max = std::min<int64_t>(s_request, max_tiles);
      chunk = ceil_div(ceil_div(lmax, s_max), tile_n) * tile_n;
    } else {
      // Aim for a family-specific number of workgroups per compute unit, with at
      // least two tiles per split so the per-split prologue and epilogue stay
      // small.  The generic family takes one tile per split when its work does
      // not fill the GPU anyway (a small problem's latency is that of its
      // longest split), and at most kGenericTileN splits, the most its
      // single-launch merge tabulates in LDS.
      const int64_t target_wgs = (int64_t)cus * target_wgs_per_cu(family);
      const int64_t work_tiles = tiles_total * units_per_req;
      int64_t chunk_tiles = ceil_div(work_tiles, target_wgs);
      if (family != ATTN_KERNEL_GENERIC || work_tiles > target_wgs)
        chunk_tiles = std::max<int64_t>(chunk_tiles, 2);
      if (family == ATTN_KERNEL_GENERIC)
        chunk_tiles = std::max<int64_t>(chunk_tiles, ceil_div(max_tiles, kGenericTileN));
      chunk_tiles = std::min<int64_t>(chunk_tiles, max_tiles);
      chunk = chunk_tiles * tile_n;
    }
    // The paged MFMA kernels stage one split's page ids in LDS.
    if (family != ATTN_KERNEL_GENERIC && p->page_table)
      chunk = std::min<int64_t>(chunk, paged_max_chunk(p, family));
    s_max = ceil_div(lmax, chunk);
  }
  if (s_max > 65535) return fail(ATTN_ERR_UNSUPPORTED, "too many splits (%lld)", (long long)s_max);
  // Work items (request, KV head, split) of the one-dimensional GQA grid; an
  // empty request still owns one item per KV head (it writes O = 0).
  int64_t n_items = 0;
  for (int b = 0; b < p->batch; ++b) {
    int64_t n = kv_lens_host ? kv_lens_host[b] : p->kv_len_max;
    n = std::min<int64_t>(std::max<int64_t>(n, 0), p->kv_len_max);
    n_items += (int64_t)p->kv_heads * std::max<int64_t>(1, ceil_div(n, chunk));
  }
  if (n_items > (1ll << 31) - 64)
    return fail(ATTN_ERR_UNSUPPORTED, "too many work items (%lld)", (long long)n_items);

  out->kernel = family;
  out->s_max = (int32_t)s_max;
  out->chunk = (int32_t)chunk;
  out->tile_n = tile_n;
  out->rows_per_unit = rows;
  out->row_tiles = row_tiles;
  if (family == ATTN_KERNEL_GENERIC) {
    out->grid[0] = (uint32_t)s_max;
    out->grid[1] = (uint32_t)row_tiles;
    out->grid[2] = (uint32_t)((int64_t)p->batch * p->kv_heads);
    out->block = kGenericBlock;
  } else if (family == ATTN_KERNEL_GQA_D128) {
    out->grid[0] = (uint32_t)(ceil_div(n_items, 8) * 8);  // workgroup x runs on XCD x % 8
    out->grid[1] = 1;
    out->grid[2] = 1;
    out->block = kGqaBlock;
  } else {
    out->grid[0] = (uint32_t)s_max;
    out->grid[1] = (uint32_t)p->kv_heads;
    out->grid[2] = (uint32_t)p->batch;
    out->block = kMlaBlock;
  }
  out->n_items = n_items;
  if (family == ATTN_KERNEL_GQA_D128) {
    // attn_decode: rounds of tile_n keys of every unit laid end to end, equal
    // runs per workgroup (one per compute unit), pieces per unit.
    int64_t rounds = 0;
    std::vector<int64_t> unit_rounds((size_t)p->batch);
    for (int b = 0; b < p->batch; ++b) {
      int64_t n = kv_lens_host ? kv_lens_host[b] : p->kv_len_max;
      n = std::min<int64_t>(std::max<int64_t>(n, 0), p->kv_len_max);
      unit_rounds[(size_t)b] = std::max<int64_t>(1, ceil_div(n, tile_n));
      rounds += unit_rounds[(size_t)b] * p->kv_heads;
    }
    // Most pieces any unit is cut into by `grid` equal runs.
    auto max_pieces = [&](int64_t grid) {
      int64_t pieces = 1, u0 = 0;
      for (int b = 0; b < p->batch; ++b)
        for (int h = 0; h < p->kv_heads; ++h) {
          const int64_t u1 = u0 + unit_rounds[(size_t)b];
          const int64_t g_first = ((u0 + 1) * grid + rounds - 1) / rounds - 1;
          const int64_t g_last = (u1 * grid + rounds - 1) / rounds - 1;
          pieces = std::max(pieces, g_last - g_first + 1);
          u0 = u1;
        }
      return pieces;
    };
    // One run per compute unit when no unit is cut (e.g. equal lengths whose
    // units fill the runs exactly: one long stream per compute unit, no
    // merge); otherwise two runs per compute unit, whose two workgroups hide
    // each other's piece boundaries and merges (measured on ragged lengths:
    // 274 us against 305 us with one run per compute unit).
    int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cus, rounds));
    int64_t pieces = max_pieces(grid);
    if (pieces > 1) {
      grid = std::max<int64_t>(1, std::min<int64_t>((int64_t)cus * kGqaStreamWgsPerCu, rounds));
      pieces = max_pieces(grid);
    }
    if (pieces > 65535 || rounds > (1ll << 40))
      return fail(ATTN_ERR_UNSUPPORTED, "too many pieces or rounds for the stream decode");
    out->stream_rounds = rounds;
    out->stream_grid = (int32_t)grid;
    out->stream_pieces = (int32_t)pieces;
  }
  const uint64_t nrows = (uint64_t)p->batch * p->q_len * p->q_heads;
  out->ws_o_bytes = (uint64_t)s_max * nrows * p->head_dim_v * sizeof(float);
  out->ws_lse_bytes = (uint64_t)s_max * nrows * sizeof(float);
  if (family == ATTN_KERNEL_GQA_D128) {
    // The stream kernel's partials: an 8 KiB block (16 rows x 128 floats in
    // thread order) and 16 LSEs per (piece, unit).
    const uint64_t units = (uint64_t)p->batch * p->kv_heads;
    out->ws_o_bytes = std::max<uint64_t>(out->ws_o_bytes,
                                         (uint64_t)out->stream_pieces * units * 16 * 128 * 4);
    out->ws_lse_bytes = std::max<uint64_t>(out->ws_lse_bytes,
                                           (uint64_t)out->stream_pieces * units * 16 * 4);
  }
  if (family == ATTN_KERNEL_MLA) {
    // The single-launch MLA merge keeps each split's partial in the kernel's
    // lane order, whole 16-row wave blocks per (request, KV head).
    const uint64_t rows16 = (uint64_t)ceil_div(rows, 16) * 16;
    const uint64_t units = (uint64_t)p->batch * p->kv_heads;
    out->ws_o_bytes = std::max<uint64_t>(out->ws_o_bytes,
                                         (uint64_t)s_max * units * rows16 * p->head_dim_v * 4);
    out->ws_lse_bytes = std::max<uint64_t>(out->ws_lse_bytes, (uint64_t)s_max * units * rows16 * 4);
  }
  // Arrival counters of the single launch: one per (request, KV head), and
  // per row tile for the generic family.
  out->ws_cnt_bytes = (uint64_t)p->batch * p->kv_heads * row_tiles * sizeof(int32_t);
  out->problem_key = problem_key(p);
  return ATTN_OK;
}

int attn_decode_split(const attn_problem* problem, const attn_plan* plan, const void* q,
                      const void* k, const void* v, float* ws_o, size_t ws_o_bytes, float* ws_lse,
                      size_t ws_lse_bytes, void* stream) {
  g_err[0] = 0;
  if (int st = check_problem(problem)) return st;
  if (int st = check_decode_layout(problem)) return st;
  const attn_problem* p = problem;
  if (!plan) return fail(ATTN_ERR_ARG, "plan is NULL");
  if (plan->problem_key != problem_key(p))
    return fail(ATTN_ERR_ARG, "plan was made for a different problem");
  if (plan->s_max < 1 || plan->chunk < 1) return fail(ATTN_ERR_ARG, "corrupt plan");
  if (p->batch == 0) return ATTN_OK;
  if (int st = check_ptrs(q, "q", k, "k", v, "v")) return st;
  if (!ws_o || !ws_lse) return fail(ATTN_ERR_ARG, "workspace pointer is NULL");
  if (ws_o_bytes < plan->ws_o_bytes || ws_lse_bytes < plan->ws_lse_bytes)
    return fail(ATTN_ERR_WORKSPACE, "workspace too small: need %llu + %llu bytes",
                (unsigned long long)plan->ws_o_bytes, (unsigned long long)plan->ws_lse_bytes);

  KParams kp = base_params(p);
  kp.q = q; kp.k = k; kp.v = v;
  kp.ws_o = ws_o; kp.ws_lse = ws_lse;
  kp.chunk = plan->chunk;
  kp.s_max = plan->s_max;
  kp.split_mode = 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  const dim3 unit_grid(plan->s_max, p->kv_heads, p->batch);
  kp.n_items = plan->n_items;
  if (plan->kernel == ATTN_KERNEL_GQA_D128 && gqa_d128_usable(p, plan, q, k, v))
    return hip_status(launch_decode_gqa_d128(kp, s), "decode_gqa_d128 launch");
  if (plan->kernel == ATTN_KERNEL_MLA && mla_usable(p, plan, q, k, v))
    return hip_status(launch_decode_mla(kp, unit_grid, s), "decode_mla launch");
  const int row_tiles = (int)ceil_div(kp.rows, kGenericRowTile);
  const dim3 grid(plan->s_max, row_tiles, (unsigned)((int64_t)p->batch * p->kv_heads));
  return hip_status(launch_generic(kp, grid, dim3(kGenericBlock), s), "generic split launch");
}

int attn_decode(const attn_problem* problem, const attn_plan* plan, const void* q, const void* k,
                const void* v, float* ws_o, size_t ws_o_bytes, float* ws_lse, size_t ws_lse_bytes,
                int32_t* ws_cnt, size_t ws_cnt_bytes, void* o, float* lse_out, void* stream) {
  g_err[0] = 0;
  if (int st = check_problem(problem)) return st;
  if (int st = check_decode_layout(problem)) return st;
  const attn_problem* p = problem;
  if (!plan) return fail(ATTN_ERR_ARG, "plan is NULL");
  if (plan->problem_key != problem_key(p))
    return fail(ATTN_ERR_ARG, "plan was made for a different problem");
  if (plan->s_max < 1 || plan->chunk < 1) return fail(ATTN_ERR_ARG, "corrupt plan");
  if (p->batch == 0) return ATTN_OK;
  if (int st = check_ptrs(q, "q", k, "k", v, "v")) return st;
  if (!o) return fail(ATTN_ERR_ARG, "o is NULL");
  if (!ws_o || !ws_lse || !ws_cnt) return fail(ATTN_ERR_ARG, "workspace pointer is NULL");
  if (ws_o_bytes < plan->ws_o_bytes || ws_lse_bytes < plan->ws_lse_bytes ||
      ws_cnt_bytes < plan->ws_cnt_bytes)
    return fail(ATTN_ERR_WORKSPACE, "workspace too small: need %llu + %llu + %llu bytes",
                (unsigned long long)plan->ws_o_bytes, (unsigned long long)plan->ws_lse_bytes,
                (unsigned long long)plan->ws_cnt_bytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (plan->kernel == ATTN_KERNEL_GQA_D128 && plan->s_max == 1 &&
      gqa_d128_usable(p, plan, q, k, v)) {
    // One split per request: one workgroup per (request, KV head) writes O.
    KParams kp = base_params(p);
    kp.q = q; kp.k = k; kp.v = v; kp.o = o;
    kp.lse_out = lse_out;
    kp.chunk = plan->chunk;
    kp.s_max = 1;
    kp.n_items = plan->n_items;
    kp.split_mode = 0;
    return hip_status(launch_decode_gqa_d128(kp, s), "decode_gqa_d128 launch");
  }
  if (plan->kernel == ATTN_KERNEL_GQA_D128 && gqa_d128_fits(p, q, k, v) &&
      plan->ws_o_bytes < (1ull << 31)) {
    // One launch: equal runs of key rounds per workgroup (paged segments are
    // staged in LDS piece by piece, so no page-count bound applies).
    KParams kp = base_params(p);
    kp.q = q; kp.k = k; kp.v = v; kp.o = o;
    kp.ws_o = ws_o; kp.ws_lse = ws_lse; kp.lse_out = lse_out;
    kp.counters = ws_cnt;
    kp.chunk = plan->chunk;
    kp.s_max = plan->s_max;
    kp.n_items = plan->stream_rounds;
    kp.stream_grid = plan->stream_grid;
    kp.split_mode = 3;
    return hip_status(launch_decode_gqa_d128(kp, s), "decode_gqa_d128 launch");
  }
  // MLA: one launch whose last split per (request, KV head) merges, when the
  // partials' byte offsets fit the kernel's 31-bit buffer offsets.
  const uint64_t nrows = (uint64_t)p->batch * p->q_len * p->q_heads;
  if (plan->kernel == ATTN_KERNEL_MLA && mla_usable(p, plan, q, k, v) &&
      plan->ws_o_bytes < (1ull << 31)) {
    KParams kp = base_params(p);
    kp.q = q; kp.k = k; kp.v = v; kp.o = o;
    kp.ws_o = ws_o; kp.ws_lse = ws_lse; kp.lse_out = lse_out;
    kp.counters = ws_cnt;
    kp.chunk = plan->chunk;
    kp.s_max = plan->s_max;
    kp.split_mode = 2;
    return hip_status(launch_decode_mla(kp, dim3(plan->s_max, p->kv_heads, p->batch), s),
                      "decode_mla launch");
  }
  if (plan->kernel == ATTN_KERNEL_GENERIC) {
    // One launch: the last split of each (request, KV head, row tile) merges.
    const int row_tiles = (int)ceil_div(p->q_heads / p->kv_heads * p->q_len, kGenericRowTile);
    KParams kp = base_params(p);
    kp.q = q; kp.k = k; kp.v = v; kp.o = o;
    kp.ws_o = ws_o; kp.ws_lse = ws_lse; kp.lse_out = lse_out;
    kp.counters = ws_cnt;
    kp.chunk = plan->chunk;
    kp.s_max = plan->s_max;
    kp.split_mode = 2;
    const dim3 grid(plan->s_max, row_tiles, (unsigned)((int64_t)p->batch * p->kv_heads));
    return hip_status(launch_generic(kp, grid, dim3(kGenericBlock), s), "generic decode launch");
  }
  // Otherwise (an MLA problem the single-launch kernel does not take): the
  // split launch, then the combine launch.
  if (int st = attn_decode_split(problem, plan, q, k, v, ws_o, ws_o_bytes, ws_lse, ws_lse_bytes,
                                 stream))
    return st;
  return attn_combine(problem, plan, ws_o, ws_lse, o, lse_out, stream);
}

int attn_combine(const attn_problem* problem, const attn_plan* plan, const float* ws_o,
                 const float* ws_lse, void* o, float* lse_out, void* stream) {
  g_err[0] = 0;
  if (int st = check_problem(problem)) return st;
  if (int st = check_decode_layout(problem)) return st;
  const attn_problem* p = problem;
  if (!plan) return fail(ATTN_ERR_ARG, "plan is NULL");
  if (plan->problem_key != problem_key(p))
    return fail(ATTN_ERR_ARG, "plan was made for a different problem");
  if (plan->s_max < 1 || plan->chunk < 1) return fail(ATTN_ERR_ARG, "corrupt plan");
  if (p->batch == 0) return ATTN_OK;
  if (!ws_o || !ws_lse) return fail(ATTN_ERR_ARG, "workspace pointer is NULL");
  if (!o) return fail(ATTN_ERR_ARG, "o is NULL");
  KParams kp = base_params(p);
  kp.ws_o = const_cast<float*>(ws_o);
  kp.ws_lse = const_cast<float*>(ws_lse);
  kp.o = o;
  kp.lse_out = lse_out;
  kp.chunk = plan->chunk;
  kp.s_max = plan->s_max;
  return hip_status(launch_combine(kp, reinterpret_cast<hipStream_t>(stream)), "combine launch");
}

int attn_prefill(const attn_problem* problem, const void* q, const void* k, const void* v, void* o,
                 float* lse_out, void* stream) {
  g_err[0] = 0;
  if (int st = check_problem(problem)) return st;
  const attn_problem* p = problem;
  if (p->batch == 0) return ATTN_OK;
  if (int st = check_ptrs(q, "q", k, "k", v, "v")) return st;
  if (!o) return fail(ATTN_ERR_ARG, "o is NULL");
  KParams kp = base_params(p);
  kp.q = q; kp.k = k; kp.v = v; kp.o = o;
  kp.lse_out = lse_out;
  kp.chunk = p->kv_len_max;
  kp.s_max = 1;
  kp.split_mode = 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (prefill_d128_fits(p, q, k, v, o))
    return hip_status(launch_prefill_d128(kp, s), "prefill_d128 launch");
  const int row_tiles = (int)ceil_div(kp.rows, kGenericRowTile);
  if (row_tiles > 65535) return fail(ATTN_ERR_UNSUPPORTED, "too many query rows per KV head");
  const dim3 grid(1, row_tiles, (unsigned)((int64_t)p->batch * p->kv_heads));
  return hip_status(launch_generic(kp, grid, dim3(kGenericBlock), s), "generic prefill launch");
}

int attn_matmul_matmul(const attn_problem* problem, const void* q, const void* k, const void* v,
                       void* o, void* stream) {
  g_err[0] = 0;
  if (int st = check_problem(problem)) return st;
  const attn_problem* p = problem;
  if (p->batch == 0) return ATTN_OK;
  if (int st = check_ptrs(q, "q", k, "k", v, "v")) return st;
  if (!o) return fail(ATTN_ERR_ARG, "o is NULL");
  if (!prefill_d128_fits(p, q, k, v, o))
    return fail(ATTN_ERR_UNSUPPORTED,
                "MatMul+MatMul needs bf16 Q/K/V with head_dim 128 and the MFMA prefill layouts");
  KParams kp = base_params(p);
  kp.q = q; kp.k = k; kp.v = v; kp.o = o;
  kp.chunk = p->kv_len_max;
  kp.s_max = 1;
  kp.split_mode = 0;
  kp.no_softmax = 1;
  kp.scale_log2 = scale_of(p);  // the kernel multiplies the fp32 scores by tau itself
  return hip_status(launch_prefill_d128(kp, reinterpret_cast<hipStream_t>(stream)),
                    "matmul_matmul launch");
}

}  // extern "C"

// ------------------------------------------------------ RMSNorm + MatMul

namespace attn {
namespace {

constexpr int kRmsTileN = 64;   // most weight rows per split-kernel workgroup
constexpr int kRmsTileM = 32;   // tokens per split-kernel workgroup
constexpr int kRmsBlock = 256;

// Output columns per workgroup (tile_n) and K parts (s) of the decode-setting
// streaming kernels.  For each tile width from 64 down to 16 columns in steps
// of 4: the most parts (at least min_steps k-steps each) whose workgroups fit
// on the compute units at once, or the requested s.  The pair that leaves the
// fewest compute units idle in the last round of workgroups wins, the wider
// tile on a tie (a narrower tile reads the same bytes; its rows past the tile
// read as zero without a memory access).
constexpr int kStreamTileMax = 64;  // the streaming kernels' four 16-row MFMA blocks
void plan_stream_split(int64_t n, int64_t tiles_m, int64_t steps, int64_t min_steps, int cus,
                       int32_t s_request, int32_t* tile_out, int64_t* s_out) {
  double best = -1.0;
  *tile_out = kStreamTileMax;
  *s_out = 1;
  for (int tile = kStreamTileMax; tile >= 16; tile -= 4) {
    const int64_t tiles = ceil_div(n, tile) * tiles_m;
    int64_t s = 1;
    if (s_request > 0)
      s = std::min<int64_t>(s_request, steps);
    else if (tiles > 0)
      s = std::max<int64_t>(1, std::min<int64_t>((int64_t)cus / tiles, steps / min_steps));
    const int64_t chunk_steps = ceil_div(steps, s);
    s = ceil_div(steps, chunk_steps);
    const int64_t wgs = tiles * s;
    const double fill = wgs > 0 ? (double)wgs / (double)(ceil_div(wgs, cus) * cus) : 0.0;
    if (fill > best + 1e-9) {
      best = fill;
      *tile_out = tile;
      *s_out = s;
    }
  }
}

int check_rms(const rmsnorm_matmul_problem* p) {
  if (!p) return fail(ATTN_ERR_ARG, "problem is NULL");
  if ((p->dtype != ATTN_F32 && p->dtype != ATTN_BF16) ||
      (p->y_dtype != ATTN_F32 && p->y_dtype != ATTN_BF16))
    return fail(ATTN_ERR_ARG, "dtype/y_dtype must be ATTN_F32 or ATTN_BF16");
  if (p->m < 0 || p->n < 0) return fail(ATTN_ERR_ARG, "m and n must be >= 0");
  if (p->k < 1) return fail(ATTN_ERR_ARG, "k must be >= 1");
  if (!std::isfinite(p->eps) || p->eps < 0.f) return fail(ATTN_ERR_ARG, "eps must be finite and >= 0");
  if (p->x_stride < p->k || p->w_stride < p->k || p->y_stride < p->n)
    return fail(ATTN_ERR_ARG, "row strides must cover the rows");
  if (p->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "only bf16 X, g and W are supported");
  if (p->k % 8 != 0) return fail(ATTN_ERR_UNSUPPORTED, "k must be a multiple of 8");
  if ((p->x_stride | p->w_stride) & 7)
    return fail(ATTN_ERR_UNSUPPORTED, "row strides of X and W must be multiples of 8 elements");
  // 32-bit buffer offsets: a workgroup's 64 weight rows and 32 tokens.
  if ((int64_t)kRmsTileN * p->w_stride * 2 >= (1ll << 31) ||
      (int64_t)kRmsTileM * p->x_stride * 2 >= (1ll << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "row strides too large");
  return ATTN_OK;
}

// The prefill setting (Cleave §7.3: at least 256 tokens) on the tiled GEMM:
// whole 64-column k-steps and row strides one buffer resource spans.
bool rms_gemm_fits(const rmsnorm_matmul_problem* p) {
  return p->m >= kGemmMinTokens && p->k % kGemmKStep == 0 && p->w_stride <= kGemmMaxStride &&
         2 * (int64_t)p->k <= kGemmMaxStride;
}

uint64_t rms_key(const rmsnorm_matmul_problem* p) {
  const int32_t f[] = {0x524d53, p->dtype, p->m, p->k, p->n};
  uint64_t h = 1469598103934665603ull;
  for (int32_t x : f)
    for (int s = 0; s < 32; s += 8) {
      h ^= (uint64_t)((x >> s) & 0xff);
      h *= 1099511628211ull;
    }
  return h | 1ull;
}

}  // namespace
}  // namespace attn

extern "C" {

int rmsnorm_matmul_plan(const rmsnorm_matmul_problem* problem, int32_t s_request, int32_t num_cus,
                        rmsnorm_matmul_config* out) {
  g_err[0] = 0;
  if (!out) return fail(ATTN_ERR_ARG, "plan output is NULL");
  std::memset(out, 0, sizeof(*out));
  if (int st = check_rms(problem)) return st;
  const rmsnorm_matmul_problem* p = problem;
  int cus = num_cus;
  if (cus <= 0 && device_cu_count(&cus) != 0)
    return fail(ATTN_ERR_HIP, "cannot query the compute-unit count of the current device");
  const int64_t steps = ceil_div(p->k, 32);   // 32-column k-steps
  if (rms_gemm_fits(p)) {
    // Prefill setting: the tiled GEMM (256 x 256 output tiles), after a pass
    // that forms X * g (exact, as bf16 pairs) and the row scales in the
    // workspace.
    out->s = 1;
    out->k_chunk = p->k;
    out->grid[0] = (uint32_t)(ceil_div(p->m, 256) * ceil_div(p->n, 256));
    out->grid[1] = out->grid[2] = 1;
    out->block = 512;
    out->kernel = 1;
    out->ws_bytes = (((uint64_t)p->m * p->k * 4 + 255) & ~uint64_t(255)) + (uint64_t)p->m * 4;
    out->problem_key = rms_key(p);
    return ATTN_OK;
  }
  // Parts of at least four k-steps per wave (a part is split over the four
  // waves of a workgroup).
  int32_t tile_n = kRmsTileN;
  int64_t s = 1;
  plan_stream_split(p->n, ceil_div(p->m, kRmsTileM), steps, 16, cus, s_request, &tile_n, &s);
  const int64_t chunk_steps = ceil_div(steps, s);
  s = ceil_div(steps, chunk_steps);
  if (s > 65535 || ceil_div(p->m, kRmsTileM) > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "too many parts or token tiles for the grid");
  out->s = (int32_t)s;
  out->k_chunk = (int32_t)(chunk_steps * 32);
  out->tile_n = tile_n;
  out->grid[0] = (uint32_t)ceil_div(p->n, tile_n);
  out->grid[1] = (uint32_t)s;
  out->grid[2] = (uint32_t)ceil_div(p->m, kRmsTileM);
  out->block = kRmsBlock;
  out->ws_bytes = s > 1 ? (uint64_t)s * p->m * ((uint64_t)p->n + 1) * sizeof(float) : 0;
  out->problem_key = rms_key(p);
  return ATTN_OK;
}

int rmsnorm_matmul(const rmsnorm_matmul_problem* problem, const rmsnorm_matmul_config* plan,
                   const void* x, const void* g, const void* w, void* y, float* ws,
                   size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (int st = check_rms(problem)) return st;
  const rmsnorm_matmul_problem* p = problem;
  if (!plan) return fail(ATTN_ERR_ARG, "plan is NULL");
  if (plan->problem_key != rms_key(p)) return fail(ATTN_ERR_ARG, "plan was made for a different problem");
  if (plan->s < 1 || plan->k_chunk < 32 || plan->k_chunk % 32 ||
      (int64_t)plan->s * plan->k_chunk < p->k || (int64_t)(plan->s - 1) * plan->k_chunk >= p->k)
    return fail(ATTN_ERR_ARG, "corrupt plan");
  if (p->m == 0 || p->n == 0) return ATTN_OK;
  if (!x || !g || !w || !y) return fail(ATTN_ERR_ARG, "x, g, w and y must not be NULL");
  if (!aligned16(x) || !aligned16(g) || !aligned16(w))
    return fail(ATTN_ERR_UNSUPPORTED, "x, g and w must be 16-byte aligned");
  if (plan->kernel == 1) {
    if (p->m < kGemmMinTokens || p->k % kGemmKStep != 0) return fail(ATTN_ERR_ARG, "corrupt plan");
    if (!rms_gemm_fits(p)) return fail(ATTN_ERR_UNSUPPORTED, "row stride beyond %lld elements",
                                       (long long)kGemmMaxStride);
    const uint64_t xg_bytes = ((uint64_t)p->m * p->k * 4 + 255) & ~uint64_t(255);
    const uint64_t need = xg_bytes + (uint64_t)p->m * 4;
    if (!ws || ws_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace too small: need %llu bytes",
                  (unsigned long long)need);
    if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(ATTN_ERR_ARG, "workspace must be 16-byte aligned");
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    RmsPrepParams rp;
    std::memset(&rp, 0, sizeof(rp));
    rp.x = x; rp.g = g;
    rp.xg = ws;
    rp.row_scale = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + xg_bytes);
    rp.x_row = p->x_stride; rp.xg_row = 2 * (int64_t)p->k;
    rp.M = p->m; rp.K = p->k; rp.eps = p->eps;
    if (int st = hip_status(launch_rms_prep(rp, hs), "rms_prep launch")) return st;
    GemmParams gp;
    std::memset(&gp, 0, sizeof(gp));
    gp.a = ws; gp.b0 = w; gp.y = y; gp.row_scale = rp.row_scale;
    gp.a_row = 2 * (int64_t)p->k; gp.b0_row = p->w_stride; gp.y_row = p->y_stride;
    gp.M = p->m; gp.N = p->n; gp.K = 2 * p->k;
    gp.y_bf16 = p->y_dtype == ATTN_BF16;
    gp.mode = 0;
    gp.b_shift = 1;
    return hip_status(launch_gemm_nt(gp, hs), "gemm launch");
  }
  if (plan->tile_n < 4 || plan->tile_n > kStreamTileMax || plan->tile_n % 4)
    return fail(ATTN_ERR_ARG, "corrupt plan");
  const uint64_t need = plan->s > 1 ? (uint64_t)plan->s * p->m * ((uint64_t)p->n + 1) * sizeof(float) : 0;
  if (need && (!ws || ws_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "workspace too small: need %llu bytes", (unsigned long long)need);
  if (need && (reinterpret_cast<uintptr_t>(ws) & 15))
    return fail(ATTN_ERR_ARG, "workspace must be 16-byte aligned");
  RmsParams k;
  std::memset(&k, 0, sizeof(k));
  k.x = x; k.g = g; k.w = w; k.y = y;
  k.ws_u = plan->s > 1 ? ws : nullptr;
  k.ws_ssq = plan->s > 1 ? ws + (int64_t)plan->s * p->m * p->n : nullptr;
  k.x_row = p->x_stride; k.w_row = p->w_stride; k.y_row = p->y_stride;
  k.M = p->m; k.K = p->k; k.N = p->n;
  k.s = plan->s;
  k.k_chunk = plan->k_chunk;
  k.tile_n = plan->tile_n;
  k.y_bf16 = p->y_dtype == ATTN_BF16;
  k.eps = p->eps;
  return hip_status(launch_rmsnorm_matmul(k, reinterpret_cast<hipStream_t>(stream)),
                    "rmsnorm_matmul launch");
}

}  // extern "C"

// ----------------------------------------------------------------- SwiGLU

namespace attn {
namespace {

constexpr int kSwTileN = 64;   // output columns per split-kernel workgroup
constexpr int kSwTileM = 32;   // tokens per split-kernel workgroup

int check_swiglu(const swiglu_problem* p) {
  if (!p) return fail(ATTN_ERR_ARG, "problem is NULL");
  if (p->reserved0 != 0) return fail(ATTN_ERR_ARG, "reserved0 must be 0");
  if ((p->dtype != ATTN_F32 && p->dtype != ATTN_BF16) ||
      (p->y_dtype != ATTN_F32 && p->y_dtype != ATTN_BF16))
    return fail(ATTN_ERR_ARG, "dtype/y_dtype must be ATTN_F32 or ATTN_BF16");
  if (p->m < 0 || p->n < 0) return fail(ATTN_ERR_ARG, "m and n must be >= 0");
  if (p->k < 1) return fail(ATTN_ERR_ARG, "k must be >= 1");
  if (p->x_stride < p->k || p->wg_stride < p->k || p->wu_stride < p->k || p->y_stride < p->n)
    return fail(ATTN_ERR_ARG, "row strides must cover the rows");
  if (p->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "only bf16 X and weights are supported");
  if (p->k % 8 != 0) return fail(ATTN_ERR_UNSUPPORTED, "k must be a multiple of 8");
  if ((p->x_stride | p->wg_stride | p->wu_stride) & 7)
    return fail(ATTN_ERR_UNSUPPORTED, "row strides of X and the weights must be multiples of 8 elements");
  if ((int64_t)kSwTileN * std::max(p->wg_stride, p->wu_stride) * 2 >= (1ll << 31) ||
      (int64_t)kSwTileM * p->x_stride * 2 >= (1ll << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "row strides too large");
  return ATTN_OK;
}

bool swiglu_gemm_fits(const swiglu_problem* p) {
  return p->m >= kGemmMinTokens && p->k % kGemmKStep == 0 && p->x_stride <= kGemmMaxStride &&
         p->wg_stride <= kGemmMaxStride && p->wu_stride <= kGemmMaxStride;
}

uint64_t swiglu_key(const swiglu_problem* p) {
  const int32_t f[] = {0x535747, p->dtype, p->m, p->k, p->n};
  uint64_t h = 1469598103934665603ull;
  for (int32_t x : f)
    for (int s = 0; s < 32; s += 8) {
      h ^= (uint64_t)((x >> s) & 0xff);
      h *= 1099511628211ull;
    }
  return h | 1ull;
}

}  // namespace
}  // namespace attn

extern "C" {

int swiglu_plan(const swiglu_problem* problem, int32_t s_request, int32_t num_cus,
                swiglu_config* out) {
  g_err[0] = 0;
  if (!out) return fail(ATTN_ERR_ARG, "config output is NULL");
  std::memset(out, 0, sizeof(*out));
  if (int st = check_swiglu(problem)) return st;
  const swiglu_problem* p = problem;
  int cus = num_cus;
  if (cus <= 0 && device_cu_count(&cus) != 0)
    return fail(ATTN_ERR_HIP, "cannot query the compute-unit count of the current device");
  const int64_t steps = ceil_div(p->k, 32);
  if (swiglu_gemm_fits(p)) {
    // Prefill setting: the tiled GEMM of both MatMuls (256-token x 128-column
    // output tiles, gate and up side by side).
    out->s = 1;
    out->k_chunk = p->k;
    out->grid[0] = (uint32_t)(ceil_div(p->m, 256) * ceil_div(p->n, 128));
    out->grid[1] = out->grid[2] = 1;
    out->block = 512;
    out->kernel = 1;
    out->ws_bytes = 0;
    out->problem_key = swiglu_key(p);
    return ATTN_OK;
  }
  // Parts of at least four k-steps per wave (a part is split over each pair
  // of waves).
  int32_t tile_n = kSwTileN;
  int64_t s = 1;
  plan_stream_split(p->n, ceil_div(p->m, kSwTileM), steps, 8, cus, s_request, &tile_n, &s);
  const int64_t chunk_steps = ceil_div(steps, s);
  s = ceil_div(steps, chunk_steps);
  if (s > 65535 || ceil_div(p->m, kSwTileM) > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "too many parts or token tiles for the grid");
  out->s = (int32_t)s;
  out->k_chunk = (int32_t)(chunk_steps * 32);
  out->tile_n = tile_n;
  out->grid[0] = (uint32_t)ceil_div(p->n, tile_n);
  out->grid[1] = (uint32_t)s;
  out->grid[2] = (uint32_t)ceil_div(p->m, kSwTileM);
  out->block = 256;
  out->ws_bytes = s > 1 ? 2ull * (uint64_t)s * p->m * p->n * sizeof(float) : 0;
  out->problem_key = swiglu_key(p);
  return ATTN_OK;
}

int swiglu(const swiglu_problem* problem, const swiglu_config* config, const void* x,
           const void* w_gate, const void* w_up, void* y, float* ws, size_t ws_bytes,
           void* stream) {
  g_err[0] = 0;
  if (int st = check_swiglu(problem)) return st;
  const swiglu_problem* p = problem;
  if (!config) return fail(ATTN_ERR_ARG, "config is NULL");
  if (config->problem_key != swiglu_key(p)) return fail(ATTN_ERR_ARG, "config was made for a different problem");
  if (config->s < 1 || config->k_chunk < 32 || config->k_chunk % 32 ||
      (int64_t)config->s * config->k_chunk < p->k || (int64_t)(config->s - 1) * config->k_chunk >= p->k)
    return fail(ATTN_ERR_ARG, "corrupt config");
  if (p->m == 0 || p->n == 0) return ATTN_OK;
  if (!x || !w_gate || !w_up || !y) return fail(ATTN_ERR_ARG, "x, w_gate, w_up and y must not be NULL");
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up))
    return fail(ATTN_ERR_UNSUPPORTED, "x, w_gate and w_up must be 16-byte aligned");
  if (config->kernel == 1) {
    if (p->m < kGemmMinTokens || p->k % kGemmKStep != 0) return fail(ATTN_ERR_ARG, "corrupt config");
    if (!swiglu_gemm_fits(p)) return fail(ATTN_ERR_UNSUPPORTED, "row stride beyond %lld elements",
                                          (long long)kGemmMaxStride);
    GemmParams gp;
    std::memset(&gp, 0, sizeof(gp));
    gp.a = x; gp.b0 = w_gate; gp.b1 = w_up; gp.y = y;
    gp.a_row = p->x_stride; gp.b0_row = p->wg_stride; gp.b1_row = p->wu_stride;
    gp.y_row = p->y_stride;
    gp.M = p->m; gp.N = p->n; gp.K = p->k;
    gp.y_bf16 = p->y_dtype == ATTN_BF16;
    gp.mode = 1;
    return hip_status(launch_gemm_nt(gp, reinterpret_cast<hipStream_t>(stream)), "gemm launch");
  }
  if (config->tile_n < 4 || config->tile_n > kStreamTileMax || config->tile_n % 4)
    return fail(ATTN_ERR_ARG, "corrupt config");
  const uint64_t need = config->s > 1 ? 2ull * (uint64_t)config->s * p->m * p->n * sizeof(float) : 0;
  if (need && (!ws || ws_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "workspace too small: need %llu bytes", (unsigned long long)need);
  if (need && (reinterpret_cast<uintptr_t>(ws) & 15))
    return fail(ATTN_ERR_ARG, "workspace must be 16-byte aligned");
  SwigluParams k;
  std::memset(&k, 0, sizeof(k));
  k.x = x; k.wg = w_gate; k.wu = w_up; k.y = y;
  if (config->s > 1) {
    k.ws_g = ws;
    k.ws_u = ws + (int64_t)config->s * p->m * p->n;
  }
  k.x_row = p->x_stride; k.wg_row = p->wg_stride; k.wu_row = p->wu_stride; k.y_row = p->y_stride;
  k.M = p->m; k.K = p->k; k.N = p->n;
  k.s = config->s;
  k.k_chunk = config->k_chunk;
  k.tile_n = config->tile_n;
  k.y_bf16 = p->y_dtype == ATTN_BF16;
  return hip_status(launch_swiglu(k, reinterpret_cast<hipStream_t>(stream)), "swiglu launch");
}

}  // extern "C"

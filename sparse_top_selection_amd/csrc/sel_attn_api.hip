// Host side of libselattn.so: argument checks, the gfx950 device check, kernel
// launches and per-thread error text. Every check that needs no data runs here,
// before anything is enqueued; checks that need the data run in the kernels and
// report through the caller's status word.
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
// section Summary (the union path runs for INT8 KV on one card family and any
// other case takes another path with a one-line reason) and section Extra Notes
// (other parts are refused by a device check). Here there is a single path: an
// unsupported case returns an error code and a reason instead.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "sel_attn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Shapes the kernels implement, and sizes whose offsets fit the kernels' index math.
int check_dims(const sel_attn_dims* d, const char* who) {
  if (!d) return fail(SEL_ATTN_EINVAL, "%s: dims is NULL", who);
  if (d->n_ctx < 1) return fail(SEL_ATTN_EINVAL, "%s: n_ctx must be >= 1 (got %d)", who, d->n_ctx);
  if (d->n_q < 0) return fail(SEL_ATTN_EINVAL, "%s: n_q must be >= 0 (got %d)", who, d->n_q);
  if (d->n_kv < 1) return fail(SEL_ATTN_EINVAL, "%s: n_kv must be >= 1 (got %d)", who, d->n_kv);
  if (d->sel_cap < 1) return fail(SEL_ATTN_EINVAL, "%s: sel_cap must be >= 1 (got %d)", who, d->sel_cap);
  if (d->n_pages < 1) return fail(SEL_ATTN_EINVAL, "%s: n_pages must be >= 1 (got %d)", who, d->n_pages);
  if (d->head_dim != SEL_ATTN_HEAD_DIM)
    return fail(SEL_ATTN_EUNSUPPORTED, "%s: head_dim %d not supported (only %d)", who, d->head_dim,
                SEL_ATTN_HEAD_DIM);
  if (d->page_size != SEL_ATTN_PAGE_SIZE)
    return fail(SEL_ATTN_EUNSUPPORTED, "%s: page_size %d not supported (only %d)", who, d->page_size,
                SEL_ATTN_PAGE_SIZE);
  if (d->q_per_kv != SEL_ATTN_Q_PER_KV)
    return fail(SEL_ATTN_EUNSUPPORTED, "%s: q_per_kv %d not supported (only %d)", who, d->q_per_kv,
                SEL_ATTN_Q_PER_KV);
  // union rows of 8*sel_cap int32 cells: the per-group length must fit an int32
  if ((int64_t)d->sel_cap * 8 > INT32_MAX)
    return fail(SEL_ATTN_EINVAL, "%s: sel_cap %d too large", who, d->sel_cap);
  // pool rows are addressed with 32-bit byte offsets: each pool stays under 4 GiB
  if ((int64_t)d->n_pages * d->n_kv * SEL_ATTN_PAGE_SIZE * SEL_ATTN_HEAD_DIM > (int64_t)UINT32_MAX)
    return fail(SEL_ATTN_EINVAL, "%s: pool of %d pages x %d KV heads exceeds 4 GiB", who,
                d->n_pages, d->n_kv);
  if ((int64_t)d->n_kv * SEL_ATTN_Q_PER_KV * ((int64_t)(d->n_q + 7) / 8) > INT32_MAX)
    return fail(SEL_ATTN_EINVAL, "%s: n_q x n_kv too large", who);
  return SEL_ATTN_OK;
}

// gfx950 only; the answer is cached per device ordinal.
int check_device(const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  static std::mutex mu;
  static int known[64];  // 0 = unknown, 1 = gfx950, 2 = other
  if (dev < 0 || dev >= 64) return fail(SEL_ATTN_EUNSUPPORTED, "%s: device ordinal %d", who, dev);
  {
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess)
        return fail(SEL_ATTN_ELAUNCH, "%s: hipGetDeviceProperties: %s", who, hipGetErrorString(e));
      known[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    if (known[dev] != 1)
      return fail(SEL_ATTN_EUNSUPPORTED, "%s: device %d is not gfx950", who, dev);
  }
  return SEL_ATTN_OK;
}

}  // namespace

extern "C" {

const char* sel_attn_last_error(void) { return g_err; }

int sel_attn_select_blocks(const sel_attn_dims* d, int32_t first_pos, const float* block_scores,
                           int32_t* sel, int32_t* sel_len, hipStream_t stream) {
  static const char* who = "sel_attn_select_blocks";
  int rc = check_dims(d, who);
  if (rc) return rc;
  if (d->sel_cap < SEL_ATTN_SEL_MAX)
    return fail(SEL_ATTN_EINVAL, "%s: sel_cap %d cannot hold a full selection (%d cells)", who,
                d->sel_cap, SEL_ATTN_SEL_MAX);
  if (d->n_ctx > SEL_ATTN_SELECT_MAX_CTX)
    return fail(SEL_ATTN_EUNSUPPORTED, "%s: n_ctx %d above %d", who, d->n_ctx,
                SEL_ATTN_SELECT_MAX_CTX);
  if (first_pos < 0 || (int64_t)first_pos + d->n_q > d->n_ctx)
    return fail(SEL_ATTN_EINVAL, "%s: positions [%d, %lld) outside [0, n_ctx=%d)", who, first_pos,
                (long long)first_pos + d->n_q, d->n_ctx);
  if (d->n_q == 0) {
    g_err[0] = 0;
    return SEL_ATTN_OK;
  }
  if (!block_scores || !sel || !sel_len) return fail(SEL_ATTN_EINVAL, "%s: NULL array pointer", who);
  if (!aligned(block_scores, 4) || !aligned(sel, 4) || !aligned(sel_len, 4))
    return fail(SEL_ATTN_EINVAL, "%s: arrays must be 4-byte aligned", who);
  rc = check_device(who);
  if (rc) return rc;
  selattn::SelectArgs a;
  a.scores = block_scores;
  a.sel = sel;
  a.sel_len = sel_len;
  a.n_q = d->n_q;
  a.first_pos = first_pos;
  a.n_blocks = (d->n_ctx + SEL_ATTN_PAGE_SIZE - 1) / SEL_ATTN_PAGE_SIZE;
  a.sel_cap = d->sel_cap;
  hipError_t e = selattn::launch_select_blocks(a, stream);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: launch: %s", who, hipGetErrorString(e));
  g_err[0] = 0;
  return SEL_ATTN_OK;
}

int sel_attn_build_union(const sel_attn_dims* d, const int32_t* sel, const int32_t* sel_len,
                         const int32_t* page_table, int32_t* union_cells, uint8_t* union_mask,
                         int32_t* union_rows, int32_t* union_len, uint32_t* status,
                         hipStream_t stream) {
  static const char* who = "sel_attn_build_union";
  int rc = check_dims(d, who);
  if (rc) return rc;
  if (!status) return fail(SEL_ATTN_EINVAL, "%s: status is NULL", who);
  if (d->n_q == 0) {
    g_err[0] = 0;
    return SEL_ATTN_OK;
  }
  if (!sel || !sel_len || !page_table || !union_cells || !union_mask || !union_rows || !union_len)
    return fail(SEL_ATTN_EINVAL, "%s: NULL array pointer", who);
  if (!aligned(sel, 4) || !aligned(sel_len, 4) || !aligned(page_table, 4) ||
      !aligned(union_cells, 4) || !aligned(union_rows, 4) || !aligned(union_len, 4) ||
      !aligned(status, 4))
    return fail(SEL_ATTN_EINVAL, "%s: int32 arrays must be 4-byte aligned", who);
  rc = check_device(who);
  if (rc) return rc;
  selattn::UnionArgs a;
  a.sel = sel;
  a.sel_len = sel_len;
  a.page_table = page_table;
  a.union_cells = union_cells;
  a.union_mask = union_mask;
  a.union_rows = union_rows;
  a.union_len = union_len;
  a.status = status;
  a.n_ctx = d->n_ctx;
  a.n_q = d->n_q;
  a.sel_cap = d->sel_cap;
  a.n_kv = d->n_kv;
  a.n_pages = d->n_pages;
  hipError_t e = selattn::launch_union_build(a, stream);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: launch: %s", who, hipGetErrorString(e));
  g_err[0] = 0;
  return SEL_ATTN_OK;
}

}  // extern "C"

namespace {

int64_t prefill_items(const sel_attn_dims* d) { return (int64_t)((d->n_q + 7) / 8) * d->n_kv; }

// the most cells a group's union can hold: 8 rows of sel_cap, within the context
int64_t prefill_max_cells(const sel_attn_dims* d) {
  return std::min<int64_t>(8LL * d->sel_cap, (int64_t)d->n_ctx);
}

// Checks shared by sel_attn_prefill and sel_attn_prefill_split, and the kernel
// arguments (one work-group per (group, KV head) and split).
int prefill_args(const sel_attn_dims* d, const char* who, const float* q, const int8_t* k_pool,
                 const int8_t* v_pool, const float* k_scale, const float* v_scale,
                 const int32_t* union_rows, const uint8_t* union_mask, const int32_t* union_len,
                 float softmax_scale, float* out, uint32_t* status, selattn::PrefillArgs& a,
                 void* workspace = nullptr, size_t workspace_bytes = 0,
                 bool split = false) {
  int rc = check_dims(d, who);
  if (rc) return rc;
  if (!status) return fail(SEL_ATTN_EINVAL, "%s: status is NULL", who);
  if (!isfinite(softmax_scale))
    return fail(SEL_ATTN_EINVAL, "%s: softmax_scale must be finite", who);
  if (d->n_q == 0) return 0;
  if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !union_rows || !union_mask ||
      !union_len || !out)
    return fail(SEL_ATTN_EINVAL, "%s: NULL array pointer", who);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(SEL_ATTN_EINVAL, "%s: q, out, k_pool and v_pool must be 16-byte aligned", who);
  if (!aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(union_rows, 4) ||
      !aligned(union_len, 4) || !aligned(status, 4))
    return fail(SEL_ATTN_EINVAL, "%s: scale and int32 arrays must be 4-byte aligned", who);
  const int64_t items = (int64_t)((d->n_q + 7) / 8) * d->n_kv;
  const int splits = split ? selattn::prefill_split_count(items, prefill_max_cells(d)) : 1;
  if (splits > 1) {
    const size_t need = (size_t)items * splits * sizeof(selattn::PrefillPartial);
    if (!workspace || workspace_bytes < need)
      return fail(SEL_ATTN_EINVAL, "%s: workspace of %zu bytes, %zu needed", who,
                  workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned(workspace, 16))
      return fail(SEL_ATTN_EINVAL, "%s: workspace must be 16-byte aligned", who);
  }
  rc = check_device(who);
  if (rc) return rc;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.union_rows = union_rows;
  a.union_mask = union_mask;
  a.union_len = union_len;
  a.out = out;
  a.status = status;
  a.score_scale = softmax_scale * 1.4426950408889634f;
  a.n_ctx = d->n_ctx;
  a.n_q = d->n_q;
  a.n_kv = d->n_kv;
  a.n_pages = d->n_pages;
  // a row r is read for KV heads 0..n_kv-1 at r + 64 h: inside the pools while
  // r < (n_pages n_kv - n_kv + 1) 64 (check_dims keeps the product in range)
  a.row_limit = (uint32_t)(((int64_t)d->n_pages * d->n_kv - d->n_kv + 1) * SEL_ATTN_PAGE_SIZE);
  a.sel_cap = d->sel_cap;
  a.n_groups = (d->n_q + 7) / 8;
  a.n_splits = splits;
  a.part = splits > 1 ? static_cast<selattn::PrefillPartial*>(workspace) : nullptr;
  a.per_xcd = (int32_t)((items * splits + 7) / 8);
  return 0;
}


}  // namespace

extern "C" {

int sel_attn_prefill(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                     const int8_t* v_pool, const float* k_scale, const float* v_scale,
                     const int32_t* union_rows, const uint8_t* union_mask,
                     const int32_t* union_len, float softmax_scale, float* out, uint32_t* status,
                     hipStream_t stream) {
  static const char* who = "sel_attn_prefill";
  selattn::PrefillArgs a;
  int rc = prefill_args(d, who, q, k_pool, v_pool, k_scale, v_scale, union_rows, union_mask,
                        union_len, softmax_scale, out, status, a);
  if (rc) return rc;
  if (d->n_q == 0) {
    g_err[0] = 0;
    return SEL_ATTN_OK;
  }
  hipError_t e = selattn::launch_prefill(a, stream);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: launch: %s", who, hipGetErrorString(e));
  g_err[0] = 0;
  return SEL_ATTN_OK;
}

size_t sel_attn_prefill_workspace_bytes(const sel_attn_dims* d) {
  if (!d || d->n_q <= 0 || d->n_kv <= 0) return 0;
  const int64_t items = prefill_items(d);
  const int splits = selattn::prefill_split_count(items, prefill_max_cells(d));
  return splits > 1 ? (size_t)items * splits * sizeof(selattn::PrefillPartial) : 0;
}

int sel_attn_prefill_split(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                           const int8_t* v_pool, const float* k_scale, const float* v_scale,
                           const int32_t* union_rows, const uint8_t* union_mask,
                           const int32_t* union_len, float softmax_scale, float* out,
                           uint32_t* status, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  static const char* who = "sel_attn_prefill_split";
  selattn::PrefillArgs a;
  int rc = prefill_args(d, who, q, k_pool, v_pool, k_scale, v_scale, union_rows, union_mask,
                        union_len, softmax_scale, out, status, a, workspace, workspace_bytes,
                        true);
  if (rc) return rc;
  if (d->n_q == 0) {
    g_err[0] = 0;
    return SEL_ATTN_OK;
  }
  hipError_t e = a.n_splits > 1 ? selattn::launch_prefill_split(a, stream)
                                 : selattn::launch_prefill(a, stream);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: launch: %s", who, hipGetErrorString(e));
  g_err[0] = 0;
  return SEL_ATTN_OK;
}

}  // extern "C"

namespace {

// Checks shared by the per-position calls, and their kernel arguments.
int positions_args(const sel_attn_dims* d, const char* who, const float* q, const int8_t* k_pool,
                   const int8_t* v_pool, const float* k_scale, const float* v_scale,
                   const int32_t* page_table, const int32_t* sel, const int32_t* sel_len,
                   float softmax_scale, float* out, uint32_t* status, selattn::PositionsArgs& a) {
  int rc = check_dims(d, who);
  if (rc) return rc;
  if (!status) return fail(SEL_ATTN_EINVAL, "%s: status is NULL", who);
  if (!isfinite(softmax_scale))
    return fail(SEL_ATTN_EINVAL, "%s: softmax_scale must be finite", who);
  if (d->sel_cap > SEL_ATTN_POSITIONS_MAX_CAP)
    return fail(SEL_ATTN_EUNSUPPORTED, "%s: sel_cap %d above %d", who, d->sel_cap,
                SEL_ATTN_POSITIONS_MAX_CAP);
  if (d->n_q == 0) return SEL_ATTN_OK;
  if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !page_table || !sel || !sel_len || !out)
    return fail(SEL_ATTN_EINVAL, "%s: NULL array pointer", who);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(SEL_ATTN_EINVAL, "%s: q, out, k_pool and v_pool must be 16-byte aligned", who);
  if (!aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(page_table, 4) ||
      !aligned(sel, 4) || !aligned(sel_len, 4) || !aligned(status, 4))
    return fail(SEL_ATTN_EINVAL, "%s: scale and int32 arrays must be 4-byte aligned", who);
  rc = check_device(who);
  if (rc) return rc;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.page_table = page_table;
  a.sel = sel;
  a.sel_len = sel_len;
  a.out = out;
  a.status = status;
  a.score_scale = softmax_scale * 1.4426950408889634f;
  a.n_ctx = d->n_ctx;
  a.n_q = d->n_q;
  a.n_kv = d->n_kv;
  a.n_pages = d->n_pages;
  a.sel_cap = d->sel_cap;
  a.per_xcd = (d->n_q + 7) / 8;
  a.n_splits = (d->sel_cap + selattn::kDecodeSplit - 1) / selattn::kDecodeSplit;
  return SEL_ATTN_OK;
}

}  // namespace

extern "C" {

int sel_attn_prefill_positions(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                               const int8_t* v_pool, const float* k_scale, const float* v_scale,
                               const int32_t* page_table, const int32_t* sel,
                               const int32_t* sel_len, float softmax_scale, float* out,
                               uint32_t* status, hipStream_t stream) {
  static const char* who = "sel_attn_prefill_positions";
  selattn::PositionsArgs a;
  const int rc = positions_args(d, who, q, k_pool, v_pool, k_scale, v_scale, page_table, sel,
                                sel_len, softmax_scale, out, status, a);
  if (rc) return rc;
  if (d->n_q == 0) {
    g_err[0] = 0;
    return SEL_ATTN_OK;
  }
  hipError_t e = selattn::launch_prefill_positions(a, stream);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: launch: %s", who, hipGetErrorString(e));
  g_err[0] = 0;
  return SEL_ATTN_OK;
}

size_t sel_attn_decode_workspace_bytes(const sel_attn_dims* d) {
  if (check_dims(d, "sel_attn_decode_workspace_bytes")) return 0;
  const size_t splits = (size_t)(d->sel_cap + selattn::kDecodeSplit - 1) / selattn::kDecodeSplit;
  return (size_t)d->n_q * (size_t)d->n_kv * splits * sizeof(selattn::DecodePartial);
}

int sel_attn_decode(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                    const int8_t* v_pool, const float* k_scale, const float* v_scale,
                    const int32_t* page_table, const int32_t* sel, const int32_t* sel_len,
                    float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                    uint32_t* status, hipStream_t stream) {
  static const char* who = "sel_attn_decode";
  // every check that needs no device comes before the device check
  int rc = check_dims(d, who);
  if (rc) return rc;
  if (d->n_q > 0) {
    const size_t need = sel_attn_decode_workspace_bytes(d);
    if (!workspace || workspace_bytes < need)
      return fail(SEL_ATTN_EINVAL, "%s: workspace of %zu bytes needed (got %zu%s)", who, need,
                  workspace_bytes, workspace ? "" : ", NULL");
    if (!aligned(workspace, 16))
      return fail(SEL_ATTN_EINVAL, "%s: workspace must be 16-byte aligned", who);
    if (d->n_q > SEL_ATTN_DECODE_MAX_Q)
      return fail(SEL_ATTN_EINVAL, "%s: n_q %d above %d (the call is meant for a few positions)",
                  who, d->n_q, SEL_ATTN_DECODE_MAX_Q);
  }
  selattn::PositionsArgs a;
  rc = positions_args(d, who, q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
                      softmax_scale, out, status, a);
  if (rc) return rc;
  if (d->n_q == 0) {
    g_err[0] = 0;
    return SEL_ATTN_OK;
  }
  hipError_t e = selattn::launch_decode(a, static_cast<selattn::DecodePartial*>(workspace), stream);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: launch: %s", who, hipGetErrorString(e));
  g_err[0] = 0;
  return SEL_ATTN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The decode call without a caller workspace. Its split records live in
// `scratch`, a file-scope device array that every GPU the library runs on
// holds until the process ends. In host code the name `scratch` is only a
// host-side stand-in for that array, so its device address is taken once per
// device with hipGetSymbolAddress (with that device current) and only that
// address is ever handed to a kernel.
__device__ __align__(256) unsigned char scratch[SEL_ATTN_DECODE_NOALLOC_MAX_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call that runs on it. Returns SEL_ATTN_OK or ELAUNCH.
int scratch_address(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SEL_ATTN_EUNSUPPORTED, "%s: device ordinal %d", who, dev);
  static std::mutex mu;
  static void* ptr[64];
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SEL_ATTN_ELAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", who, dev,
                  hipGetErrorString(e));
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return SEL_ATTN_OK;
}

}  // namespace

extern "C" {

int sel_attn_decode_noalloc(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                            const int8_t* v_pool, const float* k_scale, const float* v_scale,
                            const int32_t* page_table, const int32_t* sel, const int32_t* sel_len,
                            float softmax_scale, float* out, uint32_t* status,
                            hipStream_t stream) {
  static const char* who = "sel_attn_decode_noalloc";
  int rc = check_dims(d, who);
  if (rc) return rc;
  if (d->n_q > 0) {
    const size_t need = sel_attn_decode_workspace_bytes(d);
    if (need > (size_t)SEL_ATTN_DECODE_NOALLOC_MAX_BYTES)
      return fail(SEL_ATTN_EINVAL,
                  "%s: these dims need %zu bytes of split records, above the %d-byte static "
                  "scratch (n_q * n_kv * ceil(sel_cap / 64) must stay <= %d); use sel_attn_decode "
                  "with a workspace",
                  who, need, SEL_ATTN_DECODE_NOALLOC_MAX_BYTES,
                  (int)(SEL_ATTN_DECODE_NOALLOC_MAX_BYTES / sizeof(selattn::DecodePartial)));
    if (d->n_q > SEL_ATTN_DECODE_MAX_Q)
      return fail(SEL_ATTN_EINVAL, "%s: n_q %d above %d", who, d->n_q, SEL_ATTN_DECODE_MAX_Q);
  }
  selattn::PositionsArgs a;
  rc = positions_args(d, who, q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
                      softmax_scale, out, status, a);
  if (rc) return rc;
  if (d->n_q == 0) {
    g_err[0] = 0;
    return SEL_ATTN_OK;
  }
  void* ws = nullptr;
  rc = scratch_address(who, &ws);
  if (rc) return rc;
  // every record the merge reads is written by the split kernel of the same
  // call, so nothing in the scratch needs clearing between calls
  hipError_t e = selattn::launch_decode(a, static_cast<selattn::DecodePartial*>(ws), stream);
  if (e != hipSuccess) return fail(SEL_ATTN_ELAUNCH, "%s: launch: %s", who, hipGetErrorString(e));
  g_err[0] = 0;
  return SEL_ATTN_OK;
}

}  // extern "C"

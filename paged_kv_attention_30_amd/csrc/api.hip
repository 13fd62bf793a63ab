// C ABI of the library: host-side validation, planning and dispatch.
//
// Every entry point validates its host-visible arguments first (pointers,
// sizes, strides, alignment, workspace) and returns a status code without
// touching the HIP runtime when something is wrong, in the spirit of the
// declarative shape checks the pages describe for their store kernel
// ("Mini-SGLang complete analysis" §4.9.4: one symbolic size bound across
// several tensors, a failure reports where it happened).

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/msgl.h"
#include "internal.hpp"

namespace {

thread_local char g_last_error[512] = "";
// Set by the msgl_validate_* calls: the entry point returns MSGL_OK where it
// would make its first HIP call.
thread_local bool g_validate_only = false;

// Runs `call` (an entry point invocation) with launches suppressed.
template <typename F>
int validate_only(F call) {
  g_validate_only = true;
  const int st = call();
  g_validate_only = false;
  return st;
}

int fail(int status, const char* file, int line, const char* fmt, ...) {
  char msg[400];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof(msg), fmt, ap);
  va_end(ap);
  const char* base = strrchr(file, '/');
  snprintf(g_last_error, sizeof(g_last_error), "%s (%s:%d)", msg, base ? base + 1 : file, line);
  return status;
}

#define MSGL_FAIL(status, ...) fail((status), __FILE__, __LINE__, __VA_ARGS__)
#define MSGL_CHECK(cond, status, ...) \
  do {                                \
    if (!(cond)) return MSGL_FAIL((status), __VA_ARGS__); \
  } while (0)

constexpr int kHeadDim = 128;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool ratio_ok(int hq, int hkv) {
  if (hkv <= 0 || hq <= 0 || hq % hkv) return false;
  const int r = hq / hkv;
  return r == 1 || r == 2 || r == 4 || r == 8 || r == 16;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSGL_OK;
  return MSGL_FAIL(MSGL_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
}

#ifdef MSGL_DEBUG_CHECKS
// Debug-check build: waits for the checks queued on `s` and turns the first
// failure into MSGL_ERR_INDEX with its details (the call's own kernels are
// then not launched).
int debug_verdict(hipStream_t s, const char* where) {
  msgl::DebugFailure f;
  const hipError_t e = msgl::debug_collect(s, &f);
  if (e != hipSuccess)
    return MSGL_FAIL(MSGL_ERR_LAUNCH, "%s: index checks did not run: %s", where,
                     hipGetErrorString(e));
  if (f.bits == 0) return MSGL_OK;
  switch (f.first) {
    case msgl::kDebugOutLoc:
      return MSGL_FAIL(MSGL_ERR_INDEX, "%s: out_loc[%d] = %lld is outside [0, num_slots) "
                       "(failed checks 0x%x)", where, f.a, f.v, f.bits);
    case msgl::kDebugLength:
      return MSGL_FAIL(MSGL_ERR_INDEX, "%s: request %d: length %lld (extend_len %d) is negative, "
                       "past its declared maximum or past the page-table width (failed checks "
                       "0x%x)", where, f.a, f.v, f.b, f.bits);
    case msgl::kDebugQOffsets:
      return MSGL_FAIL(MSGL_ERR_INDEX, "%s: request %d: q_offsets[r] = %lld and q_offsets[r+1] - "
                       "q_offsets[r] = %d, not extend_len (failed checks 0x%x)", where, f.a, f.v,
                       f.b, f.bits);
    case msgl::kDebugRow:
      return MSGL_FAIL(MSGL_ERR_INDEX, "%s: request %d: req_rows entry %lld is negative (failed "
                       "checks 0x%x)", where, f.a, f.v, f.bits);
    case msgl::kDebugSlot:
      return MSGL_FAIL(MSGL_ERR_INDEX, "%s: request %d: the page-table entry read for key %d is "
                       "%lld and reaches outside the pool (failed checks 0x%x)", where, f.a, f.b,
                       f.v, f.bits);
    default:
      return MSGL_FAIL(MSGL_ERR_INDEX, "%s: request %d: out_loc = %lld is not the slot of its "
                       "newest key %d (failed checks 0x%x)", where, f.a, f.v, f.b, f.bits);
  }
}

int debug_gate_out_loc(const void* out_loc, bool i64, int64_t n, int64_t num_slots,
                       hipStream_t s, const char* where) {
  if (msgl::debug_stream_capturing(s)) return MSGL_OK;   // nothing may wait inside a capture
  const hipError_t e = msgl::debug_check_out_loc(out_loc, i64, n, num_slots, s);
  if (e != hipSuccess) return launch_status(e, where);
  return debug_verdict(s, where);
}

int debug_gate_requests(const msgl::DebugRequestCheck& c, const void* store_loc, bool i64,
                        hipStream_t s, const char* where) {
  if (msgl::debug_stream_capturing(s)) return MSGL_OK;
  hipError_t e = store_loc ? msgl::debug_check_out_loc(store_loc, i64, c.batch, c.num_slots, s)
                           : hipSuccess;
  if (e == hipSuccess) e = msgl::debug_check_requests(c, s);
  if (e != hipSuccess) return launch_status(e, where);
  return debug_verdict(s, where);
}

int32_t page_span(int32_t page_size) {
  return (page_size > 1 && (page_size & (page_size - 1)) == 0) ? page_size : 1;
}
#endif

// Compute units of the current device (cached per device).
int device_compute_units() {
  static int cu_cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cu_cache[dev];
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cu_cache[dev] = cus;
  }
  return cus;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout of one decode call: partial outputs, partial lse, and
// (balanced mode) the per-request workgroup ranges.
struct DecodeWorkspace {
  size_t part_out_bytes, part_lse_bytes, meta_bytes;
  size_t total() const { return part_out_bytes + part_lse_bytes + meta_bytes; }
};

// `grid_rows`: partial rows reserved for the balanced mode's workgroups
// (kMaxDecodeBlocks for a caller-sized workspace, which must not depend on
// the device; the launch's own grid for the library's static scratch).
DecodeWorkspace decode_workspace(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t split_tokens,
                                 int64_t grid_rows = msgl::kMaxDecodeBlocks) {
  DecodeWorkspace w{0, 0, 0};
  int64_t rows;
  if (split_tokens > 0) {
    const int64_t splits = ((int64_t)max_seq_len + split_tokens - 1) / split_tokens;
    if (splits <= 1) return w;
    rows = splits * batch;
  } else {
    rows = grid_rows + batch;
    w.meta_bytes = align256((size_t)batch * 2 * sizeof(int32_t));
  }
  w.part_out_bytes = align256((size_t)rows * num_q_heads * head_dim * sizeof(float));
  w.part_lse_bytes = align256((size_t)rows * num_q_heads * sizeof(float));
  return w;
}

int validate_pool(const void* k_cache, const void* v_cache, int64_t num_slots,
                  int64_t cache_row_stride, int32_t num_kv_heads, int32_t head_dim) {
  MSGL_CHECK(k_cache && v_cache, MSGL_ERR_NULL, "k_cache/v_cache is NULL");
  MSGL_CHECK(head_dim == kHeadDim, MSGL_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", head_dim);
  MSGL_CHECK(num_kv_heads > 0, MSGL_ERR_SHAPE, "num_kv_heads %d must be positive", num_kv_heads);
  MSGL_CHECK(num_slots > 0, MSGL_ERR_SHAPE, "num_slots %lld must be positive", (long long)num_slots);
  MSGL_CHECK(cache_row_stride >= (int64_t)num_kv_heads * head_dim, MSGL_ERR_SHAPE,
             "cache_row_stride %lld < num_kv_heads*head_dim %lld", (long long)cache_row_stride,
             (long long)num_kv_heads * head_dim);
  MSGL_CHECK(aligned(k_cache, 16) && aligned(v_cache, 16), MSGL_ERR_ALIGN,
             "k_cache/v_cache must be 16-byte aligned");
  MSGL_CHECK((cache_row_stride * 2) % 16 == 0, MSGL_ERR_ALIGN,
             "cache_row_stride*2 bytes must be a multiple of 16");
  return MSGL_OK;
}

}  // namespace

extern "C" {

int msgl_version(void) { return 100; }

int msgl_debug_checks(void) {
#ifdef MSGL_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

const char* msgl_status_string(int status) {
  switch (status) {
    case MSGL_OK: return "MSGL_OK";
    case MSGL_ERR_NULL: return "MSGL_ERR_NULL: a required pointer is NULL";
    case MSGL_ERR_SHAPE: return "MSGL_ERR_SHAPE: inconsistent or negative sizes/strides";
    case MSGL_ERR_UNSUPPORTED: return "MSGL_ERR_UNSUPPORTED: dtype, head_dim, ratio or page_size not served";
    case MSGL_ERR_ALIGN: return "MSGL_ERR_ALIGN: pointer or stride breaks required alignment";
    case MSGL_ERR_WORKSPACE: return "MSGL_ERR_WORKSPACE: workspace missing or too small";
    case MSGL_ERR_LAUNCH: return "MSGL_ERR_LAUNCH: the HIP runtime rejected a launch";
    case MSGL_ERR_INDEX: return "MSGL_ERR_INDEX: a device index or length is out of range (debug-check build)";
    default: return "unknown msgl status";
  }
}

const char* msgl_last_error(void) { return g_last_error; }

int msgl_store_kv(void* k_cache, void* v_cache, int64_t num_slots, int64_t cache_row_stride,
                  const void* k_new, const void* v_new, int64_t new_row_stride,
                  const void* out_loc, int32_t index_dtype, int64_t n, int32_t num_kv_heads,
                  int32_t head_dim, int32_t dtype, hipStream_t stream) {
  g_last_error[0] = 0;
  MSGL_CHECK(n >= 0, MSGL_ERR_SHAPE, "n %lld is negative", (long long)n);
  MSGL_CHECK(dtype == MSGL_DTYPE_BF16 || dtype == MSGL_DTYPE_F32, MSGL_ERR_UNSUPPORTED,
             "dtype %d unsupported", dtype);
  MSGL_CHECK(index_dtype == MSGL_INDEX_I32 || index_dtype == MSGL_INDEX_I64, MSGL_ERR_UNSUPPORTED,
             "index dtype %d unsupported", index_dtype);
  MSGL_CHECK(num_kv_heads > 0 && head_dim > 0, MSGL_ERR_SHAPE, "num_kv_heads/head_dim must be positive");
  MSGL_CHECK(num_slots > 0, MSGL_ERR_SHAPE, "num_slots must be positive");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  MSGL_CHECK(cache_row_stride >= row, MSGL_ERR_SHAPE, "cache_row_stride %lld < row %lld",
             (long long)cache_row_stride, (long long)row);
  MSGL_CHECK(new_row_stride >= row, MSGL_ERR_SHAPE, "new_row_stride %lld < row %lld",
             (long long)new_row_stride, (long long)row);
  if (n == 0) return MSGL_OK;
  MSGL_CHECK(k_cache && v_cache && k_new && v_new && out_loc, MSGL_ERR_NULL,
             "k_cache, v_cache, k_new, v_new and out_loc must be non-NULL");
  const int esz = dtype == MSGL_DTYPE_BF16 ? 2 : 4;
  MSGL_CHECK(aligned(k_cache, esz) && aligned(v_cache, esz) && aligned(k_new, esz) &&
                 aligned(v_new, esz),
             MSGL_ERR_ALIGN, "tensors must be aligned to their element size");
  MSGL_CHECK(aligned(out_loc, index_dtype == MSGL_INDEX_I64 ? 8 : 4), MSGL_ERR_ALIGN,
             "out_loc must be aligned to its element size");

  msgl::StoreArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_stride_bytes = cache_row_stride * esz;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_stride_bytes = new_row_stride * esz;
  a.out_loc = out_loc;
  a.index_is_i64 = index_dtype == MSGL_INDEX_I64;
  a.n = n;
  a.row_bytes = row * esz;
  a.stream = stream;
  int unit = 16;
  while (unit > esz) {
    const bool ok = aligned(k_cache, unit) && aligned(v_cache, unit) && aligned(k_new, unit) &&
                    aligned(v_new, unit) && a.cache_stride_bytes % unit == 0 &&
                    a.new_stride_bytes % unit == 0 && a.row_bytes % unit == 0;
    if (ok) break;
    unit /= 2;
  }
  a.unit_bytes = unit;
  if (g_validate_only) return MSGL_OK;
#ifdef MSGL_DEBUG_CHECKS
  if (int dst = debug_gate_out_loc(out_loc, a.index_is_i64, n, num_slots, stream, "store_kv"))
    return dst;
#endif
  return launch_status(msgl::launch_store_kv(a), "store_kv");
}

size_t msgl_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_seq_len,
                                        int32_t split_tokens, int32_t* split_tokens_out) {
  (void)num_kv_heads;
  if (split_tokens_out) *split_tokens_out = split_tokens > 0 ? split_tokens : 0;
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || split_tokens < 0)
    return 0;
  return decode_workspace(batch, num_q_heads, head_dim, max_seq_len, split_tokens).total();
}

namespace {

// The new rows a fused store+decode call writes (null: a plain decode).
struct FusedStore {
  const void* k_new;
  const void* v_new;
  int64_t new_row_stride;
  const void* out_loc;
  int32_t index_dtype;
};

int paged_decode_impl(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                      const void* k_cache, const void* v_cache, int64_t num_slots,
                      int64_t cache_row_stride, const int32_t* page_table,
                      int64_t page_table_stride, const int32_t* req_rows,
                      const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t max_seq_len, float sm_scale, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, const FusedStore* fs,
                      hipStream_t stream, const char* where,
                      int64_t grid_rows = msgl::kMaxDecodeBlocks) {
  g_last_error[0] = 0;
  MSGL_CHECK(batch >= 0, MSGL_ERR_SHAPE, "batch %d is negative", batch);
  int st = validate_pool(k_cache, v_cache, num_slots, cache_row_stride, num_kv_heads, head_dim);
  if (st) return st;
  MSGL_CHECK(ratio_ok(num_q_heads, num_kv_heads), MSGL_ERR_UNSUPPORTED,
             "num_q_heads %d / num_kv_heads %d: ratio must be 1, 2, 4, 8 or 16", num_q_heads,
             num_kv_heads);
  MSGL_CHECK(page_size >= 1, MSGL_ERR_UNSUPPORTED, "page_size %d must be >= 1", page_size);
  MSGL_CHECK(max_seq_len >= 0, MSGL_ERR_SHAPE, "max_seq_len %d is negative", max_seq_len);
  MSGL_CHECK(split_tokens >= 0 && split_tokens % 32 == 0, MSGL_ERR_SHAPE,
             "split_tokens %d must be 0 or a positive multiple of 32", split_tokens);
  MSGL_CHECK(q_row_stride >= (int64_t)num_q_heads * head_dim, MSGL_ERR_SHAPE,
             "q_row_stride %lld < num_q_heads*head_dim", (long long)q_row_stride);
  MSGL_CHECK(page_table_stride >= max_seq_len, MSGL_ERR_SHAPE,
             "page_table_stride %lld < max_seq_len %d", (long long)page_table_stride, max_seq_len);
  if (batch == 0) return MSGL_OK;
  MSGL_CHECK(out && q && page_table && seq_lens, MSGL_ERR_NULL,
             "out, q, page_table and seq_lens must be non-NULL");
  MSGL_CHECK(aligned(q, 16) && aligned(out, 16), MSGL_ERR_ALIGN, "q and out must be 16-byte aligned");
  MSGL_CHECK((q_row_stride * 2) % 16 == 0, MSGL_ERR_ALIGN, "q_row_stride*2 must be a multiple of 16");
  MSGL_CHECK(aligned(page_table, 4) && aligned(seq_lens, 4) && (!req_rows || aligned(req_rows, 4)) &&
                 (!lse_out || aligned(lse_out, 4)),
             MSGL_ERR_ALIGN, "int32/fp32 arrays must be 4-byte aligned");

  const DecodeWorkspace ws = decode_workspace(batch, num_q_heads, head_dim, max_seq_len,
                                              split_tokens, grid_rows);
  const size_t need = ws.total();
  MSGL_CHECK(workspace_bytes >= need, MSGL_ERR_WORKSPACE, "workspace %zu bytes < required %zu",
             workspace_bytes, need);
  MSGL_CHECK(need == 0 || (workspace && aligned(workspace, 256)), MSGL_ERR_WORKSPACE,
             "workspace must be non-NULL and 256-byte aligned");

  if (fs) {
    MSGL_CHECK(fs->index_dtype == MSGL_INDEX_I32 || fs->index_dtype == MSGL_INDEX_I64,
               MSGL_ERR_UNSUPPORTED, "index dtype %d unsupported", fs->index_dtype);
    MSGL_CHECK(fs->new_row_stride >= (int64_t)num_kv_heads * head_dim, MSGL_ERR_SHAPE,
               "new_row_stride %lld < num_kv_heads*head_dim", (long long)fs->new_row_stride);
    MSGL_CHECK(fs->k_new && fs->v_new && fs->out_loc, MSGL_ERR_NULL,
               "k_new, v_new and out_loc must be non-NULL");
    MSGL_CHECK(aligned(fs->k_new, 16) && aligned(fs->v_new, 16) && (fs->new_row_stride * 2) % 16 == 0,
               MSGL_ERR_ALIGN, "k_new / v_new rows must be 16-byte aligned");
    MSGL_CHECK(aligned(fs->out_loc, fs->index_dtype == MSGL_INDEX_I64 ? 8 : 4), MSGL_ERR_ALIGN,
               "out_loc must be aligned to its element size");
  }

  msgl::DecodeArgs a;
  a.k_store = fs ? const_cast<void*>(k_cache) : nullptr;
  a.v_store = fs ? const_cast<void*>(v_cache) : nullptr;
  a.k_new = fs ? fs->k_new : nullptr;
  a.v_new = fs ? fs->v_new : nullptr;
  a.new_stride = fs ? fs->new_row_stride : 0;
  a.out_loc = fs ? fs->out_loc : nullptr;
  a.out_loc_is_i64 = fs && fs->index_dtype == MSGL_INDEX_I64;
  a.out = out;
  a.lse = lse_out;
  a.q = q;
  a.q_stride = q_row_stride;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_slots = num_slots;
  a.cache_stride = cache_row_stride;
  a.page_table = page_table;
  a.pt_stride = page_table_stride;
  a.req_rows = req_rows;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.page_size = page_size;
  a.max_seq_len = max_seq_len;
  a.sm_scale = sm_scale;
  a.stream = stream;
  a.split_tokens = split_tokens;
  a.part_out = need ? (float*)workspace : nullptr;
  a.part_lse = need ? (float*)((char*)workspace + ws.part_out_bytes) : nullptr;
  a.meta = ws.meta_bytes ? (int32_t*)((char*)workspace + ws.part_out_bytes + ws.part_lse_bytes)
                         : nullptr;
  if (g_validate_only) return MSGL_OK;
#ifdef MSGL_DEBUG_CHECKS
  {
    msgl::DebugRequestCheck c;
    c.lens = seq_lens;
    c.req_rows = req_rows;
    c.pt = page_table;
    c.pt_stride = page_table_stride;
    c.batch = batch;
    c.max_total = max_seq_len;
    c.num_slots = num_slots;
    c.page_span = page_span(page_size);
    c.out_loc = fs ? fs->out_loc : nullptr;
    c.out_loc_i64 = a.out_loc_is_i64;
    if (int dst = debug_gate_requests(c, c.out_loc, a.out_loc_is_i64, stream, where)) return dst;
  }
#endif
  if (split_tokens > 0) {
    a.balanced_blocks = 0;
    a.max_splits = need ? (int32_t)(((int64_t)max_seq_len + split_tokens - 1) / split_tokens) : 1;
  } else {
    a.balanced_blocks = device_compute_units();
    a.max_splits = 0;
  }
  return launch_status(msgl::launch_paged_decode(a), where);
}

}  // namespace

int msgl_paged_decode(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                      const void* k_cache, const void* v_cache, int64_t num_slots,
                      int64_t cache_row_stride, const int32_t* page_table,
                      int64_t page_table_stride, const int32_t* req_rows,
                      const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t max_seq_len, float sm_scale, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return paged_decode_impl(out, lse_out, q, q_row_stride, k_cache, v_cache, num_slots,
                           cache_row_stride, page_table, page_table_stride, req_rows, seq_lens,
                           batch, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                           sm_scale, split_tokens, workspace, workspace_bytes, nullptr, stream,
                           "paged_decode");
}

int msgl_store_kv_paged_decode(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                               void* k_cache, void* v_cache, int64_t num_slots,
                               int64_t cache_row_stride, const void* k_new, const void* v_new,
                               int64_t new_row_stride, const void* out_loc, int32_t index_dtype,
                               const int32_t* page_table, int64_t page_table_stride,
                               const int32_t* req_rows, const int32_t* seq_lens, int32_t batch,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t max_seq_len, float sm_scale,
                               int32_t split_tokens, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const FusedStore fs{k_new, v_new, new_row_stride, out_loc, index_dtype};
  return paged_decode_impl(out, lse_out, q, q_row_stride, k_cache, v_cache, num_slots,
                           cache_row_stride, page_table, page_table_stride, req_rows, seq_lens,
                           batch, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                           sm_scale, split_tokens, workspace, workspace_bytes, &fs, stream,
                           "store_kv_paged_decode");
}

}  // extern "C"

// Device memory of msgl_store_kv_paged_decode_noalloc: the partial outputs,
// partial lse and per-request workgroup ranges that the caller-provided
// workspace holds for the other entry points.  Each GPU the library runs on
// holds one copy until the process ends; host code reaches it only through
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MSGL_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Address of `scratch` on the current device, looked up once per device.
int scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return MSGL_FAIL(MSGL_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  MSGL_CHECK(dev >= 0 && dev < kMaxDevices, MSGL_ERR_UNSUPPORTED, "device %d beyond %d", dev,
             kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return MSGL_FAIL(MSGL_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed: %s",
                       hipGetErrorString(e));
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MSGL_OK;
}

}  // namespace

extern "C" {

int msgl_store_kv_paged_decode_noalloc(void* out, float* lse_out, const void* q,
                                       int64_t q_row_stride, void* k_cache, void* v_cache,
                                       int64_t num_slots, int64_t cache_row_stride,
                                       const void* k_new, const void* v_new,
                                       int64_t new_row_stride, const void* out_loc,
                                       int32_t index_dtype, const int32_t* page_table,
                                       int64_t page_table_stride, const int32_t* req_rows,
                                       const int32_t* seq_lens, int32_t batch,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, int32_t max_seq_len,
                                       float sm_scale, int32_t split_tokens, hipStream_t stream) {
  g_last_error[0] = 0;
  // the split the launch will use sizes the partials: the balanced grid of
  // this device (one row per workgroup plus one per request) or the chunks
  MSGL_CHECK(batch >= 0 && num_q_heads > 0 && num_kv_heads > 0 && max_seq_len >= 0 &&
                 split_tokens >= 0 && head_dim == kHeadDim,
             MSGL_ERR_SHAPE, "batch, head counts, max_seq_len, split_tokens or head_dim invalid");
  MSGL_CHECK(ratio_ok(num_q_heads, num_kv_heads), MSGL_ERR_UNSUPPORTED,
             "num_q_heads %d / num_kv_heads %d: ratio must be 1, 2, 4, 8 or 16", num_q_heads,
             num_kv_heads);
  const int64_t grid = split_tokens > 0
                           ? 0
                           : msgl::decode_balanced_grid(num_kv_heads, num_q_heads / num_kv_heads,
                                                        device_compute_units());
  const size_t need =
      decode_workspace(batch, num_q_heads, head_dim, max_seq_len, split_tokens, grid).total();
  MSGL_CHECK(need <= (size_t)MSGL_DECODE_SCRATCH_BYTES, MSGL_ERR_WORKSPACE,
             "batch %d x %d q heads (max_seq_len %d, split_tokens %d) needs %zu bytes of "
             "partial results; the library's scratch holds %zu",
             batch, num_q_heads, max_seq_len, split_tokens, need,
             (size_t)MSGL_DECODE_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need) {
    const int st = scratch_on_device(&ws);
    if (st) return st;
  }
  const FusedStore fs{k_new, v_new, new_row_stride, out_loc, index_dtype};
  return paged_decode_impl(out, lse_out, q, q_row_stride, k_cache, v_cache, num_slots,
                           cache_row_stride, page_table, page_table_stride, req_rows, seq_lens,
                           batch, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                           sm_scale, split_tokens, ws, need, &fs, stream,
                           "store_kv_paged_decode_noalloc", grid);
}

size_t msgl_paged_extend_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_extend_len,
                                        int32_t max_kv_len) {
  (void)head_dim; (void)max_kv_len;
  if (batch <= 0 || max_extend_len <= 0 || !ratio_ok(num_q_heads, num_kv_heads)) return 0;
  return msgl::extend_workspace_bytes(batch, num_q_heads / num_kv_heads, max_extend_len);
}

int msgl_paged_extend(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                      const void* k_cache, const void* v_cache, int64_t num_slots,
                      int64_t cache_row_stride, const int32_t* page_table,
                      int64_t page_table_stride, const int32_t* req_rows,
                      const int32_t* prefix_lens, const int32_t* extend_lens,
                      const int32_t* q_offsets, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t max_extend_len, int32_t max_kv_len, float sm_scale,
                      int32_t causal, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  g_last_error[0] = 0;
  MSGL_CHECK(batch >= 0, MSGL_ERR_SHAPE, "batch %d is negative", batch);
  int st = validate_pool(k_cache, v_cache, num_slots, cache_row_stride, num_kv_heads, head_dim);
  if (st) return st;
  MSGL_CHECK(ratio_ok(num_q_heads, num_kv_heads), MSGL_ERR_UNSUPPORTED,
             "num_q_heads %d / num_kv_heads %d: ratio must be 1, 2, 4, 8 or 16", num_q_heads,
             num_kv_heads);
  MSGL_CHECK(causal == 1, MSGL_ERR_UNSUPPORTED, "only causal extend (causal=1) is served");
  MSGL_CHECK(page_size >= 1, MSGL_ERR_UNSUPPORTED, "page_size %d must be >= 1", page_size);
  MSGL_CHECK(max_extend_len >= 0 && max_kv_len >= max_extend_len, MSGL_ERR_SHAPE,
             "need 0 <= max_extend_len <= max_kv_len");
  MSGL_CHECK(q_row_stride >= (int64_t)num_q_heads * head_dim, MSGL_ERR_SHAPE,
             "q_row_stride %lld < num_q_heads*head_dim", (long long)q_row_stride);
  MSGL_CHECK(page_table_stride >= max_kv_len, MSGL_ERR_SHAPE,
             "page_table_stride %lld < max_kv_len %d", (long long)page_table_stride, max_kv_len);
  MSGL_CHECK(cache_row_stride * 2 <= (int64_t)UINT32_MAX, MSGL_ERR_SHAPE,
             "cache_row_stride %lld: a pool row must be under 4 GiB", (long long)cache_row_stride);
  if (batch == 0 || max_extend_len == 0) return MSGL_OK;
  MSGL_CHECK(out && q && page_table && prefix_lens && extend_lens && q_offsets, MSGL_ERR_NULL,
             "out, q, page_table, prefix_lens, extend_lens and q_offsets must be non-NULL");
  MSGL_CHECK(aligned(q, 16) && aligned(out, 16), MSGL_ERR_ALIGN, "q and out must be 16-byte aligned");
  MSGL_CHECK((q_row_stride * 2) % 16 == 0, MSGL_ERR_ALIGN, "q_row_stride*2 must be a multiple of 16");
  MSGL_CHECK(aligned(page_table, 4) && aligned(prefix_lens, 4) && aligned(extend_lens, 4) &&
                 aligned(q_offsets, 4) && (!req_rows || aligned(req_rows, 4)) &&
                 (!lse_out || aligned(lse_out, 4)),
             MSGL_ERR_ALIGN, "int32/fp32 arrays must be 4-byte aligned");
  const size_t ws_need = msgl::extend_workspace_bytes(batch, num_q_heads / num_kv_heads,
                                                      max_extend_len);
  MSGL_CHECK((int64_t)(ws_need - 16) / 4 * num_kv_heads < INT32_MAX, MSGL_ERR_SHAPE,
             "batch x query tiles x num_kv_heads exceeds the launch grid");
  MSGL_CHECK(!workspace || workspace_bytes >= ws_need, MSGL_ERR_WORKSPACE,
             "extend workspace holds %zu bytes, the work list needs %zu", workspace_bytes, ws_need);
  MSGL_CHECK(!workspace || aligned(workspace, 16), MSGL_ERR_ALIGN,
             "workspace must be 16-byte aligned");

  msgl::ExtendArgs a;
  a.out = out;
  a.lse = lse_out;
  a.q = q;
  a.q_stride = q_row_stride;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_slots = num_slots;
  a.cache_stride = cache_row_stride;
  a.page_table = page_table;
  a.pt_stride = page_table_stride;
  a.req_rows = req_rows;
  a.prefix_lens = prefix_lens;
  a.extend_lens = extend_lens;
  a.q_offsets = q_offsets;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.page_size = page_size;
  a.max_extend_len = max_extend_len;
  a.max_kv_len = max_kv_len;
  a.sm_scale = sm_scale;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = stream;
  if (g_validate_only) return MSGL_OK;
#ifdef MSGL_DEBUG_CHECKS
  {
    msgl::DebugRequestCheck c;
    c.lens = prefix_lens;
    c.ext = extend_lens;
    c.q_offsets = q_offsets;
    c.req_rows = req_rows;
    c.pt = page_table;
    c.pt_stride = page_table_stride;
    c.batch = batch;
    c.max_total = max_kv_len;
    c.max_ext = max_extend_len;
    c.num_slots = num_slots;
    c.page_span = page_span(page_size);
    if (int dst = debug_gate_requests(c, nullptr, false, stream, "paged_extend")) return dst;
  }
#endif
  return launch_status(msgl::launch_paged_extend(a), "paged_extend");
}

int msgl_embedding_gather(void* out, int64_t out_row_stride, const void* weights,
                          int64_t num_rows, int64_t weight_row_stride, const void* ids,
                          int32_t index_dtype, int64_t n, int64_t vocab_start, int32_t hidden,
                          int32_t dtype, hipStream_t stream) {
  g_last_error[0] = 0;
  MSGL_CHECK(n >= 0, MSGL_ERR_SHAPE, "n %lld is negative", (long long)n);
  MSGL_CHECK(num_rows >= 0, MSGL_ERR_SHAPE, "num_rows %lld is negative", (long long)num_rows);
  MSGL_CHECK(hidden > 0, MSGL_ERR_SHAPE, "hidden %d must be positive", hidden);
  MSGL_CHECK(dtype == MSGL_DTYPE_BF16 || dtype == MSGL_DTYPE_F32, MSGL_ERR_UNSUPPORTED,
             "dtype %d unsupported", dtype);
  MSGL_CHECK(index_dtype == MSGL_INDEX_I32 || index_dtype == MSGL_INDEX_I64, MSGL_ERR_UNSUPPORTED,
             "index dtype %d unsupported", index_dtype);
  MSGL_CHECK(out_row_stride >= hidden && weight_row_stride >= hidden, MSGL_ERR_SHAPE,
             "row strides (%lld, %lld) must be >= hidden %d", (long long)out_row_stride,
             (long long)weight_row_stride, hidden);
  if (n == 0) return MSGL_OK;
  MSGL_CHECK(out && ids && (weights || num_rows == 0), MSGL_ERR_NULL,
             "out, ids and weights must be non-NULL");
  const int esz = dtype == MSGL_DTYPE_BF16 ? 2 : 4;
  MSGL_CHECK(aligned(out, esz) && aligned(weights, esz), MSGL_ERR_ALIGN,
             "out and weights must be aligned to their element size");
  MSGL_CHECK(aligned(ids, index_dtype == MSGL_INDEX_I64 ? 8 : 4), MSGL_ERR_ALIGN,
             "ids must be aligned to their element size");

  msgl::GatherArgs a;
  a.out = out;
  a.out_stride_bytes = out_row_stride * esz;
  a.weights = weights;
  a.w_stride_bytes = weight_row_stride * esz;
  a.rows = num_rows;
  a.vocab_start = vocab_start;
  a.ids = ids;
  a.index_is_i64 = index_dtype == MSGL_INDEX_I64;
  a.n = n;
  a.row_bytes = (int64_t)hidden * esz;
  a.stream = stream;
  int unit = 16;
  while (unit > esz) {
    const bool ok = aligned(out, unit) && aligned(weights, unit) &&
                    a.out_stride_bytes % unit == 0 && a.w_stride_bytes % unit == 0 &&
                    a.row_bytes % unit == 0;
    if (ok) break;
    unit /= 2;
  }
  a.unit_bytes = unit;
  return launch_status(msgl::launch_embedding_gather(a), "embedding_gather");
}

int msgl_rope_cos_sin_cache(float* cache, int64_t max_position, int32_t rotary_dim, double base,
                            hipStream_t stream) {
  g_last_error[0] = 0;
  MSGL_CHECK(max_position >= 0, MSGL_ERR_SHAPE, "max_position %lld is negative",
             (long long)max_position);
  MSGL_CHECK(rotary_dim > 0 && rotary_dim % 2 == 0, MSGL_ERR_SHAPE,
             "rotary_dim %d must be positive and even", rotary_dim);
  MSGL_CHECK(base > 0.0, MSGL_ERR_SHAPE, "base must be positive");
  if (max_position == 0) return MSGL_OK;
  MSGL_CHECK(cache, MSGL_ERR_NULL, "cache must be non-NULL");
  MSGL_CHECK(aligned(cache, 4), MSGL_ERR_ALIGN, "cache must be 4-byte aligned");
  return launch_status(msgl::launch_rope_cache(cache, max_position, rotary_dim, base, stream),
                       "rope_cos_sin_cache");
}

int msgl_qk_norm_rope_store(void* q_out, int64_t q_out_row_stride, void* k_cache, void* v_cache,
                            int64_t num_slots, int64_t cache_row_stride, const void* qkv,
                            int64_t qkv_row_stride, const void* q_norm_weight,
                            const void* k_norm_weight, float eps, const int32_t* positions,
                            const float* cos_sin_cache, int64_t max_position, const void* out_loc,
                            int32_t index_dtype, int64_t n, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, hipStream_t stream) {
  g_last_error[0] = 0;
  MSGL_CHECK(n >= 0, MSGL_ERR_SHAPE, "n %lld is negative", (long long)n);
  MSGL_CHECK(index_dtype == MSGL_INDEX_I32 || index_dtype == MSGL_INDEX_I64, MSGL_ERR_UNSUPPORTED,
             "index dtype %d unsupported", index_dtype);
  int st = validate_pool(k_cache, v_cache, num_slots, cache_row_stride, num_kv_heads, head_dim);
  if (st) return st;
  MSGL_CHECK(ratio_ok(num_q_heads, num_kv_heads), MSGL_ERR_UNSUPPORTED,
             "num_q_heads %d / num_kv_heads %d: ratio must be 1, 2, 4, 8 or 16", num_q_heads,
             num_kv_heads);
  MSGL_CHECK(qkv_row_stride >= (int64_t)(num_q_heads + 2 * num_kv_heads) * head_dim, MSGL_ERR_SHAPE,
             "qkv_row_stride %lld < (Hq + 2 Hkv) * head_dim", (long long)qkv_row_stride);
  MSGL_CHECK(q_out_row_stride >= (int64_t)num_q_heads * head_dim, MSGL_ERR_SHAPE,
             "q_out_row_stride %lld < Hq * head_dim", (long long)q_out_row_stride);
  MSGL_CHECK(max_position > 0, MSGL_ERR_SHAPE, "max_position must be positive");
  MSGL_CHECK(eps >= 0.f, MSGL_ERR_SHAPE, "eps must be non-negative");
  if (n == 0) return MSGL_OK;
  MSGL_CHECK(q_out && qkv && positions && cos_sin_cache && out_loc, MSGL_ERR_NULL,
             "q_out, qkv, positions, cos_sin_cache and out_loc must be non-NULL");
  MSGL_CHECK(aligned(q_out, 16) && aligned(qkv, 16) &&
                 (!q_norm_weight || aligned(q_norm_weight, 16)) &&
                 (!k_norm_weight || aligned(k_norm_weight, 16)) && aligned(positions, 4) &&
                 aligned(cos_sin_cache, 16) &&
                 aligned(out_loc, index_dtype == MSGL_INDEX_I64 ? 8 : 4),
             MSGL_ERR_ALIGN, "rows, weights and table 16-byte aligned, indices element aligned");
  MSGL_CHECK(qkv_row_stride % 8 == 0 && q_out_row_stride % 8 == 0 && cache_row_stride % 8 == 0,
             MSGL_ERR_ALIGN,
             "qkv, q_out and pool row strides must be multiples of 8 elements (16 bytes)");
  MSGL_CHECK(aligned(k_cache, 16) && aligned(v_cache, 16), MSGL_ERR_ALIGN,
             "k_cache and v_cache must be 16-byte aligned");

  msgl::PrologueArgs a;
  a.q_out = q_out;
  a.q_out_stride = q_out_row_stride;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_stride = cache_row_stride;
  a.qkv = qkv;
  a.qkv_stride = qkv_row_stride;
  a.q_norm_w = q_norm_weight;
  a.k_norm_w = k_norm_weight;
  a.eps = eps;
  a.positions = positions;
  a.cache = cos_sin_cache;
  a.max_position = max_position;
  a.out_loc = out_loc;
  a.index_is_i64 = index_dtype == MSGL_INDEX_I64;
  a.n = n;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.stream = stream;
#ifdef MSGL_DEBUG_CHECKS
  if (int dst = debug_gate_out_loc(out_loc, a.index_is_i64, n, num_slots, stream,
                                   "qk_norm_rope_store"))
    return dst;
#endif
  return launch_status(msgl::launch_qk_norm_rope_store(a), "qk_norm_rope_store");
}

int msgl_merge_states(void* out, float* lse_out, const float* part_out, const float* part_lse,
                      int32_t num_parts, int64_t n, int32_t num_heads, int32_t head_dim,
                      int32_t out_dtype, hipStream_t stream) {
  g_last_error[0] = 0;
  MSGL_CHECK(num_parts >= 1, MSGL_ERR_SHAPE, "num_parts %d must be >= 1", num_parts);
  MSGL_CHECK(n >= 0 && num_heads > 0, MSGL_ERR_SHAPE, "n must be >= 0 and num_heads > 0");
  MSGL_CHECK(head_dim > 0 && head_dim % 4 == 0 && head_dim <= 256, MSGL_ERR_UNSUPPORTED,
             "head_dim %d must be a positive multiple of 4, at most 256", head_dim);
  MSGL_CHECK(out_dtype == MSGL_DTYPE_BF16 || out_dtype == MSGL_DTYPE_F32, MSGL_ERR_UNSUPPORTED,
             "out dtype %d unsupported", out_dtype);
  MSGL_CHECK(n <= 0x7fffffffLL, MSGL_ERR_SHAPE, "n too large");
  if (n == 0) return MSGL_OK;
  MSGL_CHECK(out && part_out && part_lse, MSGL_ERR_NULL, "out, part_out and part_lse must be non-NULL");
  MSGL_CHECK(aligned(part_out, 16) && aligned(part_lse, 4) && aligned(out, 16) &&
                 (!lse_out || aligned(lse_out, 4)),
             MSGL_ERR_ALIGN, "part_out/out must be 16-byte aligned, lse arrays 4-byte aligned");
  msgl::MergeArgs a;
  a.out = out;
  a.lse = lse_out;
  a.part_out = part_out;
  a.part_lse = part_lse;
  a.num_parts = num_parts;
  a.n = n;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.out_bf16 = out_dtype == MSGL_DTYPE_BF16;
  a.seq_lens = nullptr;
  a.split_tokens = 0;
  a.meta = nullptr;
  a.stream = stream;
  if (g_validate_only) return MSGL_OK;
  return launch_status(msgl::launch_merge(a), "merge_states");
}

int msgl_validate_store_kv(void* k_cache, void* v_cache, int64_t num_slots,
                           int64_t cache_row_stride, const void* k_new, const void* v_new,
                           int64_t new_row_stride, const void* out_loc, int32_t index_dtype,
                           int64_t n, int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
  return validate_only([&] {
    return msgl_store_kv(k_cache, v_cache, num_slots, cache_row_stride, k_new, v_new,
                         new_row_stride, out_loc, index_dtype, n, num_kv_heads, head_dim, dtype,
                         nullptr);
  });
}

int msgl_validate_paged_decode(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                               const void* k_cache, const void* v_cache, int64_t num_slots,
                               int64_t cache_row_stride, const int32_t* page_table,
                               int64_t page_table_stride, const int32_t* req_rows,
                               const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               int32_t max_seq_len, float sm_scale, int32_t split_tokens,
                               void* workspace, size_t workspace_bytes) {
  return validate_only([&] {
    return msgl_paged_decode(out, lse_out, q, q_row_stride, k_cache, v_cache, num_slots,
                             cache_row_stride, page_table, page_table_stride, req_rows, seq_lens,
                             batch, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                             sm_scale, split_tokens, workspace, workspace_bytes, nullptr);
  });
}

int msgl_validate_store_kv_paged_decode(
    void* out, float* lse_out, const void* q, int64_t q_row_stride, void* k_cache, void* v_cache,
    int64_t num_slots, int64_t cache_row_stride, const void* k_new, const void* v_new,
    int64_t new_row_stride, const void* out_loc, int32_t index_dtype, const int32_t* page_table,
    int64_t page_table_stride, const int32_t* req_rows, const int32_t* seq_lens, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    int32_t max_seq_len, float sm_scale, int32_t split_tokens, void* workspace,
    size_t workspace_bytes) {
  return validate_only([&] {
    return msgl_store_kv_paged_decode(out, lse_out, q, q_row_stride, k_cache, v_cache, num_slots,
                                      cache_row_stride, k_new, v_new, new_row_stride, out_loc,
                                      index_dtype, page_table, page_table_stride, req_rows,
                                      seq_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                      page_size, max_seq_len, sm_scale, split_tokens, workspace,
                                      workspace_bytes, nullptr);
  });
}

int msgl_validate_paged_extend(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                               const void* k_cache, const void* v_cache, int64_t num_slots,
                               int64_t cache_row_stride, const int32_t* page_table,
                               int64_t page_table_stride, const int32_t* req_rows,
                               const int32_t* prefix_lens, const int32_t* extend_lens,
                               const int32_t* q_offsets, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               int32_t max_extend_len, int32_t max_kv_len, float sm_scale,
                               int32_t causal, void* workspace, size_t workspace_bytes) {
  return validate_only([&] {
    return msgl_paged_extend(out, lse_out, q, q_row_stride, k_cache, v_cache, num_slots,
                             cache_row_stride, page_table, page_table_stride, req_rows,
                             prefix_lens, extend_lens, q_offsets, batch, num_q_heads,
                             num_kv_heads, head_dim, page_size, max_extend_len, max_kv_len,
                             sm_scale, causal, workspace, workspace_bytes, nullptr);
  });
}

int msgl_validate_merge_states(void* out, float* lse_out, const float* part_out,
                               const float* part_lse, int32_t num_parts, int64_t n,
                               int32_t num_heads, int32_t head_dim, int32_t out_dtype) {
  return validate_only([&] {
    return msgl_merge_states(out, lse_out, part_out, part_lse, num_parts, n, num_heads, head_dim,
                             out_dtype, nullptr);
  });
}

}  // extern "C"

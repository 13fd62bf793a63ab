// Device-side checks of the index arrays, for the debug-check build.
//
// The release kernels trust the lengths and indices that live in device
// memory, as the pages' kernels do ("Mini-SGLang complete analysis" §4.6.4:
// page_table, cache_seqlens and cu_seqlens come from the scheduler; §4.9.4:
// out_loc holds the slots store_kv writes).  The library built with
// MSGL_DEBUG_CHECKS runs the checkers below on the call's stream before the
// call's own kernels, waits for them, and refuses the call if any index is
// out of range, so a bad index never reaches a kernel that would write
// outside the pool or read outside a page-table row.  Every read a checker
// makes is bounded by host-validated sizes (the table width, the declared
// maxima), with one exception the ABI cannot close: a req_rows entry beyond
// the last table row (the calls carry no row count).
//
// A failing check sets its bit in a per-device report word and the first
// failure claims the detail fields; the host reads and clears the report.

#include <algorithm>

#include "internal.hpp"

#ifdef MSGL_DEBUG_CHECKS

namespace msgl {

namespace {

// [0] bits of every failure, [1] claimed by the first failure, [2] its bit,
// [3] request / index, [4] key or second value, [5..6] 64-bit value
__device__ __align__(16) unsigned int debug_report[8];

__device__ void report(unsigned int* w, unsigned int bit, int a, int b, long long v) {
  atomicOr(&w[0], bit);
  if (atomicCAS(&w[1], 0u, 1u) == 0u) {
    w[2] = bit;
    w[3] = (unsigned int)a;
    w[4] = (unsigned int)b;
    w[5] = (unsigned int)((unsigned long long)v & 0xffffffffull);
    w[6] = (unsigned int)((unsigned long long)v >> 32);
  }
}

template <typename Index>
__global__ void __launch_bounds__(256)
check_out_loc_kernel(const Index* out_loc, int64_t n, int64_t num_slots, unsigned int* w) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const long long v = (long long)out_loc[i];
    if (v < 0 || v >= num_slots)
      report(w, kDebugOutLoc, (int)std::min<int64_t>(i, INT32_MAX), -1, v);
  }
}

// One workgroup per request (grid-stride): lengths, query offsets, table row
// and the table entries the attention kernels read for that request.
__global__ void __launch_bounds__(256) check_requests_kernel(DebugRequestCheck c) {
  for (int r = blockIdx.x; r < c.batch; r += gridDim.x) {
    const int P = c.lens[r];                 // seq_len (decode) or prefix_len (extend)
    const int E = c.ext ? c.ext[r] : 0;
    const long long total = (long long)P + E;
    const long long width = std::min<long long>(c.max_total, c.pt_stride);
    if (threadIdx.x == 0) {
      const bool bad = P < 0 || E < 0 || total > c.max_total || total > c.pt_stride ||
                       (c.ext && E > c.max_ext);
      if (bad) report(c.w, kDebugLength, r, E, P);
      if (c.q_offsets) {
        const int o0 = c.q_offsets[r];
        const int o1 = c.q_offsets[r + 1];
        if (o0 < 0 || o1 - o0 != E) report(c.w, kDebugQOffsets, r, o1 - o0, o0);
      }
    }
    const int row = c.req_rows ? c.req_rows[r] : r;
    if (row < 0) {
      if (threadIdx.x == 0) report(c.w, kDebugRow, r, -1, row);
      continue;
    }
    const int32_t* prow = c.pt + (int64_t)row * c.pt_stride;
    const long long lim = std::max(0LL, std::min(total, width));
    const int span = c.page_span;
    for (long long k = (long long)threadIdx.x * span; k < lim; k += (long long)blockDim.x * span) {
      const long long e = prow[k];
      const long long reach = std::min<long long>(span, lim - k);
      if (e < 0 || e + reach - 1 >= c.num_slots) report(c.w, kDebugSlot, r, (int)k, e);
    }
    // fused store + decode: the new row's slot must be the request's newest key
    if (c.out_loc && threadIdx.x == 0 && P >= 1 && P <= lim) {
      const long long key = P - 1;
      const long long off = key % span;
      const long long slot = (long long)prow[key - off] + off;
      const long long want = c.out_loc_i64 ? reinterpret_cast<const int64_t*>(c.out_loc)[r]
                                           : reinterpret_cast<const int32_t*>(c.out_loc)[r];
      if (want != slot) report(c.w, kDebugNewestSlot, r, (int)key, want);
    }
  }
}

// Address of this device's report (looked up once per device).
hipError_t report_word(unsigned int** out) {
  static unsigned int* cache[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!cache[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_report));
    if (e != hipSuccess) return e;
    cache[dev] = static_cast<unsigned int*>(p);
  }
  *out = cache[dev];
  return hipSuccess;
}

}  // namespace

bool debug_stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

hipError_t debug_check_out_loc(const void* out_loc, bool i64, int64_t n, int64_t num_slots,
                               hipStream_t s) {
  unsigned int* w = nullptr;
  hipError_t e = report_word(&w);
  if (e != hipSuccess || n <= 0) return e;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
  if (i64)
    hipLaunchKernelGGL(check_out_loc_kernel<int64_t>, dim3(blocks), dim3(256), 0, s,
                       (const int64_t*)out_loc, n, num_slots, w);
  else
    hipLaunchKernelGGL(check_out_loc_kernel<int32_t>, dim3(blocks), dim3(256), 0, s,
                       (const int32_t*)out_loc, n, num_slots, w);
  return hipGetLastError();
}

hipError_t debug_check_requests(DebugRequestCheck c, hipStream_t s) {
  hipError_t e = report_word(&c.w);
  if (e != hipSuccess || c.batch <= 0) return e;
  const unsigned blocks = (unsigned)std::min(c.batch, 1024);
  hipLaunchKernelGGL(check_requests_kernel, dim3(blocks), dim3(256), 0, s, c);
  return hipGetLastError();
}

hipError_t debug_collect(hipStream_t s, DebugFailure* f) {
  unsigned int* w = nullptr;
  hipError_t e = report_word(&w);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  unsigned int h[8];
  e = hipMemcpy(h, w, sizeof(h), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  f->bits = h[0];
  f->first = h[2];
  f->a = (int)h[3];
  f->b = (int)h[4];
  f->v = (long long)(((unsigned long long)h[6] << 32) | h[5]);
  if (h[0] != 0u) {
    const unsigned int zero[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    e = hipMemcpy(w, zero, sizeof(zero), hipMemcpyHostToDevice);
  }
  return e;
}

}  // namespace msgl

#endif  // MSGL_DEBUG_CHECKS

// store_kv: scatter new K/V rows into one layer's pool planes.
//
// "Mini-SGLang complete analysis" §4.4.3: the pool, flattened per layer to
// (slots, kv heads, head_dim), is written at the batch's out_loc slots;
// §4.9.4 fixes the shape contract (pool [-1, D] with a row stride, new rows
// [L, D] with their own stride, L indices of int32 or int64); §4.9.5 copies a
// row with the widest vector unit its byte size allows.
//
// gfx950 mapping: one lane moves one W-byte unit of K and the same unit of V;
// consecutive lanes walk one row, so every wave issues fully coalesced
// 16-byte loads and stores (1 KiB per wave instruction for W = 16).

#include "common.hpp"
#include "internal.hpp"

namespace msgl {

template <int W, typename Index>
__global__ void __launch_bounds__(256)
store_kv_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                int64_t cache_stride_bytes, const char* __restrict__ k_new,
                const char* __restrict__ v_new, int64_t new_stride_bytes,
                const Index* __restrict__ out_loc, int64_t n, int32_t units_per_row) {
  typedef typename VecOf<W>::type T;
  const int64_t total = n * (int64_t)units_per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / units_per_row;
    const int64_t unit = i - row * units_per_row;
    const int64_t slot = (int64_t)out_loc[row];
    const int64_t src = row * new_stride_bytes + unit * W;
    const int64_t dst = slot * cache_stride_bytes + unit * W;
    const T kv = *reinterpret_cast<const T*>(k_new + src);
    const T vv = *reinterpret_cast<const T*>(v_new + src);
    *reinterpret_cast<T*>(k_cache + dst) = kv;
    *reinterpret_cast<T*>(v_cache + dst) = vv;
  }
}

template <int W, typename Index>
static hipError_t launch_store_w(const StoreArgs& a) {
  const int32_t units = (int32_t)(a.row_bytes / W);
  const int64_t total = a.n * (int64_t)units;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  hipLaunchKernelGGL((store_kv_kernel<W, Index>), dim3((unsigned)blocks), dim3(threads), 0,
                     a.stream, (char*)a.k_cache, (char*)a.v_cache, a.cache_stride_bytes,
                     (const char*)a.k_new, (const char*)a.v_new, a.new_stride_bytes,
                     (const Index*)a.out_loc, a.n, units);
  return hipGetLastError();
}

template <typename Index>
static hipError_t launch_store_idx(const StoreArgs& a) {
  switch (a.unit_bytes) {
    case 16: return launch_store_w<16, Index>(a);
    case 8: return launch_store_w<8, Index>(a);
    case 4: return launch_store_w<4, Index>(a);
    default: return launch_store_w<2, Index>(a);
  }
}

hipError_t launch_store_kv(const StoreArgs& a) {
  return a.index_is_i64 ? launch_store_idx<int64_t>(a) : launch_store_idx<int32_t>(a);
}

}  // namespace msgl

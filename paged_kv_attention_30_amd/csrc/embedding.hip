// Vocabulary-sharded embedding gather.
//
// "Mini-SGLang complete analysis" §4.9.3: one indexing(weights, ids,
// vocab_range) call copies one embedding-table row per token id; §4.7.8:
// embed_tokens is split along the vocabulary across tensor-parallel ranks
// and combined by masked indexing followed by an all-reduce, so a rank
// writes zeros for ids outside its vocabulary range.
//
// gfx950 mapping: one workgroup per output row at a time (grid-stride over
// rows).  The row's id is read once (uniform across the workgroup) and its
// 256 lanes copy the row in W-byte units (16 B when every address allows),
// so each wave moves 1 KiB per load or store instruction, fully coalesced.

#include "common.hpp"
#include "internal.hpp"

namespace msgl {

template <int W, typename Index>
__global__ void __launch_bounds__(256)
embedding_gather_kernel(char* __restrict__ out, int64_t out_stride_bytes,
                        const char* __restrict__ weights, int64_t w_stride_bytes,
                        const Index* __restrict__ ids, int64_t n, int64_t vocab_start,
                        int64_t rows, int32_t units_per_row) {
  typedef typename VecOf<W>::type T;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int64_t local = (int64_t)ids[r] - vocab_start;
    const bool hit = local >= 0 && local < rows;
    const char* src = weights + (hit ? local : 0) * w_stride_bytes;
    char* dst = out + r * out_stride_bytes;
    for (int32_t u = threadIdx.x; u < units_per_row; u += blockDim.x) {
      T v{};
      if (hit) v = *reinterpret_cast<const T*>(src + (int64_t)u * W);
      *reinterpret_cast<T*>(dst + (int64_t)u * W) = v;
    }
  }
}

template <int W, typename Index>
static hipError_t launch_gather_w(const GatherArgs& a) {
  const int32_t units = (int32_t)(a.row_bytes / W);
  int64_t blocks = a.n < 65536 ? a.n : 65536;   // grid-stride beyond this
  hipLaunchKernelGGL((embedding_gather_kernel<W, Index>), dim3((unsigned)blocks), dim3(256), 0,
                     a.stream, (char*)a.out, a.out_stride_bytes, (const char*)a.weights,
                     a.w_stride_bytes, (const Index*)a.ids, a.n, a.vocab_start, a.rows, units);
  return hipGetLastError();
}

template <typename Index>
static hipError_t launch_gather_idx(const GatherArgs& a) {
  switch (a.unit_bytes) {
    case 16: return launch_gather_w<16, Index>(a);
    case 8: return launch_gather_w<8, Index>(a);
    case 4: return launch_gather_w<4, Index>(a);
    default: return launch_gather_w<2, Index>(a);
  }
}

hipError_t launch_embedding_gather(const GatherArgs& a) {
  if (a.n == 0) return hipSuccess;
  return a.index_is_i64 ? launch_gather_idx<int64_t>(a) : launch_gather_idx<int32_t>(a);
}

}  // namespace msgl

// Log-sum-exp merge of partial attention states.
//
// The pages do not describe split-KV.  The merge is the identity that makes
// a softmax split over disjoint key sets equal the unsplit one: with part s
// holding the normalised output o_s and log-sum-exp lse_s of its keys,
//   M = max_s lse_s,  w_s = exp(lse_s - M),
//   o = sum_s w_s o_s / sum_s w_s,  lse = M + ln sum_s w_s.
//
// One lane handles four consecutive head dims of one (row, head); the
// partials are read with 16-byte loads in part order, so the result does not
// depend on scheduling.

#include "common.hpp"
#include "internal.hpp"

namespace msgl {

namespace {

struct MergeParams {
  void* out;
  float* lse;
  const float* part_out;
  const float* part_lse;
  int32_t num_parts;
  int64_t n;
  int32_t num_heads;
  int32_t head_dim;
  int32_t lanes_per_head;
  int32_t heads_per_block;
  int32_t out_bf16;
  const int32_t* seq_lens;
  int32_t split_tokens;
  const int32_t* meta;
};

__global__ void __launch_bounds__(256) merge_kernel(MergeParams p) {
  const int row = blockIdx.x;
  const int hl = threadIdx.x / p.lanes_per_head;
  const int d4 = threadIdx.x % p.lanes_per_head;
  const int h = blockIdx.y * p.heads_per_block + hl;
  if (hl >= p.heads_per_block || h >= p.num_heads) return;

  // part s of this row lives at partial row base + s * step
  int parts = p.num_parts;
  int64_t base = row, step = p.n;
  if (p.seq_lens) {
    const int L = p.seq_lens[row];
    parts = (L + p.split_tokens - 1) / p.split_tokens;
    if (parts <= 1) return;  // the decode kernel wrote this row itself
    if (parts > p.num_parts) parts = p.num_parts;
  } else if (p.meta) {
    const int bf = p.meta[2 * row];
    const int bl = p.meta[2 * row + 1];
    if (bf < 0) return;      // finished by a single workgroup
    parts = bl - bf + 1;
    base = (int64_t)bf + row;
    step = 1;
  }

  // One pass over the parts in order, eight at a time: their loads are
  // issued together, then folded with a running maximum (o and the weight
  // sum are rescaled whenever the maximum grows).  The fold order is the
  // part order, so the result does not depend on scheduling.
  const int64_t rh = (int64_t)row * p.num_heads + h;
  constexpr int kBatch = 8;
  float M = -INFINITY;
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < parts; s0 += kBatch) {
    const int n = min(kBatch, parts - s0);
    float ls[kBatch];
    f32x4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k < n) {
        const int64_t ph = (base + (int64_t)(s0 + k) * step) * p.num_heads + h;
        ls[k] = p.part_lse[ph];
        v[k] = *reinterpret_cast<const f32x4*>(p.part_out + ph * p.head_dim + 4 * d4);
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k < n && ls[k] != -INFINITY) {
        const float m_new = fmaxf(M, ls[k]);
        const float scale_old = fast_exp2((M - m_new) * kLog2e);
        const float w = fast_exp2((ls[k] - m_new) * kLog2e);
        acc = acc * scale_old + v[k] * w;
        wsum = wsum * scale_old + w;
        M = m_new;
      }
    }
  }
  if (M != -INFINITY) acc = acc * (1.f / wsum);

  if (p.out_bf16) {
    uint16_t* o = (uint16_t*)p.out + rh * p.head_dim + 4 * d4;
    u32x2 v;
    v[0] = pack_bf16x2(acc[0], acc[1]);
    v[1] = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<u32x2*>(o) = v;
  } else {
    float* o = (float*)p.out + rh * p.head_dim + 4 * d4;
    *reinterpret_cast<f32x4*>(o) = acc;
  }
  if (p.lse && d4 == 0)
    p.lse[rh] = (M == -INFINITY) ? -INFINITY : M + fast_log2(wsum) * kLn2;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a) {
  MergeParams p;
  p.out = a.out;
  p.lse = a.lse;
  p.part_out = a.part_out;
  p.part_lse = a.part_lse;
  p.num_parts = a.num_parts;
  p.n = a.n;
  p.num_heads = a.num_heads;
  p.head_dim = a.head_dim;
  p.lanes_per_head = a.head_dim / 4;
  p.heads_per_block = 256 / p.lanes_per_head;
  p.out_bf16 = a.out_bf16 ? 1 : 0;
  p.seq_lens = a.seq_lens;
  p.split_tokens = a.split_tokens;
  p.meta = a.meta;
  if (a.n == 0) return hipSuccess;
  dim3 grid((unsigned)a.n, (unsigned)((a.num_heads + p.heads_per_block - 1) / p.heads_per_block));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace msgl

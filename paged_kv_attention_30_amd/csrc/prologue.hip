// Attention-layer prologue: q/k RMSNorm + RoPE + store of K/V, fused.
//
// "Mini-SGLang complete analysis" §4.6.7: the merged qkv projection output is
// split into q, k, v; with q/k norms (Qwen3) q and k are RMS-normalised per
// head; RoPE rotates q and k at the batch's positions; k and v are stored
// into the paged pool at out_loc before the attention kernel runs.  §4.5.6:
// one cos/sin table (max_position x rotary_dim) is shared by every layer.
//
// gfx950 mapping: one wave per token, its heads four at a time; 16 lanes per
// head, lane j of a head holding dims 8j .. 8j+7 (one 16-byte load, so a wave
// instruction moves 1 KiB).  The RMS is a sum over the 16 lanes; rotate-half
// pairs dim i with dim i + 64, which sits in lane j ^ 8, so one cross-lane
// exchange per value brings the partner.  Math in fp32, one rounding to bf16
// at the end.  The table kernel builds cos/sin in double precision (angle
// and functions) and rounds to fp32 once.

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace msgl {

namespace {

__global__ void __launch_bounds__(256)
rope_cache_kernel(float* __restrict__ cache, int64_t max_position, int32_t rotary_dim, double base) {
  const int half = rotary_dim / 2;
  const int64_t total = max_position * half;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t pos = idx / half;
    const int i = (int)(idx - pos * half);
    const double theta = pow(base, -2.0 * (double)i / (double)rotary_dim);
    const double ang = (double)pos * theta;
    cache[pos * rotary_dim + i] = (float)cos(ang);
    cache[pos * rotary_dim + half + i] = (float)sin(ang);
  }
}

// sum over the 16 lanes of a lane group
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) v += shfl_xor(v, d);
  return v;
}

// One wave per token (grid-stride over tokens).  The token's position,
// slot and cos/sin row are read once; its heads are handled four at a time
// (16 lanes per head), kChunk groups of four per step with all their 16-byte
// loads issued before any is used, so a wave keeps kChunk KiB of reads in
// flight.
constexpr int kChunk = 4;

template <typename Index>
__global__ void __launch_bounds__(256) qk_norm_rope_store_kernel(PrologueArgs a) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4;          // head within a group of four
  const int j = lane & 15;            // this lane's dims 8j .. 8j+7
  const int heads = a.num_q_heads + 2 * a.num_kv_heads;
  const int groups = (heads + 3) / 4;
  const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t wstep = (int64_t)gridDim.x * (blockDim.x >> 6);
  // norm weights of this lane's dims (the same for every token)
  u32x4 wq = {0u, 0u, 0u, 0u}, wk = {0u, 0u, 0u, 0u};
  if (a.q_norm_w) wq = ld16((const uint16_t*)a.q_norm_w + 8 * j);
  if (a.k_norm_w) wk = ld16((const uint16_t*)a.k_norm_w + 8 * j);
  const float sgn = j < 8 ? -1.f : 1.f;    // first half: x cos - x' sin
  for (int64_t t = wave0; t < a.n; t += wstep) {
    const int64_t slot = (int64_t)((const Index*)a.out_loc)[t];
    int64_t pos = a.positions[t];
    pos = pos < 0 ? 0 : (pos >= a.max_position ? a.max_position - 1 : pos);
    // rotate-half: dims 8j+e (j < 8) pair with 8j+e+64, held by lane ^ 8
    const float* trow = a.cache + pos * kHeadDim + 8 * (j & 7);
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(trow);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(trow + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(trow + 64);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(trow + 68);
    const uint16_t* src_row = (const uint16_t*)a.qkv + t * a.qkv_stride + 8 * j;
    for (int g0 = 0; g0 < groups; g0 += kChunk) {
      u32x4 raw[kChunk];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int h = 4 * (g0 + k) + sub;
        const int hh = h < heads ? h : heads - 1;
        raw[k] = ld16(src_row + (int64_t)hh * kHeadDim);
      }
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        if (g0 + k >= groups) break;
        const int h = 4 * (g0 + k) + sub;
        const bool live = h < heads;
        const int hh = live ? h : heads - 1;
        const bool is_q = hh < a.num_q_heads;
        const bool is_v = hh >= a.num_q_heads + a.num_kv_heads;
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_lo(raw[k][e]);
          x[2 * e + 1] = bf16_hi(raw[k][e]);
        }
        // RMSNorm over the 128 dims of the head (16 lanes x 8)
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        ss = group16_sum(ss);
        const bool has_w = is_q ? a.q_norm_w != nullptr : a.k_norm_w != nullptr;
        if (has_w && !is_v) {
          const float inv = 1.f / sqrtf(ss * (1.f / kHeadDim) + a.eps);
          const u32x4 wr = is_q ? wq : wk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = x[2 * e] * inv * bf16_lo(wr[e]);
            x[2 * e + 1] = x[2 * e + 1] * inv * bf16_hi(wr[e]);
          }
        }
        u32x4 outw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ca = e < 2 ? c0[2 * e] : c1[2 * e - 4];
          const float cb = e < 2 ? c0[2 * e + 1] : c1[2 * e - 3];
          const float sa = e < 2 ? s0[2 * e] : s1[2 * e - 4];
          const float sb = e < 2 ? s0[2 * e + 1] : s1[2 * e - 3];
          const float pa = shfl_xor(x[2 * e], 8);
          const float pb = shfl_xor(x[2 * e + 1], 8);
          outw[e] = pack_bf16x2(x[2 * e] * ca + sgn * pa * sa, x[2 * e + 1] * cb + sgn * pb * sb);
        }
        if (!live) continue;
        if (is_v) {
          st16((uint16_t*)a.v_cache + slot * a.cache_stride +
                   (int64_t)(hh - a.num_q_heads - a.num_kv_heads) * kHeadDim + 8 * j,
               raw[k]);
        } else if (is_q) {
          st16((uint16_t*)a.q_out + t * a.q_out_stride + (int64_t)hh * kHeadDim + 8 * j, outw);
        } else {
          st16((uint16_t*)a.k_cache + slot * a.cache_stride +
                   (int64_t)(hh - a.num_q_heads) * kHeadDim + 8 * j,
               outw);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_rope_cache(float* cache, int64_t max_position, int32_t rotary_dim, double base,
                             hipStream_t stream) {
  const int64_t total = max_position * (rotary_dim / 2);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, cache,
                     max_position, rotary_dim, base);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope_store(const PrologueArgs& a) {
  const int64_t waves = a.n;   // one per token
  if (waves == 0) return hipSuccess;
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 65536) blocks = 65536;   // grid-stride beyond this
  if (a.index_is_i64)
    hipLaunchKernelGGL(qk_norm_rope_store_kernel<int64_t>, dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, a);
  else
    hipLaunchKernelGGL(qk_norm_rope_store_kernel<int32_t>, dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, a);
  return hipGetLastError();
}

}  // namespace msgl

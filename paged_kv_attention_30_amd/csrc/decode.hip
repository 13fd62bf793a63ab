// Paged GQA decode with split-KV.
//
// Method ("Mini-SGLang complete analysis"): §1.2 — a decode step carries one
// new token per request and is bound by reading the cached K/V; §1.4 — the
// K/V of every request lives in one pool and is reached through the
// request's page-table row; §4.5.3 — a group of ratio = Hq / Hkv query heads
// shares one kv head; §4.6.4 — the table is token granular (page_size 1
// view), so key j of a request sits in slot page_table[row, j]; §4.6.7 — the
// new token was stored before the kernel runs, so seq_len counts it.
//
// gfx950 design (one wave = one kv head of one request over one key chunk):
// * Keys are processed 32 at a time.  Each lane fetches the page-table entry
//   of "its" token and issues 16-byte loads of that token's K and V row
//   segment (a wave reads 64 contiguous bytes per token per instruction).
// * S^T = K Q^T runs on the 16x16x32 bf16 MFMA: K rows go straight from the
//   loads into the A operand (row = token), q heads of the group are the
//   B operand columns (ratio <= 16, unused columns are zero).  The output
//   layout gives every lane one q head, so running max / sum / rescale are
//   per-lane scalars; the max needs two cross-lane steps.
// * O^T = V^T P^T also runs on MFMA: P^T is the QK output repacked to bf16
//   in place (its C layout is exactly the B layout of the next MFMA), and V^T
//   is staged through a wave-private LDS tile written transposed.
// * Split-KV: chunk c of request r covers keys [c*S, (c+1)*S).  Requests with
//   one chunk write the final bf16 output; the others write normalised fp32
//   partials + lse that msgl_merge_states' kernel combines.
// * Reduction order depends only on logical key positions, so results are
//   bit-identical under any slot permutation and for any page_size.

#include <float.h>

#include "common.hpp"
#include "internal.hpp"

namespace msgl {

namespace {

constexpr int kTile = 32;          // keys per inner iteration
constexpr int kVtPitch = 32;       // LDS elements per head-dim row of V^T

struct DecodeParams {
  uint16_t* out;
  float* lse;
  const uint16_t* q;
  int64_t q_stride;
  const char* k_cache;
  const char* v_cache;
  int64_t cache_stride_bytes;
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* req_rows;
  const int32_t* seq_lens;
  int32_t batch;
  int32_t num_q_heads;
  int32_t ratio;
  int32_t split_tokens;
  int32_t max_splits;
  float scale_log2;       // sm_scale * log2(e)
  float* part_out;
  float* part_lse;
};

// position of key t (0..31 of a tile) inside a V^T row: the B-operand slot
// (l / 16, e) of the PV MFMA stands for key 4*(l/16) + e (e < 4) or
// 16 + 4*(l/16) + (e - 4) (e >= 4), i.e. the keys the QK output left in lane l.
__device__ __forceinline__ int vt_pos(int t) {
  return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3);
}

template <int KVB>
__global__ void __launch_bounds__(KVB * 64)
paged_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[KVB][kHeadDim * kVtPitch];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = blockIdx.x % p.batch;
  const int split = blockIdx.x / p.batch;
  const int g = blockIdx.y * KVB + w;
  const int c = lane & 15;      // q-head column / token row inside the MFMA
  const int j = lane >> 4;      // k-slot group
  const int R = p.ratio;
  const int S = p.split_tokens;

  const int L = p.seq_lens[r];
  const int t0 = split * S;
  // a length beyond the host bound folds its tail into the last chunk, so
  // no chunk index ever exceeds the workspace
  const int nsplit = min((L + S - 1) / S, p.max_splits);

  if (L <= 0) {
    // empty request: output 0, lse -inf (written once, by chunk 0)
    if (split == 0 && c < R) {
      const int h = g * R + c;
      uint16_t* o = p.out + ((int64_t)r * p.num_q_heads + h) * kHeadDim;
      for (int mb = 0; mb < 8; ++mb) {
        u32x2 z = {0u, 0u};
        *reinterpret_cast<u32x2*>(o + 16 * mb + 4 * j) = z;
      }
      if (p.lse && j == 0) p.lse[(int64_t)r * p.num_q_heads + h] = -INFINITY;
    }
    return;
  }
  if (t0 >= L) return;
  const int t1 = (split == p.max_splits - 1) ? L : min(t0 + S, L);

  const int row = p.req_rows ? p.req_rows[r] : r;
  const int32_t* pt = p.page_table + (int64_t)row * p.pt_stride;

  // q of this lane's head as the B operand of S^T = K Q^T:
  // column c, k-slot (j, e) of step kk <-> head dim 32*kk + 8*j + e.
  u32x4 qb[4];
  {
    const bool valid = c < R;
    const uint16_t* qrow = p.q + (int64_t)r * p.q_stride + (int64_t)(g * R + (valid ? c : 0)) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = ld16(qrow + 32 * kk + 8 * j);
      qb[kk] = valid ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int64_t cs = p.cache_stride_bytes;
  const char* kbase = p.k_cache + (int64_t)g * kHeadDim * 2 + (32 * 0 + 8 * j) * 2;
  const char* vbase = p.v_cache + (int64_t)g * kHeadDim * 2 + (8 * j) * 2;
  uint16_t* vt = vt_lds[w];
  const int pos_a = vt_pos(c);        // key c of the tile
  const int pos_b = vt_pos(16 + c);   // key 16 + c

  f32x4 acc[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max, log2 units
  float l_run = 0.f;         // this lane's share of the running sum

  for (int tb = t0; tb < t1; tb += kTile) {
    const int ta = min(tb + c, t1 - 1);
    const int tbb = min(tb + 16 + c, t1 - 1);
    const int64_t sa = (int64_t)pt[ta];
    const int64_t sb = (int64_t)pt[tbb];

    u32x4 ka[4], kb[4], va[4], vb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      ka[kk] = ld16(kbase + sa * cs + 64 * kk);
      kb[kk] = ld16(kbase + sb * cs + 64 * kk);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      va[kk] = ld16(vbase + sa * cs + 64 * kk);
      vb[kk] = ld16(vbase + sb * cs + 64 * kk);
    }

    f32x4 s_a = {0.f, 0.f, 0.f, 0.f}, s_b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s_a = mfma16x16x32(ka[kk], qb[kk], s_a);
      s_b = mfma16x16x32(kb[kk], qb[kk], s_b);
    }

    // lane holds scores of keys tb+4j+i (s_a) and tb+16+4j+i (s_b), head c
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ka_i = tb + 4 * j + i;
      sv[i] = (ka_i < t1) ? s_a[i] * p.scale_log2 : -INFINITY;
      sv[4 + i] = (ka_i + 16 < t1) ? s_b[i] * p.scale_log2 : -INFINITY;
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    uint32_t pw[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // the running sum takes the fp32 weights (an exact lse); the PV
      // contraction takes them rounded to bf16
      const float p0 = fast_exp2(sv[2 * e] - m_new);
      const float p1 = fast_exp2(sv[2 * e + 1] - m_new);
      pw[e] = pack_bf16x2(p0, p1);
      psum += p0 + p1;
    }
    l_run = l_run * alpha + psum;
    const u32x4 pb = {pw[0], pw[1], pw[2], pw[3]};

    // V^T tile: lane holds V[key c][dims 32kk+8j .. +7] and V[key 16+c][...]
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * kk + 8 * j + 2 * e;
        const uint32_t wa = va[kk][e];
        const uint32_t wb = vb[kk][e];
        vt[d * kVtPitch + pos_a] = (uint16_t)(wa & 0xffffu);
        vt[(d + 1) * kVtPitch + pos_a] = (uint16_t)(wa >> 16);
        vt[d * kVtPitch + pos_b] = (uint16_t)(wb & 0xffffu);
        vt[(d + 1) * kVtPitch + pos_b] = (uint16_t)(wb >> 16);
      }
    }
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(vt + (16 * mb + c) * kVtPitch + 8 * j);
      acc[mb] = acc[mb] * alpha;
      acc[mb] = mfma16x16x32(a, pb, acc[mb]);
    }
    __builtin_amdgcn_wave_barrier();
  }

  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  if (c >= R) return;
  const int h = g * R + c;
  const float inv = 1.f / l_tot;
  const float lse_nat = (m_run + fast_log2(l_tot)) * kLn2;

  if (nsplit == 1) {
    uint16_t* o = p.out + ((int64_t)r * p.num_q_heads + h) * kHeadDim;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      u32x2 v;
      v[0] = pack_bf16x2(acc[mb][0] * inv, acc[mb][1] * inv);
      v[1] = pack_bf16x2(acc[mb][2] * inv, acc[mb][3] * inv);
      *reinterpret_cast<u32x2*>(o + 16 * mb + 4 * j) = v;
    }
    if (p.lse && j == 0) p.lse[(int64_t)r * p.num_q_heads + h] = lse_nat;
  } else {
    const int64_t idx = ((int64_t)split * p.batch + r) * p.num_q_heads + h;
    float* o = p.part_out + idx * kHeadDim;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      f32x4 v = acc[mb] * inv;
      *reinterpret_cast<f32x4*>(o + 16 * mb + 4 * j) = v;
    }
    if (j == 0) p.part_lse[idx] = lse_nat;
  }
}

template <int KVB>
hipError_t launch_kvb(const DecodeArgs& a, const DecodeParams& p) {
  dim3 grid((unsigned)((int64_t)a.max_splits * a.batch), (unsigned)(a.num_kv_heads / KVB));
  hipLaunchKernelGGL((paged_decode_kernel<KVB>), grid, dim3(KVB * 64), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a) {
  DecodeParams p;
  p.out = (uint16_t*)a.out;
  p.lse = a.lse;
  p.q = (const uint16_t*)a.q;
  p.q_stride = a.q_stride;
  p.k_cache = (const char*)a.k_cache;
  p.v_cache = (const char*)a.v_cache;
  p.cache_stride_bytes = a.cache_stride * 2;
  p.page_table = a.page_table;
  p.pt_stride = a.pt_stride;
  p.req_rows = a.req_rows;
  p.seq_lens = a.seq_lens;
  p.batch = a.batch;
  p.num_q_heads = a.num_q_heads;
  p.ratio = a.num_q_heads / a.num_kv_heads;
  p.split_tokens = a.split_tokens;
  p.max_splits = a.max_splits;
  p.scale_log2 = a.sm_scale * kLog2e;
  p.part_out = a.part_out;
  p.part_lse = a.part_lse;

  hipError_t err;
  if (a.num_kv_heads % 8 == 0) err = launch_kvb<8>(a, p);
  else if (a.num_kv_heads % 4 == 0) err = launch_kvb<4>(a, p);
  else if (a.num_kv_heads % 2 == 0) err = launch_kvb<2>(a, p);
  else err = launch_kvb<1>(a, p);
  if (err != hipSuccess || a.max_splits <= 1) return err;

  MergeArgs m;
  m.out = a.out;
  m.lse = a.lse;
  m.part_out = a.part_out;
  m.part_lse = a.part_lse;
  m.num_parts = a.max_splits;
  m.n = a.batch;
  m.num_heads = a.num_q_heads;
  m.head_dim = kHeadDim;
  m.out_bf16 = true;
  m.seq_lens = a.seq_lens;
  m.split_tokens = a.split_tokens;
  m.stream = a.stream;
  return launch_merge(m);
}

}  // namespace msgl

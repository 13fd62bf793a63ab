// Causal chunked-prefill ("extend") attention over a paged KV pool.
//
// Method: "Deep dive into mini-sglang: chunked prefill and overlap
// scheduling" (chunked-prefill section) — a long prompt is processed in
// chunks and each chunk attends to the KV its earlier chunks left in the
// cache plus itself; "Mini-SGLang complete analysis" §4.2.3 — a request has
// cached_len keys already in place and extend_len = device_len - cached_len
// new tokens this step; §4.6.5 — the queries of all requests are packed
// back to back (cu_seqlens_q); §4.6.7 — the new K/V were stored before the
// kernel.  Query i of a request with prefix P sees keys 0 .. P+i.
//
// gfx950 design: one workgroup of 4 waves takes one request, one kv head and
// 128 query rows made of (q head of the group, query position) pairs, so the
// K/V tiles staged in LDS serve the whole GQA group.  Per 64-key tile:
// * every lane loads the page-table entry of one key and 16-byte pieces of
//   that key's K and V rows into registers (prefetched one tile ahead),
//   then writes K row-major and V transposed (V^T) into LDS;
// * S^T = K Q^T on the 32x32x16 bf16 MFMA (A = K rows from LDS, B = q
//   rows held in registers);
// * online softmax per query row: every lane owns one query row, so the
//   rescale is a per-lane scalar; the row max needs one cross-lane step;
// * O^T = V^T P^T on MFMA, P^T being the S^T output repacked to bf16 in
//   place (its C layout is the next MFMA's B layout).

#include <float.h>

#include "common.hpp"
#include "internal.hpp"

namespace msgl {

namespace {

constexpr int kBN = 64;            // keys per tile
constexpr int kRows = 128;         // (head, position) rows per workgroup
constexpr int kKPitch = 136;       // LDS elements per key row of K (272 B)
constexpr int kVPitch = 72;        // LDS elements per head-dim row of V^T (144 B)

struct ExtendParams {
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
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  const int32_t* q_offsets;
  int32_t batch;
  int32_t num_q_heads;
  int32_t ratio;
  int32_t bq;              // query positions per workgroup = kRows / ratio
  int32_t n_qtiles;
  float scale_log2;
};

// LDS position of key k (0..63) inside a V^T row: slot (l/32, e) of PV step u
// holds key 16u + 8*(e/4) + 4*(l/32) + e%4, the keys the S^T output left in
// lane l; stored at 16u + 8*(l/32) + e.  Swaps bits 2 and 3 of k.
__device__ __forceinline__ int vt_pos64(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Rescale threshold of the online softmax, in log2 units: the running
// maximum is only moved (and O, l rescaled) when a new score exceeds it by
// more than this, so p = 2^(s - m) stays <= 2^8 while most tiles skip the
// rescale.  Softmax does not depend on the reference maximum, so this
// changes rounding only.
constexpr float kRescaleSlack = 8.f;

__global__ void __launch_bounds__(256, 2)
paged_extend_kernel(ExtendParams p) {
  // two K / V^T tile buffers: tile i+1 is written while tile i is read
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kBN * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][kHeadDim * kVPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = blockIdx.x % p.batch;
  const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / p.batch);   // heavy tiles first
  const int g = blockIdx.y;
  const int E = p.extend_lens[r];
  const int q0 = qt * p.bq;
  if (q0 >= E) return;
  const int P = p.prefix_lens[r];
  const int qoff = p.q_offsets[r];
  const int row = p.req_rows ? p.req_rows[r] : r;
  const int32_t* pt = p.page_table + (int64_t)row * p.pt_stride;
  const int R = p.ratio;

  // this lane's query row (column of S^T / O^T)
  const int col = lane & 31;
  const int jh = lane >> 5;
  const int rho = 32 * w + col;
  const int head_local = rho / p.bq;
  const int qpos_raw = q0 + rho % p.bq;
  const bool row_valid = qpos_raw < E;
  const int qpos = row_valid ? qpos_raw : E - 1;
  const int head = g * R + head_local;
  const int vis_end = P + qpos + 1;          // keys [0, vis_end) are visible

  // q as the B operand: column = query row, k-slot (jh, e) of step kk <->
  // head dim 16*kk + 8*jh + e
  u32x4 qb[8];
  {
    const uint16_t* qr = p.q + (int64_t)(qoff + qpos) * p.q_stride + (int64_t)head * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[kk] = ld16(qr + 16 * kk + 8 * jh);
  }

  // keys this workgroup needs: [0, kv_end)
  const int last_q = min(q0 + p.bq, E) - 1;
  const int kv_end = P + last_q + 1;
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // loader role: key tid % 64 of the tile, 16-byte chunks (tid / 64) + 4u
  const int ld_key = tid & 63;
  const int ld_chunk = tid >> 6;
  const int64_t cs = p.cache_stride_bytes;
  const char* kb = p.k_cache + (int64_t)g * kHeadDim * 2;
  const int64_t v_minus_k = p.v_cache - p.k_cache;
  const int vpos = vt_pos64(ld_key);

  // page-table entry of this lane's key, fetched one tile before its K/V so
  // the table walk never sits in front of the data loads
  auto slot_of = [&](int tile) -> int { return pt[min(tile * kBN + ld_key, kv_end - 1)]; };
  int next_slot = slot_of(0);
  u32x4 pk[4], pv[4];
  auto prefetch = [&](int tile) {
    const char* src = kb + (int64_t)next_slot * cs;
    next_slot = slot_of(tile + 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int off = (ld_chunk + 4 * u) * 16;
      pk[u] = ld16(src + off);
      pv[u] = ld16(src + v_minus_k + off);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int chunk = ld_chunk + 4 * u;
      *reinterpret_cast<u32x4*>(&k_lds[buf][ld_key * kKPitch + chunk * 8]) = pk[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = chunk * 8 + 2 * e;
        vt_lds[buf][d * kVPitch + vpos] = (uint16_t)(pv[u][e] & 0xffffu);
        vt_lds[buf][(d + 1) * kVPitch + vpos] = (uint16_t)(pv[u][e] >> 16);
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_run = -INFINITY;   // reference maximum, log2 units
  float l_run = 0.f;         // this lane's share of the running sum
  const float c = p.scale_log2;

  // the lowest visible-key bound among this wave's rows decides whether a
  // tile needs the causal mask
  int vis_min = vis_end;
  vis_min = min(vis_min, __builtin_amdgcn_ds_bpermute(((lane ^ 32) << 2), vis_min));
  for (int d = 16; d >= 1; d >>= 1)
    vis_min = min(vis_min, __builtin_amdgcn_ds_bpermute(((lane ^ d) << 2), vis_min));
  vis_min = __builtin_amdgcn_readfirstlane(vis_min);

  prefetch(0);
  stash(0);
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) prefetch(tile + 1);
    const int kt = tile * kBN;

    // S^T for key blocks 0 and 1 of the tile
    f32x16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb2][i] = 0.f;
      const uint16_t* krow = &k_lds[buf][(32 * kb2 + col) * kKPitch + 8 * jh];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 16 * kk);
        s[kb2] = mfma32x32x16(a, qb[kk], s[kb2]);
      }
    }

    // causal mask (only tiles that reach past some row's last visible key)
    const bool masked_tile = kt + kBN > vis_min;
    if (masked_tile) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt + 32 * kb2 + 8 * (i >> 2) + 4 * jh + (i & 3);
          if (key >= vis_end) s[kb2][i] = c >= 0.f ? -INFINITY : INFINITY;
        }
    }
    // tile maximum of c * s, in log2 units
    float ext = s[0][0];
    if (c >= 0.f) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) ext = fmaxf(ext, s[kb2][i]);
      ext = fmaxf(ext, shfl_xor(ext, 32));
    } else {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) ext = fminf(ext, s[kb2][i]);
      ext = fminf(ext, shfl_xor(ext, 32));
    }
    const float m_tile = c * ext;
    if (__any(m_tile > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = acc[mb] * alpha;
    }

    u32x4 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int i0 = 8 * (u & 1) + 2 * e2;
        float p0 = fast_exp2(fmaf(s[u >> 1][i0], c, -m_run));
        float p1 = fast_exp2(fmaf(s[u >> 1][i0 + 1], c, -m_run));
        if (masked_tile) {
          const int key0 = kt + 32 * (u >> 1) + 8 * (i0 >> 2) + 4 * jh + (i0 & 3);
          p0 = key0 < vis_end ? p0 : 0.f;
          p1 = key0 + 1 < vis_end ? p1 : 0.f;
        }
        pb[u][e2] = pack_bf16x2(p0, p1);
        psum += p0 + p1;
      }
    }
    l_run += psum;

#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint16_t* vrow = &vt_lds[buf][(32 * mb + col) * kVPitch + 8 * jh];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vrow + 16 * u);
        acc[mb] = mfma32x32x16(a, pb[u], acc[mb]);
      }
    }

    if (tile + 1 < n_tiles) stash(buf ^ 1);
    __syncthreads();
  }

  float l_tot = l_run + shfl_xor(l_run, 32);
  if (!row_valid) return;
  const float inv = 1.f / l_tot;
  const int64_t orow = (int64_t)(qoff + qpos) * p.num_q_heads + head;
  uint16_t* o = p.out + orow * kHeadDim;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      u32x2 v;
      v[0] = pack_bf16x2(acc[mb][4 * a4 + 0] * inv, acc[mb][4 * a4 + 1] * inv);
      v[1] = pack_bf16x2(acc[mb][4 * a4 + 2] * inv, acc[mb][4 * a4 + 3] * inv);
      *reinterpret_cast<u32x2*>(o + 32 * mb + 8 * a4 + 4 * jh) = v;
    }
  }
  if (p.lse && jh == 0) p.lse[orow] = (m_run + fast_log2(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_paged_extend(const ExtendArgs& a) {
  ExtendParams p;
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
  p.prefix_lens = a.prefix_lens;
  p.extend_lens = a.extend_lens;
  p.q_offsets = a.q_offsets;
  p.batch = a.batch;
  p.num_q_heads = a.num_q_heads;
  p.ratio = a.num_q_heads / a.num_kv_heads;
  p.bq = kRows / p.ratio;
  p.n_qtiles = (a.max_extend_len + p.bq - 1) / p.bq;
  p.scale_log2 = a.sm_scale * kLog2e;
  if (a.batch == 0 || p.n_qtiles == 0) return hipSuccess;
  dim3 grid((unsigned)((int64_t)p.n_qtiles * a.batch), (unsigned)a.num_kv_heads);
  hipLaunchKernelGGL(paged_extend_kernel, grid, dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace msgl

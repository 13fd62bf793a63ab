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
// gfx950 design.  A planning pass orders the (request, query tile) work
// items longest first; the attention grid is 1-D with the kv head varying
// fastest, so each XCD serves fixed kv heads and takes the longest items
// first.  One workgroup of 8 waves takes one request, one kv head and 256
// query rows made of (q head of the group, query position) pairs, so the
// K/V tiles staged in LDS serve the whole GQA group.  Per 64-key tile:
// * K and V go from HBM straight into LDS (global_load_lds_dwordx4: each
//   wave instruction fills 1 KiB of LDS, lane l at +16 l), issued from
//   inline assembly two tiles ahead into four stages, with explicit vmcnt
//   waits and one barrier per tile; no register staging.  Which key /
//   16-byte piece a lane fetches is chosen so the LDS tiles come out
//   XOR-swizzled for conflict-free operand reads.  The page-table entries
//   arrive the same way, into a small per-wave ring.
// * S^T = K Q^T on the 32x32x16 bf16 MFMA (A = K rows read from LDS, B = q
//   rows held in registers).
// * online softmax per query row (every lane owns one row); the reference
//   maximum moves only when a score exceeds it by more than 2^8 (see
//   kRescaleSlack), so most tiles skip the rescale of O.
// * O^T = V^T P^T on MFMA: P^T is the S^T output repacked to bf16 in place
//   (its C layout is the next MFMA's B layout); V^T operands come from the
//   key-major V tile through the transposing LDS read (ds_read_b64_tr_b16).

#include <float.h>

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"


namespace msgl {

namespace {

constexpr int kBN = 64;            // keys per tile
constexpr int kPvDepth = 3;        // V^T operand reads in flight ahead of the P V MFMAs
constexpr int kTileElems = kBN * kHeadDim;   // one K or V tile, bf16 elements
constexpr int kPieces = kTileElems * 2 / 1024;  // 1-KiB LDS pieces per K (or V) tile

// Workgroup barrier without the memory fence __syncthreads() carries (that
// fence waits for every outstanding load, including tiles meant to stay in
// flight).  Callers order LDS themselves: every wave has waited for its own
// tile loads (vmcnt) and consumed its LDS reads before arriving.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS accesses done
  asm volatile("s_barrier" ::: "memory");
}

// Rescale threshold of the online softmax, in log2 units: the running
// maximum is only moved (and O, l rescaled) when a new score exceeds it by
// more than this, so p = 2^(s - m) stays <= 2^8 while most tiles skip the
// rescale.  Softmax does not depend on the reference maximum, so this
// changes rounding only.
constexpr float kRescaleSlack = 8.f;

struct ExtendParams {
  uint16_t* out;
  float* lse;
  const uint16_t* q;
  int64_t q_stride;
  const char* k_cache;
  const char* v_cache;
  int64_t cache_stride_bytes;
  int64_t num_slots;
  const int32_t* page_table;
  int64_t pt_stride;
  int32_t page_mask;       // page_size - 1 for a power-of-two page_size, else 0
  const int32_t* req_rows;
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  const int32_t* q_offsets;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t ratio;
  int32_t bq;              // query positions per workgroup = 32 * waves / ratio
  int32_t n_qtiles;
  float scale_log2;
  const int32_t* work_count;   // sorted work list (null: natural order)
  const int32_t* work_list;
};

// K tile: key-major rows of 16 sixteen-byte chunks; chunk c of key t sits at
// position c ^ (t & 15), so 8 consecutive keys read at one chunk index hit 8
// different bank groups.  Returns the element offset.
__device__ __forceinline__ int k_off(int t, int chunk) {
  return t * kHeadDim + 8 * (chunk ^ (t & 15));
}

// V tile: key-major rows of 32 eight-byte groups; group cg of key t sits at
// cg ^ (8 * (t & 3)).  A transposed read serves 32 lanes = 4 keys (t & 3
// distinct) x 8 consecutive groups at once; the XOR sends the four keys to
// four disjoint blocks of 8 bank slots, so the read is conflict free, and it
// keeps the 16-byte pairs a direct load writes together.
__device__ __forceinline__ int v_off(int t, int cg) {
  return t * kHeadDim + 4 * (cg ^ (8 * (t & 3)));
}

constexpr int kWaves = 8;          // two groups of four: one wave of each group per SIMD
constexpr int kStages = 4;         // LDS K/V tile buffers
constexpr int kPtRing = 4;         // page-table entry slots per wave
constexpr int kPPW = kPieces / kWaves;   // 1-KiB pieces each wave loads per K (or V) tile

// Eight waves of 32 query rows each.  Waves 0-3 ("lead") and 4-7 ("lag")
// run the same tile loop half a tile apart: between two barriers the lead
// waves compute S = K Q^T, softmax and O += P V of tile k while the lag
// waves finish softmax and P V of tile k-1 and then compute S of tile k.
// Each SIMD holds one wave of each group, so one wave's MFMA work runs
// beside the other's softmax (exp and VALU) instead of both contending for
// the same unit at the same time.  A wave raises its issue priority while it
// issues MFMAs (S = K Q^T, O += P V) and drops it for the softmax, so the
// SIMD feeds the matrix unit first and fills the gaps with vector work.
// kPageOffsets: page_size > 1 (a power of two), so keys add their offset
// inside the page to the entry of the page's first column; the page_size 1
// instance drops that arithmetic from the load path.
template <bool kPageOffsets>
__global__ void __launch_bounds__(kWaves * 64, 1)
paged_extend_kernel(ExtendParams p) {
  // stage t % kStages holds the K and V of tile t
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[kStages * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[kStages * kTileElems];
  __shared__ __attribute__((aligned(16))) int32_t pt_ring[kWaves][kPtRing][kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  // Workgroup L takes kv head L % Hkv of work item L / Hkv.  Workgroups go
  // to the XCDs round-robin, so with the head index varying fastest each
  // XCD serves a fixed set of heads (their K/V stay in its L2) and receives
  // the work items in list order: longest first when the planner sorted
  // them, else last query tile first.
  const int L = blockIdx.x;
  const int g = L % p.num_kv_heads;
  const int slot = L / p.num_kv_heads;
  int r, qt;
  if (p.work_list) {
    if (slot >= *p.work_count) return;
    const int item = p.work_list[slot];
    r = item / p.n_qtiles;
    qt = item - r * p.n_qtiles;
  } else {
    r = slot % p.batch;
    qt = p.n_qtiles - 1 - slot / p.batch;
  }
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
  // head dim 16*kk + 8*jh + e.  A negative scale is applied as a sign flip
  // of q (exact in bf16, and every product and partial sum of the MFMA
  // flips sign with it under round-to-nearest-even), so the scores below
  // are always scaled by |scale|.
  u32x4 qb[8];
  {
    const uint16_t* qr = p.q + (int64_t)(qoff + qpos) * p.q_stride + (int64_t)head * kHeadDim;
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[kk] = ld16(qr + 16 * kk + 8 * jh) ^ qsign;
    // q is in registers before the look-ahead loads start (a wait the
    // compiler sees, so it adds none inside the tile loop)
    __builtin_amdgcn_s_waitcnt(0);
  }

  // keys this workgroup needs: [0, kv_end)
  const int last_q = min(q0 + p.bq, E) - 1;
  const int kv_end = P + last_q + 1;
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // Loader role: wave w issues the 1-KiB LDS pieces kPPW*w .. kPPW*w+kPPW-1
  // of each tile.  Piece I holds keys 4I .. 4I+3; lane l of it lands on key
  // 4I + l/16 at physical 16-byte position l % 16, i.e. K chunk
  // (l%16) ^ (key & 15) and V 16-byte unit (l%16) ^ (4 * (key & 3)).
  // row offsets in 32 x 32 -> 64-bit arithmetic (the host checks that the
  // row stride fits 32 bits); slots clamp to the pool (an unsigned minimum:
  // a negative entry takes the last slot)
  const uint32_t cs32 = (uint32_t)p.cache_stride_bytes;
  const uint32_t slot_max = (uint32_t)min(p.num_slots - 1, (int64_t)INT32_MAX);
  const char* kbase = p.k_cache + (int64_t)g * kHeadDim * 2;
  const int64_t v_minus_k = p.v_cache - p.k_cache;
  const int ld_keyoff = lane >> 4;     // key within a piece
  const int ld_phys = lane & 15;       // physical 16-byte position within the row
  // The page-table entries of tile t (64 ints) are fetched into this wave's
  // ring slot t % kPtRing by one 4-byte direct load per lane; the K/V loads
  // of tile t read their slots back from LDS.  Slots are clamped to the pool
  // so that an address can never leave it.
  // With page_size P > 1 (a power of two) the slots of a page are
  // consecutive: each lane fetches the entry of its key's page start (the
  // every-P-th-column view of "Mini-SGLang complete analysis" §4.6.4) and the
  // offset inside the page is added when the slot is read back.
  int32_t* ring = &pt_ring[w][0][0];
  const int pmask = kPageOffsets ? p.page_mask : 0;
  auto fetch_pt = [&](int tile) {
    const int key = min(tile * kBN + lane, kv_end - 1);
    dma4(pt + (key & ~pmask), ring + (tile & (kPtRing - 1)) * kBN);
  };
  auto issue_tile = [&](int tile) {
    const int stg = tile & (kStages - 1);
    uint16_t* kd = kbuf + stg * kTileElems;
    uint16_t* vd = vbuf + stg * kTileElems;
    const int32_t* rs = ring + (tile & (kPtRing - 1)) * kBN;
    // all table reads first: the loads below are opaque to the compiler,
    // so a read placed after one of them would wait for it
    int32_t slot[kPPW];
#pragma unroll
    for (int u = 0; u < kPPW; ++u) {
      const int key = 4 * (kPPW * w + u) + ld_keyoff;
      slot[u] = rs[key] + (min(tile * kBN + key, kv_end - 1) & pmask);
    }
#pragma unroll
    for (int u = 0; u < kPPW; ++u) {
      const int piece = kPPW * w + u;
      const int key = 4 * piece + ld_keyoff;       // key within the tile
      const uint32_t sl = min((uint32_t)slot[u], slot_max);
      const char* rowp = kbase + (uint64_t)sl * cs32;
      const int kchunk = ld_phys ^ (key & 15);
      const int vunit = ld_phys ^ (4 * (key & 3));
      dma16(rowp + 16 * kchunk, kd + piece * 512);
      dma16(rowp + v_minus_k + 16 * vunit, vd + piece * 512);
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_run = -INFINITY;   // reference maximum, log2 units
  float l_run = 0.f;         // this lane's share of the running sum
  const float c = fabsf(p.scale_log2);   // > 0 (the sign went into q)

  // the lowest visible-key bound among this wave's rows decides whether a
  // tile needs the causal mask
  int vis_min = vis_end;
  vis_min = min(vis_min, __builtin_amdgcn_ds_bpermute(((lane ^ 32) << 2), vis_min));
  for (int d = 16; d >= 1; d >>= 1)
    vis_min = min(vis_min, __builtin_amdgcn_ds_bpermute(((lane ^ d) << 2), vis_min));
  vis_min = __builtin_amdgcn_readfirstlane(vis_min);

  // transposed-read coordinates of this lane (16-lane group G = lane / 16):
  // lane 4k + q of the group points at key k of the 4-key run, dims
  // 32 mb + 16 (G & 1) + 4q
  const int tr_key = (lane & 15) >> 2;
  const int tr_cg = 4 * ((lane >> 4) & 1) + (lane & 3);

  // S^T for key blocks 0 and 1 of a tile
  f32x16 s[2];
  auto qk = [&](int tile) {
    __builtin_amdgcn_s_setprio(1);
    const uint16_t* kt_lds = kbuf + (tile & (kStages - 1)) * kTileElems;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb2][i] = 0.f;
      const int key = 32 * kb2 + col;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt_lds + k_off(key, 2 * kk + jh));
        s[kb2] = mfma32x32x16(a, qb[kk], s[kb2]);
      }
    }
  };

  // online softmax of the scores in s, then O^T += V^T P^T
  auto softmax_pv = [&](int tile) {
    const uint16_t* vt_lds = vbuf + (tile & (kStages - 1)) * kTileElems;
    const int kt = tile * kBN;
    __builtin_amdgcn_s_setprio(0);
    // causal mask (only tiles that reach past some row's last visible key)
    const bool masked_tile = kt + kBN > vis_min;
    if (masked_tile) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt + 32 * kb2 + 8 * (i >> 2) + 4 * jh + (i & 3);
          if (key >= vis_end) s[kb2][i] = -INFINITY;
        }
    }
    // tile maximum of c * s, in log2 units
    float ext = s[0][0];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) ext = fmaxf(ext, s[kb2][i]);
    const float m_tile = c * max_xor32(ext);
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
        // a masked score is -inf and m_run is finite here (key 0 is visible
        // to every row, and c > 0), so a masked key's weight is exactly 0
        const float p0 = fast_exp2(fmaf(s[u >> 1][i0], c, -m_run));
        const float p1 = fast_exp2(fmaf(s[u >> 1][i0 + 1], c, -m_run));
        pb[u][e2] = pack_bf16x2(p0, p1);
        psum += p0 + p1;
      }
    }
    l_run += psum;
    __builtin_amdgcn_s_setprio(1);

    // O^T += V^T P^T: slot (jh, e) of step u is key 16u + 8(e/4) + 4jh + e%4
    // 16 steps (u, mb) with the accumulator changing every step; the
    // operands of step st + kPvDepth - 1 are read while step st's MFMA runs
    // (the fences keep that order, so an LDS read is never waited for right
    // after it is issued)
    auto rdv = [&](int st) __attribute__((always_inline)) {
      const int u = st >> 2, mb = st & 3;
      const int key_lo = 16 * u + 4 * jh + tr_key;
      const u32x2 lo = lds_read_tr16(vt_lds + v_off(key_lo, 8 * mb + tr_cg));
      const u32x2 hi = lds_read_tr16(vt_lds + v_off(key_lo + 8, 8 * mb + tr_cg));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 va[kPvDepth];
#pragma unroll
    for (int d = 0; d < kPvDepth - 1; ++d) va[d] = rdv(d);
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      if (st + kPvDepth - 1 < 16) va[(st + kPvDepth - 1) % kPvDepth] = rdv(st + kPvDepth - 1);
      __builtin_amdgcn_sched_barrier(0);
      acc[st & 3] = mfma32x32x16(va[st % kPvDepth], pb[st >> 2], acc[st & 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Load schedule per wave (vector-memory loads complete in order):
  //   prologue: pt0 pt1 | tile0 pt2 | tile1 pt3
  //   at barrier k: tile k+2 (into the stage of tile k-2), pt k+4
  // Before barrier k a wave has its pieces of tile k and the table entries
  // of tile k+2 (read right after the barrier); only tile k+1 and pt k+3
  // may still be in flight.  The stage of tile k-2 is free at barrier k:
  // its last reader, the lag group's P V of tile k-2, ran before barrier k.
  // Tiles past the end re-read the last key, so every barrier sees the same
  // loads in flight.
  auto sync_tile = [&](int k) {
    wait_vmcnt<2 * kPPW + 1>();
    tile_barrier();
    issue_tile(k + 2);
    fetch_pt(k + 4);
  };
  fetch_pt(0);
  fetch_pt(1);
  wait_vmcnt<1>();                     // pt0 landed
  issue_tile(0);
  fetch_pt(2);
  wait_vmcnt<2 * kPPW + 1>();          // pt1 landed
  issue_tile(1);
  fetch_pt(3);

  // Both groups pass barriers 0 .. n_tiles.
  if (w < kWaves / 2) {
    for (int k = 0; k < n_tiles; ++k) {
      sync_tile(k);
      qk(k);
      softmax_pv(k);
    }
    sync_tile(n_tiles);
  } else {
    sync_tile(0);
    qk(0);
    for (int k = 1; k <= n_tiles; ++k) {
      sync_tile(k);
      softmax_pv(k - 1);
      if (k < n_tiles) qk(k);
    }
  }
  wait_vmcnt<0>();   // drain the look-ahead loads before the waves retire

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

// ---------------------------------------------------------------------------
// Work planner: one workgroup orders the (request, query tile) items by the
// number of key tiles they visit, longest first (a counting sort over
// kPlanBuckets buckets), so that the attention workgroups dispatched first
// are the longest ones and the short ones fill in at the end.  The order of
// items within a bucket is whatever the LDS atomics give; every item is
// computed the same way wherever it lands, so results do not depend on it.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = kPlanThreads;

struct PlanParams {
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  int32_t batch;
  int32_t n_qtiles;
  int32_t bq;
  int32_t shift;          // bucket = key tiles >> shift
  int32_t* count;
  int32_t* list;
};

__device__ __forceinline__ int plan_bucket(const PlanParams& p, int item) {
  const int r = item / p.n_qtiles;
  const int qt = item - r * p.n_qtiles;
  const int E = p.extend_lens[r];
  const int q0 = qt * p.bq;
  if (q0 >= E) return -1;                    // no query rows: not an item
  const int64_t kv_end = (int64_t)p.prefix_lens[r] + min(q0 + p.bq, E);
  const int64_t tiles = (kv_end + kBN - 1) / kBN;
  return (int)max((int64_t)0, min((int64_t)(kPlanBuckets - 1), tiles >> p.shift));
}

__global__ void __launch_bounds__(kPlanThreads) extend_plan_kernel(PlanParams p) {
  __shared__ int hist[kPlanBuckets];
  __shared__ int scan[kPlanBuckets];
  const int tid = threadIdx.x;
  const int total = p.batch * p.n_qtiles;
  hist[tid] = 0;
  __syncthreads();
  for (int it = tid; it < total; it += kPlanThreads) {
    const int b = plan_bucket(p, it);
    if (b >= 0) atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  // inclusive scan over the buckets from the longest down
  const int own = hist[kPlanBuckets - 1 - tid];
  scan[tid] = own;
  __syncthreads();
  for (int d = 1; d < kPlanBuckets; d <<= 1) {
    const int add = tid >= d ? scan[tid - d] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  hist[kPlanBuckets - 1 - tid] = scan[tid] - own;   // first list position of the bucket
  if (tid == kPlanThreads - 1) p.count[0] = scan[tid];
  __syncthreads();
  for (int it = tid; it < total; it += kPlanThreads) {
    const int b = plan_bucket(p, it);
    if (b >= 0) p.list[atomicAdd(&hist[b], 1)] = it;
  }
}

int extend_rows_per_block(int ratio) { return 32 * kWaves / ratio; }

}  // namespace

size_t extend_workspace_bytes(int64_t batch, int ratio, int64_t max_extend_len) {
  const int64_t bq = extend_rows_per_block(ratio);
  const int64_t nq = (max_extend_len + bq - 1) / bq;
  return 16 + 4 * (size_t)(batch * nq);
}

hipError_t launch_paged_extend(const ExtendArgs& a) {
  ExtendParams p;
  p.out = (uint16_t*)a.out;
  p.lse = a.lse;
  p.q = (const uint16_t*)a.q;
  p.q_stride = a.q_stride;
  p.k_cache = (const char*)a.k_cache;
  p.v_cache = (const char*)a.v_cache;
  p.cache_stride_bytes = a.cache_stride * 2;
  p.num_slots = a.num_slots;
  p.page_table = a.page_table;
  p.pt_stride = a.pt_stride;
  p.page_mask = (a.page_size > 1 && (a.page_size & (a.page_size - 1)) == 0) ? a.page_size - 1 : 0;
  p.req_rows = a.req_rows;
  p.prefix_lens = a.prefix_lens;
  p.extend_lens = a.extend_lens;
  p.q_offsets = a.q_offsets;
  p.batch = a.batch;
  p.num_q_heads = a.num_q_heads;
  p.ratio = a.num_q_heads / a.num_kv_heads;
  p.scale_log2 = a.sm_scale * kLog2e;
  // a zero scale (uniform weights) becomes the smallest normal float: the
  // weights stay 2^0 = 1 to the last bit, and masked scores (-inf) still
  // give -inf instead of inf * 0
  if (p.scale_log2 == 0.f) p.scale_log2 = FLT_MIN;
  p.num_kv_heads = a.num_kv_heads;
  p.bq = extend_rows_per_block(p.ratio);
  p.n_qtiles = (a.max_extend_len + p.bq - 1) / p.bq;
  p.work_count = nullptr;
  p.work_list = nullptr;
  if (a.batch == 0 || p.n_qtiles == 0) return hipSuccess;
  // a single request's query tiles already run longest first in the natural
  // order (later tiles see more keys), so it is not planned
  if (a.workspace && a.batch > 1) {
    PlanParams pp;
    pp.prefix_lens = a.prefix_lens;
    pp.extend_lens = a.extend_lens;
    pp.batch = a.batch;
    pp.n_qtiles = p.n_qtiles;
    pp.bq = p.bq;
    int shift = 0;
    while ((((int64_t)a.max_kv_len + kBN - 1) / kBN >> shift) >= kPlanBuckets) ++shift;
    pp.shift = shift;
    pp.count = (int32_t*)a.workspace;
    pp.list = (int32_t*)((char*)a.workspace + 16);
    hipLaunchKernelGGL(extend_plan_kernel, dim3(1), dim3(kPlanThreads), 0, a.stream, pp);
    p.work_count = pp.count;
    p.work_list = pp.list;
  }
  const int64_t blocks = (int64_t)p.n_qtiles * a.batch * a.num_kv_heads;
  if (p.page_mask)
    hipLaunchKernelGGL(paged_extend_kernel<true>, dim3((unsigned)blocks), dim3(kWaves * 64), 0,
                       a.stream, p);
  else
    hipLaunchKernelGGL(paged_extend_kernel<false>, dim3((unsigned)blocks), dim3(kWaves * 64), 0,
                       a.stream, p);
  return hipGetLastError();
}

}  // namespace msgl

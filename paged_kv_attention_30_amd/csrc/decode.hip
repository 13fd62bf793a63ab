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
// gfx950 design.  A workgroup has two waves per kv head (up to 8 heads, 16
// waves) and walks one range of keys; all its waves read the same tokens, so
// every gathered K/V row (num_kv_heads x 256 B) is fetched by one workgroup
// at one time.
// * Page table: with page_size P > 1 (a power of two) the slots of a page
//   are consecutive, so only the page's first column is read and key j sits
//   in slot page_table[row, j - j % P] + j % P — the every-P-th-column view
//   of §4.6.4; P = 1 (or any other P) reads every column.  Slots are clamped
//   to the pool, so a bad entry cannot address memory outside it.
// * Work split ("balanced" mode, split_tokens = 0): the keys of the whole
//   batch, laid end to end in request order with a fixed start-up cost
//   (kSegmentCost) in front of each request's keys, are cut into ranges of
//   equal cost, one per workgroup; each working workgroup's range costs at
//   least kMinKeysPerBlock, so a small batch uses fewer workgroups.
//   The grid is at most the number of workgroups the GPU holds at once, so
//   the whole batch runs in a single round.  A range may cover the tail of one
//   request, several whole requests and the head of another; a request
//   covered by one workgroup is finished there, a request cut across
//   workgroups leaves normalised fp32 partials + lse that the merge kernel
//   combines.  One workgroup fills a compute unit: two waves per kv head
//   take alternate tiles and combine their states in LDS at the end of each
//   segment (two workgroups per unit were measured slower: the younger one
//   is served after the older and ends the kernel alone).  ("Fixed" mode,
//   split_tokens = S > 0: chunk c of request r is keys [cS, (c+1)S), one
//   workgroup per (chunk, request).)
// * Keys are processed 32 at a time.  Each lane fetches the page-table entry
//   of "its" token and issues 16-byte loads of that token's K row segment
//   into registers (a wave reads 64 contiguous bytes per token per
//   instruction); the tile's V rows go straight from HBM into the wave's LDS
//   tile (global_load_lds_dwordx4, 1 KiB per wave instruction), so they hold
//   no registers on the way.
// * S^T = K Q^T runs on the 16x16x32 bf16 MFMA: K rows go straight from the
//   loads into the A operand (row = token), q heads of the group are the
//   B operand columns (ratio <= 16, unused columns are zero).  The output
//   layout gives every lane one q head, so running max / sum / rescale are
//   per-lane scalars; the max needs two cross-lane steps.
// * O^T = V^T P^T also runs on MFMA: P^T is the QK output repacked to bf16
//   in place (its C layout is exactly the B layout of the next MFMA), and the
//   V^T operand comes from the key-major V tile through the transposing LDS
//   read (ds_read_b64_tr_b16).
// * Reduction order depends only on logical key positions and lengths, so
//   results are bit-identical under any slot permutation and for any
//   page_size.

#include <float.h>

#include "common.hpp"
#include "internal.hpp"

namespace msgl {

namespace {

constexpr int kTile = 32;          // keys per inner iteration
constexpr int kMinKeysPerBlock = 128;   // balanced mode: fewest keys a working workgroup takes
// balanced mode: a request segment costs its keys plus this start-up (q rows,
// page-table entries and the first keys arrive one after the other before
// any work overlaps them; measured ~6 us, about one 32-key tile of work)
constexpr int kSegmentCost = 32;
// LDS elements of one wave: its V tile, then a 128-byte slot for the
// per-column (max, sum) a paired wave hands over
constexpr int kWaveLds = kTile * kHeadDim + 64;

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
  uint32_t slot_max;      // num_slots - 1 (slots are clamped to the pool)
  int32_t page_mask;      // page_size - 1 for a power-of-two page_size, else 0
  int32_t batch;
  int32_t num_q_heads;
  int32_t ratio;
  int32_t split_tokens;   // fixed mode chunk size (> 0), 0 in balanced mode
  int32_t max_splits;     // fixed mode: chunks per request in the grid
  float scale_log2;       // sm_scale * log2(e)
  float* part_out;        // [slots, Hq, 128]
  float* part_lse;        // [slots, Hq]
  int32_t* meta;          // balanced mode: per request (first, last) workgroup
  // Store fused into the launch (k_store null: none).  Row r of k_new /
  // v_new is request r's newest token, stored at slot out_loc[r], which is
  // key seq_lens[r] - 1 of the request; the one wave per kv head that reads
  // that key stores it first (see attend_segment), so no workgroup reads a
  // slot another one writes.
  char* k_store;
  char* v_store;
  const char* k_new;
  const char* v_new;
  int64_t new_stride_bytes;
  const void* out_loc;
  int32_t out_loc_i64;
};

// The lane index, hidden from loop-invariant code motion: per-lane addresses
// of the rarely taken paths below are then formed where they are used
// instead of being hoisted out of the segment loop into registers (and
// spilled, as the tile loop needs all of them).
__device__ __forceinline__ int lane_here() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

// The fused store, one kv head's slice of request r's new row: lanes 0-15
// carry the 256 bytes of K, lanes 16-31 those of V, one 16-byte unit each.
// new_slice loads them; store_slice writes them to slot out_loc[r].
__device__ __forceinline__ u32x4 new_slice(const DecodeParams& p, int r, int g) {
  const int lane = lane_here();
  u32x4 v = {0u, 0u, 0u, 0u};
  if (lane < 32)
    v = ld16((lane < 16 ? p.k_new : p.v_new) + (int64_t)r * p.new_stride_bytes +
             (int64_t)g * kHeadDim * 2 + 16 * (lane & 15));
  return v;
}

__device__ __forceinline__ void store_slice(const DecodeParams& p, int r, int g, u32x4 v) {
  const int lane = lane_here();
  const int64_t slot = p.out_loc_i64 ? reinterpret_cast<const int64_t*>(p.out_loc)[r]
                                     : (int64_t)reinterpret_cast<const int32_t*>(p.out_loc)[r];
  if (lane < 32)
    st16((lane < 16 ? p.k_store : p.v_store) + slot * p.cache_stride_bytes +
             (int64_t)g * kHeadDim * 2 + 16 * (lane & 15),
         v);
}

// Slot of key `key` of a request whose table row starts at `pt`: read from
// the column of the key's page start, offset inside the page, clamped to the
// pool (negative entries clamp to the last slot).
__device__ __forceinline__ int slot_of(const DecodeParams& p, const int32_t* pt, int key) {
  const int off = key & p.page_mask;
  return (int)min((uint32_t)(pt[key - off] + off), p.slot_max);
}

// A wave's V tile: key-major rows of 128 dims (256 bytes); the 8-byte group
// g (dims 4g .. 4g+3) of key t sits at group position g ^ 4 (t & 7).  A
// transposed read takes 8 keys (t & 7 distinct) x 4 consecutive groups per
// 32 lanes; the XOR spreads them over all 32 group positions of a 256-byte
// bank row, so the read is free of bank conflicts, and it keeps together the
// group pairs a 16-byte direct load writes.

__device__ __forceinline__ int shfl_up_i(int v, int d) {
  const int lane = __lane_id();
  const int src = lane >= d ? lane - d : lane;
  return __builtin_amdgcn_ds_bpermute(src << 2, v);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = shfl_up_i(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

// A value every lane holds identically, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)(v & 0xffffffff));
  const int hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((int64_t)hi << 32) | (uint32_t)lo;
}

// Output of an empty request: zeros and lse = -inf.
__device__ __forceinline__ void write_empty(const DecodeParams& p, int r, int g) {
  const int lane = lane_here();
  const int c = lane & 15, j = lane >> 4;
  if (c >= p.ratio) return;
  const int h = g * p.ratio + c;
  uint16_t* o = p.out + ((int64_t)r * p.num_q_heads + h) * kHeadDim;
  const u32x2 z = {0u, 0u};
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<u32x2*>(o + 16 * mb + 4 * j) = z;
  if (p.lse && j == 0) p.lse[(int64_t)r * p.num_q_heads + h] = -INFINITY;
}

// One wave: attention of request r's q heads of kv head g over keys
// [t0, t1) (t0 < t1).  Writes the final bf16 output + lse when `whole`,
// else the normalised fp32 partial + lse at partial row `slot`.
// `vt` is the wave's V tile (32 keys x 128 dims), `qs` its group's q rows
// (ratio x 128).  With NPAR = 2 two waves share the segment: wave `par`
// takes the tiles t0 + 32 (2i + par); at the end the parity-1 wave leaves
// its state in its V tile (`pvt` is that tile, seen from the pair) and the
// parity-0 wave folds it in and writes the result.  Every wave of the
// workgroup must call this for the same segments (it holds workgroup
// barriers).
// `row` is the request's page-table row.  With the store fused, `last_key`
// is the request's newest key when this segment holds it (else -1): the
// wave whose tiles include that key stores the head's slice of the new row
// at the start of the segment and reads it back from the pool like every
// other key (a wave sees its own stores once they have completed), so no
// other wave or workgroup touches that slot.
template <int NPAR>
__device__ __forceinline__ void attend_segment(const DecodeParams& p, uint16_t* vt,
                                               uint16_t* qs, uint16_t* pvt, int par, int r,
                                               int g, int t0, int t1, bool whole,
                                               int64_t slot, int last_key, int row) {
  const int lane = __lane_id();
  const int c = lane & 15;      // q-head column / token row inside the MFMA
  const int j = lane >> 4;      // k-slot group
  const int R = p.ratio;

  const int32_t* pt = p.page_table + (int64_t)row * p.pt_stride;

  // q rows of the group (ratio x 128 bf16) are loaded now and parked in LDS
  // once the first page-table entries are in flight, so the two memory
  // round trips of a segment start overlap.
  const uint16_t* qg = p.q + (int64_t)r * p.q_stride + (int64_t)g * R * kHeadDim;
  u32x4 qv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = lane + 64 * k;
    if (u < R * 16) qv[k] = ld16(qg + 8 * u);
  }
  // the wave whose tiles hold the newest key stores it (waves take tiles
  // t0 + 32 (NPAR i + par)).  That key is the last of the segment, so its
  // tile is the segment's last one: the other wave's tiles all lie below it
  // and never touch the slot, not even through the lanes a tail tile clamps
  // to its last key.
  const bool stores_new = last_key >= t0 && ((last_key - t0) / kTile) % NPAR == par;
  u32x4 nv;
  if (stores_new) nv = new_slice(p, r, g);
  // B operand of S^T = K Q^T: column c, k-slot (j, e) of step kk <-> head dim
  // 32*kk + 8*j + e.  Columns c >= ratio read a real row again; their output
  // columns are never used and MFMA columns do not mix.
  const uint16_t* qcol = qs + (c % R) * kHeadDim + 8 * j;

  const int64_t cs = p.cache_stride_bytes;
  const char* kbase = p.k_cache + (int64_t)g * kHeadDim * 2 + (8 * j) * 2;
  // V direct loads: this lane's key within each 4-key load (ld_key), the
  // byte address of the lane holding that key's slot, and the byte offset of
  // the 16-byte unit it fetches for load 0 (its physical unit lane % 16 holds
  // logical unit (lane % 16) ^ 2 (key & 7))
  const int ld_key = lane >> 4;
  const int bp_addr = 4 * ld_key;
  const int uoff = 16 * ((lane & 15) ^ (2 * ld_key));
  // transposed reads: lane 4k + q of 16-lane group j addresses key
  // tr_t = 4j + k, group q of the dim block (the byte offset of dim block mb
  // is 32 mb ^ tr_sw within the row; the hi keys sit 16 rows = 4 KiB on)
  const int tr_t = 4 * j + ((lane & 15) >> 2);
  const int tr_base = 256 * tr_t + 8 * (lane & 3);
  const int tr_sw = 32 * (tr_t & 7);
  const char* vbase = p.v_cache + (int64_t)g * kHeadDim * 2;

  f32x4 acc[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max, log2 units
  float l_run = 0.f;         // this lane's share of the running sum

  // The page-table entries of tile i+1 are fetched while tile i computes,
  // so each iteration waits on one memory latency (its K/V), not two.
  constexpr int kStep = kTile * NPAR;
  const int tfirst = t0 + kTile * par;
  int na = slot_of(p, pt, min(tfirst + c, t1 - 1));
  int nb = slot_of(p, pt, min(tfirst + 16 + c, t1 - 1));
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = lane + 64 * k;
    if (u < R * 16) *reinterpret_cast<u32x4*>(qs + 8 * u) = qv[k];
  }
  if (stores_new) store_slice(p, r, g, nv);
  __builtin_amdgcn_wave_barrier();

  for (int tb = tfirst; tb < t1; tb += kStep) {
    // V tile: straight from HBM into this wave's LDS tile, key-major rows of
    // 256 bytes.  Load i fills rows 4i .. 4i+3 (lane l: key 4i + l/16,
    // physical 16-byte unit l % 16, holding logical unit (l % 16) ^ 2(key & 7),
    // the tile layout above).  A lane takes the slot of its key from the lane that holds
    // it (keys c in na, 16 + c in nb).  The previous tile's V reads finished
    // before its P V MFMAs, and every wave reads only its own tile.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    // the tile holding the newest key of a fused store: its row was stored
    // by this wave at the start of the segment; wait until it has landed
    // (the table entries of this tile, the only other loads in flight, are
    // needed now anyway)
    if ((unsigned)(last_key - tb) < (unsigned)kTile) wait_vmcnt<0>();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // key 4i + ld_key: its slot sits in lane 4 (i % 4) + ld_key, and its
      // swizzle 2 (key & 7) = 2 ld_key + 8 (i % 2) only flips unit bit 3
      const int sl = __builtin_amdgcn_ds_bpermute(bp_addr + 16 * (i & 3), i < 4 ? na : nb);
      const int uo = uoff ^ (128 * (i & 1));
      dma16(vbase + (int64_t)sl * cs + uo, vt + 512 * i);
    }
    // K rows of keys c and 16 + c go to registers: the A operand of S^T = K Q^T
    const char* ra = kbase + (int64_t)na * cs;
    const char* rb = kbase + (int64_t)nb * cs;
    u32x4 ka[4], kb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      ka[kk] = ld16(ra + 64 * kk);
      kb[kk] = ld16(rb + 64 * kk);
    }
    if (tb + kStep < t1) {
      na = slot_of(p, pt, min(tb + kStep + c, t1 - 1));
      nb = slot_of(p, pt, min(tb + kStep + 16 + c, t1 - 1));
    }

    f32x4 s_a = {0.f, 0.f, 0.f, 0.f}, s_b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 qk = *reinterpret_cast<const u32x4*>(qcol + 32 * kk);
      s_a = mfma16x16x32(ka[kk], qk, s_a);
      s_b = mfma16x16x32(kb[kk], qk, s_b);
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
    mt = max_xor32(max_xor16(mt));
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

    // the V loads are older than the K loads and the table entries after
    // them, so at most those two entries may still be in flight
    wait_vmcnt<2>();
    // V^T operand of dim block mb: lane (c, j) gets dims 16 mb + c of keys
    // 4j .. 4j+3 and 16 + 4j .. 16 + 4j + 3 from two transposed reads, the
    // k order of the P^T operand
    // (the empty asm makes the swizzle look new every tile, so the eight
    // addresses are formed here, two VALU ops each, rather than hoisted out
    // of the loop into eight registers)
    int sw = tr_sw;
    asm volatile("" : "+v"(sw));
    const char* vrow = reinterpret_cast<const char*>(vt) + tr_base;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const char* at = vrow + (sw ^ (32 * mb));
      const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(at));
      const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(at + 4096));
      const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
      acc[mb] = acc[mb] * alpha;
      acc[mb] = mfma16x16x32(a, pb, acc[mb]);
    }
  }

  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  if (NPAR > 1) {
    // the parity-1 wave's state: acc as [mb][lane] f32x4 in its V tile,
    // (max, sum) per head column in the slot after it
    f32x4* xacc = reinterpret_cast<f32x4*>(pvt);
    float* xml = reinterpret_cast<float*>(pvt + kTile * kHeadDim);
    if (par == 1) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) xacc[mb * 64 + lane] = acc[mb];
      if (j == 0) {
        xml[c] = m_run;
        xml[16 + c] = l_tot;
      }
    }
    __syncthreads();
    if (par == 0) {
      // fold in the partner's keys (it may have had no tile: max -inf)
      const float m1 = xml[c];
      const float l1 = xml[16 + c];
      const float mm = fmaxf(m_run, m1);
      const float a0 = fast_exp2(m_run - mm);
      const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb] = acc[mb] * a0 + xacc[mb * 64 + lane] * a1;
      l_tot = l_tot * a0 + l1 * a1;
      m_run = mm;
    }
    __syncthreads();
    if (par != 0) return;
  }
  if (c >= R) return;
  const int h = g * R + c;
  const float inv = 1.f / l_tot;
  const float lse_nat = (m_run + fast_log2(l_tot)) * kLn2;

  if (whole) {
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
    const int64_t idx = slot * p.num_q_heads + h;
    float* o = p.part_out + idx * kHeadDim;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      f32x4 v = acc[mb] * inv;
      *reinterpret_cast<f32x4*>(o + 16 * mb + 4 * j) = v;
    }
    if (j == 0) p.part_lse[idx] = lse_nat;
  }
}

// LDS of a workgroup with `nw` waves: the V tile (+ hand-over slot) of
// every wave, then the q rows of every kv-head group (shared by the waves of
// a pair).
__device__ __forceinline__ uint16_t* wave_vt(uint16_t* base, int w) {
  return base + (size_t)w * kWaveLds;
}
__device__ __forceinline__ uint16_t* group_qs(uint16_t* base, int nw, int gi, int ratio) {
  return base + (size_t)nw * kWaveLds + (size_t)gi * ratio * kHeadDim;
}

// Fixed chunks: workgroup (chunk, request) = blockIdx.x.
template <int KVB>
__global__ void __launch_bounds__(KVB * 64, 4)
decode_fixed_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t dyn_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
  uint16_t* vt = wave_vt(dyn_lds, w);
  uint16_t* qs = group_qs(dyn_lds, KVB, w, p.ratio);
  const int r = blockIdx.x % p.batch;
  const int split = blockIdx.x / p.batch;
  const int g = blockIdx.y * KVB + w;
  const int S = p.split_tokens;
  const int L = p.seq_lens[r];
  if (L <= 0) {
    if (split == 0) {
      write_empty(p, r, g);
      if (p.k_store) store_slice(p, r, g, new_slice(p, r, g));
    }
    return;
  }
  const int t0 = split * S;
  if (t0 >= L) return;
  // a length beyond the host bound folds its tail into the last chunk, so
  // no chunk index ever exceeds the workspace
  const int nsplit = min((L + S - 1) / S, p.max_splits);
  const int t1 = (split == p.max_splits - 1) ? L : min(t0 + S, L);
  attend_segment<1>(p, vt, qs, vt, 0, r, g, t0, t1, nsplit == 1, (int64_t)split * p.batch + r,
                    p.k_store && t1 == L ? L - 1 : -1, p.req_rows ? p.req_rows[r] : r);
}

// Balanced ranges: workgroup b of G owns flattened keys [b*T/G, (b+1)*T/G).
// NPAR = 2: two waves per kv head (one workgroup fills a compute unit).
template <int KVB, int NPAR>
__global__ void __launch_bounds__(KVB * 64 * NPAR, 4)
decode_balanced_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t dyn_lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
  const int wk = w % KVB;
  const int par = w / KVB;
  uint16_t* vt = wave_vt(dyn_lds, w);
  uint16_t* pvt = wave_vt(dyn_lds, wk + KVB * (NPAR - 1));
  uint16_t* qs = group_qs(dyn_lds, KVB * NPAR, wk, p.ratio);
  const int g = blockIdx.y * KVB + wk;
  const int b = blockIdx.x;
  const int Ggrid = gridDim.x;
  const int B = p.batch;

  // total keys of the batch (every wave computes it; it is tiny)
  // total cost of the batch: every non-empty request costs its keys plus
  // kSegmentCost, laid out as [start-up | keys] on one line
  int64_t tl = 0;
  for (int i = lane; i < B; i += 64) {
    const int Li = p.seq_lens[i];
    tl += Li > 0 ? Li + kSegmentCost : 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const int lo = __builtin_amdgcn_ds_bpermute(((lane ^ d) << 2), (int)(uint32_t)(tl & 0xffffffff));
    const int hi = __builtin_amdgcn_ds_bpermute(((lane ^ d) << 2), (int)(uint32_t)(tl >> 32));
    tl += ((int64_t)hi << 32) | (uint32_t)lo;
  }
  const int64_t T = uniform64(tl);
  // every workgroup that takes keys takes at least kMinKeysPerBlock of them
  // (a small batch cut into a few-key range per workgroup would spend its time
  // in start-up latency and in merging hundreds of parts); the rest exit
  const int64_t G = min((int64_t)Ggrid, max((int64_t)1, (T + kMinKeysPerBlock - 1) / kMinKeysPerBlock));
  // (64-bit division runs on the vector unit; move the results back to
  // scalar registers)
  const int64_t start = uniform64((G > 0 && b < G) ? (int64_t)b * T / G : T);
  const int64_t end = uniform64((G > 0 && b < G) ? (int64_t)(b + 1) * T / G : T);
  const bool last = (b == Ggrid - 1);
  if (start == end && !last) return;

  // Requests are visited in order; each step re-scans the lengths to find
  // the next request (index > r_prev) whose keys meet this workgroup's range
  // (or, for an empty request, whose position it owns), so nothing per-lane
  // stays live across a segment.
  const bool writer = (w == 0 && blockIdx.y == 0 && lane == 0);
  int r_prev = -1;
  while (true) {
    int r = -1, row = 0;
    int64_t r0 = 0, r1 = 0;
    int64_t running = 0;
    for (int base = 0; base < B; base += 64) {
      if (running > end || (running == end && !last)) break;
      const int i = base + lane;
      const int Li = i < B ? max(p.seq_lens[i], 0) : 0;
      // (the table rows come with the lengths, one round trip for both)
      const int Ri = (i < B && p.req_rows) ? p.req_rows[i] : i;
      const int Ci = Li > 0 ? Li + kSegmentCost : 0;
      const int incl = wave_incl_scan(Ci);
      const int64_t c0 = running + (incl - Ci);
      const int64_t c1 = running + incl;
      bool own;
      if (i >= B || i <= r_prev) own = false;
      else if (Li > 0) own = c1 > start && c0 + kSegmentCost < end;   // meets the keys
      else own = (c0 >= start && c0 < end) || (last && c0 == T);
      const uint64_t mask = __ballot(own);
      if (mask) {
        const int bit = __builtin_ctzll(mask);
        r = base + bit;
        r1 = running + __builtin_amdgcn_readlane(incl, bit);
        const int Lr = __builtin_amdgcn_readlane(Li, bit);
        row = __builtin_amdgcn_readlane(Ri, bit);
        r0 = r1 - Lr;            // position of the request's first key (after its start-up)
        break;
      }
      running += __builtin_amdgcn_readlane(incl, 63);
    }
    if (r < 0) break;
    r_prev = r;
    if (r1 == r0) {             // an empty request (its new row is still stored)
      if (par == 0) {
        write_empty(p, r, g);
        if (p.k_store) store_slice(p, r, g, new_slice(p, r, g));
      }
      if (writer) {
        p.meta[2 * r] = -1;
        p.meta[2 * r + 1] = -1;
      }
      continue;
    }
    const int s0 = (int)(max(start, r0) - r0);
    const int s1 = (int)(min(end, r1) - r0);
    const bool whole = r0 >= start && r1 <= end;
    attend_segment<NPAR>(p, vt, qs, pvt, par, r, g, s0, s1, whole, (int64_t)b + r,
                         p.k_store && r1 <= end ? (int)(r1 - r0) - 1 : -1, row);
    if (writer) {
      // workgroups holding the first and the last key of request r
      const int64_t bf = ((r0 + 1) * G - 1) / T;
      const int64_t bl = (r1 * G - 1) / T;
      p.meta[2 * r] = whole ? -1 : (int32_t)bf;
      p.meta[2 * r + 1] = whole ? -1 : (int32_t)bl;
    }
  }
}

size_t decode_lds_bytes(int kvb, int npar, int ratio) {
  return ((size_t)kvb * npar * kWaveLds + (size_t)kvb * ratio * kHeadDim) * sizeof(uint16_t);
}

// LDS a workgroup may hold on gfx950
constexpr size_t kLdsLimit = 160 * 1024;

// Workgroups of the balanced kernel resident per compute unit (cached per
// device and ratio).
template <int KVB, int NPAR>
int resident_blocks_per_cu(int ratio) {
  static int cached[64][5] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const int ri = ratio == 1 ? 0 : ratio == 2 ? 1 : ratio == 4 ? 2 : ratio == 8 ? 3 : 4;
  if (cached[dev][ri] > 0) return cached[dev][ri];
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_balanced_kernel<KVB, NPAR>,
                                                   KVB * 64 * NPAR,
                                                   decode_lds_bytes(KVB, NPAR, ratio)) != hipSuccess ||
      n <= 0)
    n = 1;
  cached[dev][ri] = n;
  return n;
}

// Balanced mode: workgroups along x (all resident at once, at most
// kMaxDecodeBlocks).
template <int KVB, int NPAR>
int64_t balanced_grid_x(int num_kv_heads, int ratio, int compute_units) {
  const int64_t gy = num_kv_heads / KVB;
  int64_t g = (int64_t)compute_units * resident_blocks_per_cu<KVB, NPAR>(ratio) / gy;
  if (g < 1) g = 1;
  if (g > kMaxDecodeBlocks) g = kMaxDecodeBlocks;
  return g;
}

template <int KVB>
int64_t balanced_grid_kvb(int num_kv_heads, int ratio, int compute_units) {
  if (decode_lds_bytes(KVB, 2, ratio) <= kLdsLimit)
    return balanced_grid_x<KVB, 2>(num_kv_heads, ratio, compute_units);
  return balanced_grid_x<KVB, 1>(num_kv_heads, ratio, compute_units);
}

template <int KVB, int NPAR>
hipError_t launch_balanced(const DecodeArgs& a, const DecodeParams& p) {
  const unsigned gy = (unsigned)(a.num_kv_heads / KVB);
  const int64_t g = balanced_grid_x<KVB, NPAR>(a.num_kv_heads, p.ratio, a.balanced_blocks);
  hipLaunchKernelGGL((decode_balanced_kernel<KVB, NPAR>), dim3((unsigned)g, gy),
                     dim3(KVB * 64 * NPAR), decode_lds_bytes(KVB, NPAR, p.ratio), a.stream, p);
  return hipGetLastError();
}

template <int KVB>
hipError_t launch_kvb(const DecodeArgs& a, const DecodeParams& p) {
  const unsigned gy = (unsigned)(a.num_kv_heads / KVB);
  const size_t lds = decode_lds_bytes(KVB, 1, p.ratio);
  if (a.balanced_blocks > 0) {
    // two waves per kv head when their LDS fits
    if (decode_lds_bytes(KVB, 2, p.ratio) <= kLdsLimit) return launch_balanced<KVB, 2>(a, p);
    return launch_balanced<KVB, 1>(a, p);
  } else {
    dim3 grid((unsigned)((int64_t)a.max_splits * a.batch), gy);
    hipLaunchKernelGGL((decode_fixed_kernel<KVB>), grid, dim3(KVB * 64), lds, a.stream, p);
  }
  return hipGetLastError();
}

}  // namespace

int decode_kv_heads_per_block(int num_kv_heads) {
  return num_kv_heads % 8 == 0 ? 8 : num_kv_heads % 4 == 0 ? 4 : num_kv_heads % 2 == 0 ? 2 : 1;
}

int64_t decode_balanced_grid(int num_kv_heads, int ratio, int compute_units) {
  switch (decode_kv_heads_per_block(num_kv_heads)) {
    case 8: return balanced_grid_kvb<8>(num_kv_heads, ratio, compute_units);
    case 4: return balanced_grid_kvb<4>(num_kv_heads, ratio, compute_units);
    case 2: return balanced_grid_kvb<2>(num_kv_heads, ratio, compute_units);
    default: return balanced_grid_kvb<1>(num_kv_heads, ratio, compute_units);
  }
}

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
  p.slot_max = (uint32_t)min(a.num_slots - 1, (int64_t)INT32_MAX);
  p.page_mask = (a.page_size > 1 && (a.page_size & (a.page_size - 1)) == 0) ? a.page_size - 1 : 0;
  p.batch = a.batch;
  p.num_q_heads = a.num_q_heads;
  p.ratio = a.num_q_heads / a.num_kv_heads;
  p.split_tokens = a.split_tokens;
  p.max_splits = a.max_splits;
  p.scale_log2 = a.sm_scale * kLog2e;
  p.part_out = a.part_out;
  p.part_lse = a.part_lse;
  p.meta = a.meta;
  p.k_store = (char*)a.k_store;
  p.v_store = (char*)a.v_store;
  p.k_new = (const char*)a.k_new;
  p.v_new = (const char*)a.v_new;
  p.new_stride_bytes = a.new_stride * 2;
  p.out_loc = a.out_loc;
  p.out_loc_i64 = a.out_loc_is_i64 ? 1 : 0;

  hipError_t err;
  switch (decode_kv_heads_per_block(a.num_kv_heads)) {
    case 8: err = launch_kvb<8>(a, p); break;
    case 4: err = launch_kvb<4>(a, p); break;
    case 2: err = launch_kvb<2>(a, p); break;
    default: err = launch_kvb<1>(a, p); break;
  }
  if (err != hipSuccess) return err;
  if (a.balanced_blocks <= 0 && a.max_splits <= 1) return hipSuccess;

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
  m.seq_lens = a.balanced_blocks > 0 ? nullptr : a.seq_lens;
  m.split_tokens = a.split_tokens;
  m.meta = a.balanced_blocks > 0 ? a.meta : nullptr;
  m.stream = a.stream;
  return launch_merge(m);
}

}  // namespace msgl

// Graph-replayed decode step: store_kv + paged_decode captured once per batch
// size of a ladder, replayed on fixed-address buffers.
//
// "Mini-SGLang complete analysis" §4.6.6 (CUDA graphs and attention): the
// backend keeps persistent device buffers (seq_lens, positions, cu_seqlens,
// page table) that every captured batch points at; at run time the live data
// are written into them in place and the graph for the batch size is
// replayed.  §5.3: one graph per size of [1, 2, 4, 8, 16, 24, ..., max_bs],
// captured from the largest down; batches are padded up to the next captured
// size with a dummy request whose page points at one extra sentinel page, so
// any padding is safe.  §4.6.5: for decode the per-request query count is 1,
// so the query offsets are a constant arange (here: implicit in the decode
// call's layout).
//
// Here each graph holds one decode step: the padding kernel, then store_kv
// + decode (+ merge), either as the two library calls or, when the caller's
// allocator guarantees that a request's new slot is its own newest key and
// no other request's key (the pages' allocator hands out a fresh slot per
// new token), as the one store + decode launch the attention layer's forward
// amounts to (§4.6.7).  The padding kernel turns rows [bs, bucket) into the
// dummy request: seq_len 1, the caller's dummy page-table row, out_loc = the
// sentinel slot, zero q / k / v rows, so every padded row writes the same
// zero row into the sentinel slot and attends to it alone.  Its row range
// changes with the live batch size, so before each replay its arguments are
// set on the instantiated graph (hipGraphExecKernelNodeSetParams, a host-side
// update): a step is one graph launch.

#include <algorithm>
#include <new>
#include <vector>

#include "msgl.h"
#include "internal.hpp"

struct msgl_decode_graph {
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  int64_t num_slots = 0;
  int64_t cache_row_stride = 0;
  const int32_t* page_table = nullptr;
  int64_t pt_stride = 0;
  int32_t hq = 0, hkv = 0, page_size = 1, max_bs = 0, max_seq_len = 0;
  float sm_scale = 0.f;
  int32_t dummy_row = 0, sentinel_slot = 0;
  int32_t fused = 0;                    // capture msgl_store_kv_paged_decode
  char* q = nullptr;
  char* k_new = nullptr;
  char* v_new = nullptr;
  char* out = nullptr;
  float* lse = nullptr;
  int32_t* seq_lens = nullptr;
  int32_t* req_rows = nullptr;
  int32_t* out_loc = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::vector<int32_t> ladder;          // ascending
  std::vector<hipGraph_t> graphs;       // per ladder entry
  std::vector<hipGraphExec_t> execs;
  std::vector<hipGraphNode_t> pad_nodes; // the padding kernel of each graph
};

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// rows [r0, r1) of the fixed buffers become the dummy request (workgroup i
// takes row r0 + i; r0 == r1: nothing)
__global__ void __launch_bounds__(256) pad_rows_kernel(char* q, char* k_new, char* v_new,
                                                       int32_t* seq_lens, int32_t* req_rows,
                                                       int32_t* out_loc, int32_t r0, int32_t r1,
                                                       int32_t hq, int32_t hkv, int32_t dummy_row,
                                                       int32_t sentinel) {
  const int32_t r = r0 + (int32_t)blockIdx.x;
  if (r >= r1) return;
  const int64_t qb = (int64_t)hq * 128 * 2;     // bytes of one q row
  const int64_t kb = (int64_t)hkv * 128 * 2;    // bytes of one k / v row
  const uint4 z = {0u, 0u, 0u, 0u};
  for (int64_t o = 16 * (int64_t)threadIdx.x; o < qb; o += 16 * blockDim.x)
    *reinterpret_cast<uint4*>(q + r * qb + o) = z;
  for (int64_t o = 16 * (int64_t)threadIdx.x; o < kb; o += 16 * blockDim.x) {
    *reinterpret_cast<uint4*>(k_new + r * kb + o) = z;
    *reinterpret_cast<uint4*>(v_new + r * kb + o) = z;
  }
  if (threadIdx.x == 0) {
    seq_lens[r] = 1;
    req_rows[r] = dummy_row;
    out_loc[r] = sentinel;
  }
}

// Launch of the padding kernel for rows [r0, r1) (at least one workgroup,
// so the node exists in every captured graph), or its node parameters.
struct PadLaunch {
  void* args[12];
  char* q;
  char* k_new;
  char* v_new;
  int32_t* seq_lens;
  int32_t* req_rows;
  int32_t* out_loc;
  int32_t r0, r1, hq, hkv, dummy_row, sentinel;
  PadLaunch(const msgl_decode_graph* g, int32_t a, int32_t b)
      : q(g->q), k_new(g->k_new), v_new(g->v_new), seq_lens(g->seq_lens),
        req_rows(g->req_rows), out_loc(g->out_loc), r0(a), r1(b), hq(g->hq), hkv(g->hkv),
        dummy_row(g->dummy_row), sentinel(g->sentinel_slot) {
    void* a12[12] = {&q, &k_new, &v_new, &seq_lens, &req_rows, &out_loc, &r0, &r1, &hq, &hkv,
                     &dummy_row, &sentinel};
    for (int i = 0; i < 12; ++i) args[i] = a12[i];
  }
  unsigned blocks() const { return (unsigned)std::max(1, r1 - r0); }
};

hipError_t pad(const msgl_decode_graph* g, int32_t r0, int32_t r1, hipStream_t s) {
  PadLaunch l(g, r0, r1);
  hipLaunchKernelGGL(pad_rows_kernel, dim3(l.blocks()), dim3(256), 0, s, l.q, l.k_new, l.v_new,
                     l.seq_lens, l.req_rows, l.out_loc, l.r0, l.r1, l.hq, l.hkv, l.dummy_row,
                     l.sentinel);
  return hipGetLastError();
}

// the step for a batch of bs rows (after the padding)
int step(const msgl_decode_graph* g, int32_t bs, hipStream_t s) {
  if (g->fused)
    return msgl_store_kv_paged_decode(
        g->out, g->lse, g->q, (int64_t)g->hq * 128, g->k_cache, g->v_cache, g->num_slots,
        g->cache_row_stride, g->k_new, g->v_new, (int64_t)g->hkv * 128, g->out_loc,
        MSGL_INDEX_I32, g->page_table, g->pt_stride, g->req_rows, g->seq_lens, bs, g->hq, g->hkv,
        128, g->page_size, g->max_seq_len, g->sm_scale, 0, g->ws, g->ws_bytes, s);
  int st = msgl_store_kv(g->k_cache, g->v_cache, g->num_slots, g->cache_row_stride, g->k_new,
                         g->v_new, (int64_t)g->hkv * 128, g->out_loc, MSGL_INDEX_I32, bs, g->hkv,
                         128, MSGL_DTYPE_BF16, s);
  if (st != MSGL_OK) return st;
  return msgl_paged_decode(g->out, g->lse, g->q, (int64_t)g->hq * 128, g->k_cache, g->v_cache,
                           g->num_slots, g->cache_row_stride, g->page_table, g->pt_stride,
                           g->req_rows, g->seq_lens, bs, g->hq, g->hkv, 128, g->page_size,
                           g->max_seq_len, g->sm_scale, 0, g->ws, g->ws_bytes, s);
}

// The padding kernel's node in a captured graph (null if not found).
hipGraphNode_t find_pad_node(hipGraph_t gr) {
  size_t n = 0;
  if (hipGraphGetNodes(gr, nullptr, &n) != hipSuccess || n == 0) return nullptr;
  std::vector<hipGraphNode_t> nodes(n);
  if (hipGraphGetNodes(gr, nodes.data(), &n) != hipSuccess) return nullptr;
  for (hipGraphNode_t nd : nodes) {
    hipGraphNodeType t;
    if (hipGraphNodeGetType(nd, &t) != hipSuccess || t != hipGraphNodeTypeKernel) continue;
    hipKernelNodeParams kp;
    if (hipGraphKernelNodeGetParams(nd, &kp) == hipSuccess &&
        kp.func == reinterpret_cast<const void*>(pad_rows_kernel))
      return nd;
  }
  return nullptr;
}

void release(msgl_decode_graph* g) {
  for (hipGraphExec_t e : g->execs)
    if (e) (void)hipGraphExecDestroy(e);
  for (hipGraph_t gr : g->graphs)
    if (gr) (void)hipGraphDestroy(gr);
  delete g;
}

}  // namespace

extern "C" {

int msgl_decode_graph_layout(int32_t max_bs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_seq_len, size_t* offsets) {
  if (!offsets || max_bs < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim != 128 ||
      max_seq_len < 1)
    return MSGL_ERR_SHAPE;
  const size_t B = (size_t)max_bs;
  const size_t sizes[9] = {
      B * num_q_heads * 128 * 2,            // q
      B * num_kv_heads * 128 * 2,           // k_new
      B * num_kv_heads * 128 * 2,           // v_new
      B * num_q_heads * 128 * 2,            // out
      B * num_q_heads * 4,                  // lse
      B * 4,                                // seq_lens
      B * 4,                                // req_rows
      B * 4,                                // out_loc
      msgl_paged_decode_workspace_size(max_bs, num_q_heads, num_kv_heads, 128, max_seq_len, 0,
                                        nullptr)};
  size_t off = 0;
  for (int i = 0; i < 9; ++i) {
    offsets[i] = off;
    off += align256(sizes[i]);
  }
  offsets[9] = off;
  return MSGL_OK;
}

int msgl_decode_graph_create(void* k_cache, void* v_cache, int64_t num_slots,
                             int64_t cache_row_stride, const int32_t* page_table,
                             int64_t page_table_stride, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t max_bs,
                             int32_t max_seq_len, float sm_scale, int32_t dummy_row,
                             int32_t sentinel_slot, int32_t fused_store, void* buffer,
                             size_t buffer_bytes, msgl_decode_graph** out) {
  if (!out) return MSGL_ERR_NULL;
  *out = nullptr;
  if (!k_cache || !v_cache || !page_table || !buffer) return MSGL_ERR_NULL;
  size_t off[10];
  int st = msgl_decode_graph_layout(max_bs, num_q_heads, num_kv_heads, head_dim, max_seq_len, off);
  if (st != MSGL_OK) return st;
  if (buffer_bytes < off[9]) return MSGL_ERR_WORKSPACE;
  if (((uintptr_t)buffer & 255) != 0) return MSGL_ERR_ALIGN;
  if (dummy_row < 0 || sentinel_slot < 0 || sentinel_slot >= num_slots) return MSGL_ERR_SHAPE;

  msgl_decode_graph* g = new (std::nothrow) msgl_decode_graph();
  if (!g) return MSGL_ERR_LAUNCH;
  g->k_cache = k_cache;
  g->v_cache = v_cache;
  g->num_slots = num_slots;
  g->cache_row_stride = cache_row_stride;
  g->page_table = page_table;
  g->pt_stride = page_table_stride;
  g->hq = num_q_heads;
  g->hkv = num_kv_heads;
  g->page_size = page_size;
  g->max_bs = max_bs;
  g->max_seq_len = max_seq_len;
  g->sm_scale = sm_scale;
  g->dummy_row = dummy_row;
  g->sentinel_slot = sentinel_slot;
  g->fused = fused_store ? 1 : 0;
  char* b = (char*)buffer;
  g->q = b + off[0];
  g->k_new = b + off[1];
  g->v_new = b + off[2];
  g->out = b + off[3];
  g->lse = (float*)(b + off[4]);
  g->seq_lens = (int32_t*)(b + off[5]);
  g->req_rows = (int32_t*)(b + off[6]);
  g->out_loc = (int32_t*)(b + off[7]);
  g->ws = off[9] > off[8] ? (void*)(b + off[8]) : nullptr;
  g->ws_bytes = off[9] - off[8];
  for (int32_t s : {1, 2, 4})
    if (s < max_bs) g->ladder.push_back(s);
  for (int32_t s = 8; s < max_bs; s += 8) g->ladder.push_back(s);
  g->ladder.push_back(max_bs);

  // capture on a private stream (default priority), largest batch first
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
    release(g);
    return MSGL_ERR_LAUNCH;
  }
  st = MSGL_OK;
  g->graphs.assign(g->ladder.size(), nullptr);
  g->execs.assign(g->ladder.size(), nullptr);
  g->pad_nodes.assign(g->ladder.size(), nullptr);
  if (pad(g, 0, max_bs, s) != hipSuccess) st = MSGL_ERR_LAUNCH;
  for (int i = (int)g->ladder.size() - 1; i >= 0 && st == MSGL_OK; --i) {
    const int32_t bs = g->ladder[i];
    st = step(g, bs, s);              // eager warm-up (also validates every argument)
    if (st != MSGL_OK) break;
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      st = MSGL_ERR_LAUNCH;
      break;
    }
    // the padding node (captured with an empty row range; set per replay)
    const hipError_t pe = pad(g, bs, bs, s);
    const int cst = pe == hipSuccess ? step(g, bs, s) : MSGL_ERR_LAUNCH;
    hipGraph_t gr = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &gr);
    g->graphs[i] = gr;
    if (cst != MSGL_OK || e != hipSuccess || !gr) {
      st = cst != MSGL_OK ? cst : MSGL_ERR_LAUNCH;
      break;
    }
    g->pad_nodes[i] = find_pad_node(gr);
    if (!g->pad_nodes[i] ||
        hipGraphInstantiate(&g->execs[i], gr, nullptr, nullptr, 0) != hipSuccess) {
      st = MSGL_ERR_LAUNCH;
      break;
    }
  }
  if (hipStreamSynchronize(s) != hipSuccess && st == MSGL_OK) st = MSGL_ERR_LAUNCH;
  (void)hipStreamDestroy(s);
  if (st != MSGL_OK) {
    release(g);
    return st;
  }
  *out = g;
  return MSGL_OK;
}

int msgl_decode_graph_run(msgl_decode_graph* g, int32_t batch, hipStream_t stream) {
  if (!g) return MSGL_ERR_NULL;
  if (batch < 0 || batch > g->max_bs) return MSGL_ERR_SHAPE;
  if (batch == 0) return MSGL_OK;
  const size_t i = std::lower_bound(g->ladder.begin(), g->ladder.end(), batch) - g->ladder.begin();
  PadLaunch l(g, batch, g->ladder[i]);
  hipKernelNodeParams kp = {};
  kp.func = reinterpret_cast<void*>(pad_rows_kernel);
  kp.gridDim = dim3(l.blocks());
  kp.blockDim = dim3(256);
  kp.sharedMemBytes = 0;
  kp.kernelParams = l.args;
  kp.extra = nullptr;
  if (hipGraphExecKernelNodeSetParams(g->execs[i], g->pad_nodes[i], &kp) != hipSuccess)
    return MSGL_ERR_LAUNCH;
  if (hipGraphLaunch(g->execs[i], stream) != hipSuccess) return MSGL_ERR_LAUNCH;
  return MSGL_OK;
}

int32_t msgl_decode_graph_bucket(const msgl_decode_graph* g, int32_t batch) {
  if (!g || batch < 1 || batch > g->max_bs) return -1;
  return *std::lower_bound(g->ladder.begin(), g->ladder.end(), batch);
}

void msgl_decode_graph_destroy(msgl_decode_graph* g) {
  if (g) release(g);
}

}  // extern "C"

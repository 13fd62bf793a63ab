// Host-side argument bundles and kernel launchers (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msgl {

template <int W> struct VecOf;
template <> struct VecOf<16> { typedef uint4 type; };
template <> struct VecOf<8> { typedef uint2 type; };
template <> struct VecOf<4> { typedef uint32_t type; };
template <> struct VecOf<2> { typedef uint16_t type; };

struct StoreArgs {
  void* k_cache;
  void* v_cache;
  int64_t cache_stride_bytes;
  const void* k_new;
  const void* v_new;
  int64_t new_stride_bytes;
  const void* out_loc;
  bool index_is_i64;
  int64_t n;
  int64_t row_bytes;
  int unit_bytes;  // 16, 8, 4 or 2: widest unit every address is aligned to
  hipStream_t stream;
};

struct GatherArgs {
  void* out;
  int64_t out_stride_bytes;
  const void* weights;
  int64_t w_stride_bytes;
  int64_t rows;            // table rows this shard holds
  int64_t vocab_start;     // vocabulary id of the shard's row 0
  const void* ids;
  bool index_is_i64;
  int64_t n;
  int64_t row_bytes;
  int unit_bytes;          // 16, 8, 4 or 2: widest unit every address is aligned to
  hipStream_t stream;
};

struct PrologueArgs {
  void* q_out;             // bf16 [n, Hq, 128], row stride q_out_stride elements
  int64_t q_out_stride;
  void* k_cache;           // bf16 pool planes [slots, Hkv, 128], row stride cache_stride
  void* v_cache;
  int64_t cache_stride;
  const void* qkv;         // bf16 [n, (Hq + 2 Hkv) * 128], row stride qkv_stride
  int64_t qkv_stride;
  const void* q_norm_w;    // bf16 [128] or null (no q norm)
  const void* k_norm_w;    // bf16 [128] or null (no k norm)
  float eps;
  const int32_t* positions;
  const float* cache;      // fp32 [max_position, 128]: cos | sin
  int64_t max_position;
  const void* out_loc;
  bool index_is_i64;
  int64_t n;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  hipStream_t stream;
};

struct DecodeArgs {
  void* out;               // bf16 [B, Hq, 128]
  float* lse;              // fp32 [B, Hq] or null
  const void* q;           // bf16, row stride q_stride elements
  int64_t q_stride;
  const void* k_cache;
  const void* v_cache;
  int64_t num_slots;
  int64_t cache_stride;    // elements between slots
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* req_rows; // null -> identity
  const int32_t* seq_lens;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t max_seq_len;
  float sm_scale;
  int32_t split_tokens;    // fixed mode chunk size; 0 in balanced mode
  int32_t max_splits;      // fixed mode: ceil(max_seq_len / split_tokens)
  int32_t balanced_blocks; // balanced mode: compute units of the device (0 = fixed mode)
  float* part_out;         // fp32 [rows, Hq, 128]
  float* part_lse;         // fp32 [rows, Hq]
  int32_t* meta;           // balanced mode: int32 [B, 2]
  // store fused into the decode launch (k_store null: none): row r of
  // k_new / v_new (row stride new_stride elements) goes to slot out_loc[r]
  void* k_store;
  void* v_store;
  const void* k_new;
  const void* v_new;
  int64_t new_stride;
  const void* out_loc;
  bool out_loc_is_i64;
  hipStream_t stream;
};

struct ExtendArgs {
  void* out;               // bf16 [T, Hq, 128]
  float* lse;              // fp32 [T, Hq] or null
  const void* q;
  int64_t q_stride;
  const void* k_cache;
  const void* v_cache;
  int64_t num_slots;
  int64_t cache_stride;
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* req_rows;
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  const int32_t* q_offsets;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t max_extend_len;
  int32_t max_kv_len;
  float sm_scale;
  void* workspace;         // optional work list (see extend_workspace_bytes) or null
  size_t workspace_bytes;
  hipStream_t stream;
};

// Extend work list: 16 bytes of header (item count) plus one int32 per
// (request, query tile) item.
size_t extend_workspace_bytes(int64_t batch, int ratio, int64_t max_extend_len);

struct MergeArgs {
  void* out;
  float* lse;
  const float* part_out;   // [S, N, H, D]
  const float* part_lse;   // [S, N, H]
  int32_t num_parts;
  int64_t n;
  int32_t num_heads;
  int32_t head_dim;
  bool out_bf16;
  // decode-internal use: per-row part counts from seq_lens (fixed chunks)
  // or from (first, last) workgroup pairs (balanced ranges); else num_parts
  const int32_t* seq_lens;
  int32_t split_tokens;
  const int32_t* meta;
  hipStream_t stream;
};

// Most workgroups the balanced decode launches along x (sizes its workspace).
constexpr int kMaxDecodeBlocks = 2048;

int decode_kv_heads_per_block(int num_kv_heads);
// Workgroups the balanced decode launches along x on a device with this
// many compute units (its partial-output rows are this plus the batch).
int64_t decode_balanced_grid(int num_kv_heads, int ratio, int compute_units);
hipError_t launch_store_kv(const StoreArgs& a);
hipError_t launch_embedding_gather(const GatherArgs& a);
hipError_t launch_rope_cache(float* cache, int64_t max_position, int32_t rotary_dim, double base,
                             hipStream_t stream);
hipError_t launch_qk_norm_rope_store(const PrologueArgs& a);
hipError_t launch_paged_decode(const DecodeArgs& a);
hipError_t launch_paged_extend(const ExtendArgs& a);
hipError_t launch_merge(const MergeArgs& a);

// Debug-check build (MSGL_DEBUG_CHECKS): device-side checks of the index
// arrays, run on the call's stream before its kernels (debug_checks.hip).
enum : unsigned int {
  kDebugOutLoc = 1u,       // out_loc entry outside [0, num_slots)
  kDebugLength = 2u,       // length negative, past its declared maximum or the table width
  kDebugQOffsets = 4u,     // q_offsets[r] negative or q_offsets[r+1] - q_offsets[r] != extend_len
  kDebugRow = 8u,          // req_rows entry negative
  kDebugSlot = 16u,        // page-table entry read by the call outside the pool
  kDebugNewestSlot = 32u,  // fused store: out_loc[r] is not the slot of request r's newest key
};

struct DebugRequestCheck {
  const int32_t* lens = nullptr;       // seq_lens (decode) or prefix_lens (extend)
  const int32_t* ext = nullptr;        // extend_lens, or null for decode
  const int32_t* q_offsets = nullptr;  // [batch + 1], or null
  const int32_t* req_rows = nullptr;   // or null (request r reads row r)
  const int32_t* pt = nullptr;
  int64_t pt_stride = 0;
  int32_t batch = 0;
  int32_t max_total = 0;               // max_seq_len, or max_kv_len for extend
  int32_t max_ext = 0;                 // max_extend_len (extend)
  int64_t num_slots = 0;
  int32_t page_span = 1;               // P for a power-of-two page_size P > 1, else 1
  const void* out_loc = nullptr;       // fused store + decode: new rows' slots, or null
  int32_t out_loc_i64 = 0;
  unsigned int* w = nullptr;           // set by debug_check_requests
};

struct DebugFailure {
  unsigned int bits = 0;   // every failed check
  unsigned int first = 0;  // the check of the first failure, and its details:
  int a = 0;               // index / request
  int b = 0;               // key, extend_len or offset step
  long long v = 0;         // offending value
};

bool debug_stream_capturing(hipStream_t s);
hipError_t debug_check_out_loc(const void* out_loc, bool i64, int64_t n, int64_t num_slots,
                               hipStream_t s);
hipError_t debug_check_requests(DebugRequestCheck c, hipStream_t s);
// Waits for the stream, reads this device's report into *f and clears it.
hipError_t debug_collect(hipStream_t s, DebugFailure* f);

}  // namespace msgl

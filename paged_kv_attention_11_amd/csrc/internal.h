// Internal interface between the C-ABI layer (abi.hip) and the kernel
// translation units.  Not installed; the public interface is
// include/pagedattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Decode tiling constants shared by the host plan and the kernels.
constexpr int kDecodeWaves = 4;           // waves per decode work-group
constexpr int kDecodeTokPerIter = 16;     // keys one wave handles per iteration
constexpr int kSplitQuantum = kDecodeWaves * kDecodeTokPerIter;  // 64
constexpr int kMaxSplitTokens = 2048;     // decode: LDS slot staging bound
constexpr int kVerifyMaxSplit = 2048;     // verify: longest piece (its page ids are staged in LDS)
constexpr int kMaxGroup = 8;              // query heads per KV head (decode)

struct StoreArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
  void* k_pool;
  void* v_pool;
  int64_t num_rows;
  int32_t row_chunks;  // bytes of one [num_kv_heads, head_dim] row / 16
};

struct RopeArgs {
  const void* q;
  void* q_out;
  const void* k_new;
  const void* v_new;
  const int32_t* positions;
  const int64_t* slot_mapping;
  const float* cos_table;  // [max_position, head_dim / 2]
  const float* sin_table;
  void* k_pool;
  void* v_pool;
  int64_t num_rows;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_position;
  int32_t bf16;
};

struct GatherArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int64_t* out_offsets;
  void* k_out;
  void* v_out;
  int64_t pt_stride;
  int32_t num_seqs;
  int32_t max_seq_len;
  int32_t log2_page;
  int32_t row_chunks;
};

// Inputs of the decode partial kernel's work order (plan.h).
struct PlanArgs {
  int4* plan;                // [max_splits * num_seqs] entries written; null: no order
  const int32_t* seq_lens;   // [B]
  const int32_t* key_begin;  // [B] first key of each request's range, or null (0)
  const int32_t* q_indptr;   // [B+1] mixed batches (only one-row requests get pieces), or null
  int32_t num_seqs;
  int32_t split_tokens;
  int32_t max_splits;
  int32_t always_partial;
  int32_t xcd_classes;  // 1 .. 8: contiguous request ranges whose full pieces are interleaved (1: request order)
};

struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* key_begin;  // [B] first key of each request's range, or null (0)
  // [B+1] mixed batches: request b's new rows start at q_indptr[b]; only
  // requests with exactly one new row are handled here.  Null: row b.
  const int32_t* q_indptr;
  float* o_part;  // [B, Hq, ws_pieces, D]
  float* lse;     // [B, Hq, ws_pieces], log2 domain
  void* out;      // [B, Hq, D]
  int64_t pt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t log2_page;
  int32_t split_tokens;
  int32_t max_splits;    // pieces per request in the grid
  int32_t piece_offset;  // workspace index of a request's piece 0
  int32_t ws_pieces;     // pieces per (request, head) row of the workspace
  int32_t always_partial;  // 1: never finish a single-piece request in the partial kernel
  int32_t heads_per_block;  // KV heads one work-group serves (1, 2 or 4; divides num_kv_heads)
  // pieces starting at or after this key are read with nontemporal loads
  // (the leading keys, which prefix caching shares, through the caches)
  int32_t cached_keys;
  // leading pieces written by the shared-prefix kernel (combine only)
  const int32_t* group_lens;  // [B] keys covered by those pieces, or null
  int32_t group_piece_keys;
  int32_t bf16;
  float scale_log2;  // softmax scale * log2(e)
  // [max_splits * num_seqs] work order of the partial kernel, written before
  // it runs (plan.h); null: every (piece, request, head) of the grid in
  // piece-major order
  int4* plan;
};

// Matrix-core attention tiles: the extend call, and the shared-prefix pass of
// the cascade decode (rows = members of a request group x query heads, keys =
// the group's shared pages, results written as split partials).
struct ExtendArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  const int32_t* q_indptr;     // extend: [B+1]; prefix: group starts [G+1]
  const int32_t* page_table;   // extend: per request; prefix: per group
  const int32_t* seq_lens;     // extend: [B]; prefix: shared lengths per request [B]
  void* out;                   // extend: [T_q, Hq, D] bf16
  float* o_part;               // prefix: decode workspace partials; split extend: [T_q, Hq, num_pieces, D]
  float* lse;                  // log2-sum-exp of each partial
  int64_t pt_stride;
  int32_t num_seqs;            // extend: requests; prefix: groups
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t log2_page;
  int32_t max_q_len;           // extend: longest chunk; prefix: largest group
  int32_t max_keys;            // prefix: bound on the shared lengths (larger ones are clamped)
  int32_t piece_keys;          // prefix and split extend: keys per piece
  int32_t num_pieces;          // prefix: pieces per group; extend: pieces per request (1: not split)
  int32_t ws_pieces;           // prefix: workspace row stride in pieces
  int32_t skip_single;         // extend: leave requests with one new row to the decode kernels
  float scale_log2;
  // prefix: when plan.plan is set, one more work-group writes the work order
  // of the decode partial kernel that follows
  PlanArgs plan;
};

// Short chunks (parallel verification of drafted tokens): split-K over keys,
// the chunk's rows x G heads packed into 16x16 matrix-core tiles.
struct VerifyArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;               // [T_q, H_q, D] bf16
  const int32_t* q_indptr;     // [B+1]
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* out;                   // [T_q, H_q, D] bf16
  float* o_part;               // [B, max_q_len, H_q, max_splits, D]
  float* lse;                  // [B, max_q_len, H_q, max_splits]
  int64_t pt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t log2_page;
  int32_t max_q_len;           // rows per request; max_q_len * G <= 32
  int32_t split_tokens;        // keys per piece, multiple of 64, <= kVerifyMaxSplit
  int32_t max_splits;
  float scale_log2;
};

struct CheckArgs {
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_indptr;      // may be null
  const int64_t* slot_mapping;  // may be null
  uint32_t* flags;
  int64_t num_pages;
  int64_t num_rows;
  int32_t pt_stride;
  int32_t num_seqs;
  int32_t max_seq_len;
  int32_t max_q_len;
  int32_t page_size;
};

struct CascadeCheckArgs {
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* group_starts;
  const int32_t* prefix_page_table;
  const int32_t* shared_lens;
  uint32_t* flags;
  int64_t num_pages;
  int32_t pt_stride;
  int32_t prefix_pt_stride;
  int32_t num_seqs;
  int32_t num_groups;
  int32_t max_group_size;
  int32_t max_shared_len;
  int32_t page_size;
};

hipError_t launch_kv_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_rope_store(const RopeArgs& a, hipStream_t stream);
// Return hipErrorInvalidValue for an instantiation that does not exist
// (the ABI layer validates first, so this is a guard, not a code path).
hipError_t launch_decode_plan(const PlanArgs& p, hipStream_t stream);
// The work order (when p.plan is set) and the store of s.num_rows new rows in
// one launch.
hipError_t launch_decode_plan_store(const PlanArgs& p, const StoreArgs& s, hipStream_t stream);
hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream);
hipError_t launch_prefix(const ExtendArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);
hipError_t launch_check_cascade(const CascadeCheckArgs& a, hipStream_t stream);

}  // namespace pa

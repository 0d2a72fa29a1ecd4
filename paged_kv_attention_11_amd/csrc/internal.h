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
constexpr int kMaxSplitTokens = 1024;     // LDS slot staging bound
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

struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* o_part;  // [B, Hq, S, D]
  float* lse;     // [B, Hq, S], log2 domain
  void* out;      // [B, Hq, D]
  int64_t pt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t log2_page;
  int32_t split_tokens;
  int32_t max_splits;
  int32_t bf16;
  float scale_log2;  // softmax scale * log2(e)
};

struct ExtendArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  const int32_t* q_indptr;
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* out;
  int64_t pt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t log2_page;
  int32_t max_q_len;
  float scale_log2;
};

hipError_t launch_kv_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
// Return hipErrorInvalidValue for an instantiation that does not exist
// (the ABI layer validates first, so this is a guard, not a code path).
hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream);

}  // namespace pa

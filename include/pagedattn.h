/*
 * pagedattn.h -- C ABI of a gfx950 (MI355X) library for attention over a
 * paged KV cache.
 *
 * The operations are the hot path of the small SGLang-style serving engines
 * described on the pages (nanoSGLang README, mini-sglang README, nanollmserve
 * README, "mini-sglang from Scratch", Mini-SGLang README of the yangyonggit
 * fork):
 *
 *   pa_kv_store    write a step's new K/V rows into the pool slots given by a
 *                  slot mapping ("mini-sglang from Scratch", section "How this
 *                  book works": the KV-cache writes);
 *   pa_rope_kv_store
 *                  the same store fused with the rotary position embedding
 *                  that precedes it: q and k rotated with half-split pairing
 *                  (nanoSGLang README, section Notable Fixes), k and v
 *                  written to the pool;
 *   pa_decode      one new token per request attends every cached key of its
 *                  request through the page table, grouped-query heads
 *                  (Mini-SGLang README, section Reference Attention Backends;
 *                  nanoSGLang README, section Ablation: zero-copy paged
 *                  attention through page-table indirection);
 *   pa_extend      a chunk of new tokens per request (chunked prefill, or the
 *                  parallel verification of drafted tokens) attends the cached
 *                  prefix and, causally, the chunk itself (Mini-SGLang README,
 *                  sections Reference Attention Backends and Speculative
 *                  Decoding; nanollmserve README, section v0.7 Chunked
 *                  Prefill);
 *   pa_decode_cascade
 *                  the result of pa_decode, computed for requests whose
 *                  leading pages are shared through a prefix cache (the radix
 *                  tree of nanoSGLang README, section Architecture; prefix
 *                  match in the mini-sglang README, TODO list; the radix
 *                  cache with matching and reference counting of "mini-sglang
 *                  from Scratch", section "What you will be able to do"):
 *                  each shared page is read once per group of requests
 *                  instead of once per request;
 *   pa_attend_mixed
 *                  one call for the mixed batches continuous batching makes
 *                  (nanoSGLang README, section Features: continuous batching
 *                  with mixed prefill and decode): requests with one new
 *                  token take the decode kernels, the others the extend
 *                  kernel; fixed buffers padded with empty requests
 *                  ("mini-sglang from Scratch": CUDA Graph's fixed-buffer
 *                  contract) let a whole step be captured once and replayed;
 *   pa_verify      the same attention as pa_extend for short chunks: the
 *                  parallel verification of k drafted tokens (Mini-SGLang
 *                  README, section Speculative Decoding: one parallel
 *                  prefill rather than k decodes), split over the keys like
 *                  decode;
 *   pa_gather      copy requests' pages out to contiguous K/V (test and
 *                  calibration helper: the legacy per-token copy that paged
 *                  attention removes, nanoSGLang README, section Ablation).
 *
 * Data layout (all device memory, owned by the caller):
 *   k_pool, v_pool  [num_pages, page_size, num_kv_heads, head_dim], contiguous
 *                   ("NHD", nanoSGLang README, section Architecture).  Token
 *                   t of a request lives in physical page page_table[t /
 *                   page_size] at offset t % page_size; its flat slot is
 *                   page * page_size + offset.
 *   page_table      int32 [num_seqs, pt_stride], row-major.  Entries at or
 *                   beyond ceil(seq_len / page_size) are never read.
 *   seq_lens        int32 [num_seqs]: keys of each request *including* the
 *                   new tokens, which must already have been stored.
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless stated otherwise; `stream` is a
 *     hipStream_t (NULL = the default stream).  Every call only enqueues work
 *     on `stream` and returns; none synchronises, allocates or frees memory,
 *     so the calls can be captured into a HIP graph.
 *   - Scalars and pointers are validated on the host before any HIP call; a
 *     call that returns an error has launched nothing.  PA_ERR_HIP reports a
 *     launch failure (hipGetLastError after the launch).
 *   - Values that live in device memory (page ids, seq_lens, slot mapping,
 *     q_indptr) are a caller contract and are not checked: page ids must be in
 *     [0, num_pages), seq_lens in [0, max_seq_len], slots in
 *     [0, num_pages * page_size) or negative (skip), distinct.
 *   - The library keeps no state between calls and is thread-safe, except
 *     for the static scratch buffer of pa_decode_noalloc (see there).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  PA_ERR_SHAPE = 2,       /* sizes are negative or inconsistent                 */
  PA_ERR_DTYPE = 3,       /* unknown dtype, or a dtype this call does not take  */
  PA_ERR_UNSUPPORTED = 4, /* valid, but head_dim / group / page size not built  */
  PA_ERR_WORKSPACE = 5,   /* workspace missing, too small or misaligned         */
  PA_ERR_HIP = 6,         /* a HIP runtime call reported an error               */
  PA_ERR_SCRATCH = 7      /* pa_decode_noalloc: more than the static scratch    */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* A paged K/V pool in caller-owned device memory. */
typedef struct {
  void* k_pool;         /* [num_pages, page_size, num_kv_heads, head_dim]     */
  void* v_pool;         /* same shape and dtype                               */
  int64_t num_pages;    /* > 0; num_pages * page_size must be < 2^31          */
  int32_t page_size;    /* power of two, 1 .. 256                             */
  int32_t num_kv_heads; /* >= 1                                               */
  int32_t head_dim;     /* 64 or 128                                          */
  int32_t dtype;        /* pa_dtype; elements of K, V, q and out              */
} pa_kv_pool;

/* Library version string (static storage). */
const char* pa_version(void);

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(int32_t status);

/*
 * pa_kv_store: for each i in [0, num_rows) with slot_mapping[i] >= 0, copy row
 * k_new[i] ([num_kv_heads, head_dim], pool dtype) to flat slot
 * slot_mapping[i] of k_pool, and v_new[i] to the same slot of v_pool.  A byte
 * copy: bit-exact, no conversion.  Negative slots are padding and are skipped
 * (fixed-size buffers can be reused).  k_new, v_new: [num_rows, num_kv_heads,
 * head_dim] contiguous, 16-byte aligned.  num_rows == 0 is a no-op.
 * Overlapping slots are undefined.
 */
pa_status pa_kv_store(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int64_t num_rows, void* stream);

/*
 * pa_rope_kv_store: pa_kv_store with the rotary position embedding of q and k
 * done on the way.  For each row i in [0, num_rows) with slot_mapping[i] >= 0
 * and p = positions[i]:
 *   q_out[i, h, :] = rope(q[i, h, :], p)   for every query head h
 *   k pool at flat slot slot_mapping[i] = rope(k_new[i], p)
 *   v pool at that slot = v_new[i]          (byte copy)
 * where rope turns each channel pair (j, j + head_dim/2) of a head by the
 * angle whose cosine and sine are cos_table[p, j] and sin_table[p, j]:
 *   (a, b) -> (a * cos - b * sin, b * cos + a * sin).
 * Rows with a negative slot are padding: nothing is read or written for them
 * (their q_out rows are left as they are).
 *   q, q_out        [num_rows, num_q_heads, head_dim], pool dtype, 16-byte
 *                   aligned; q_out may be q (in place).  num_q_heads may be
 *                   0 (keys only; q and q_out are then not used).
 *   k_new, v_new    [num_rows, num_kv_heads, head_dim], pool dtype, 16-byte
 *                   aligned.
 *   positions       int32 [num_rows]; values outside [0, max_position) are a
 *                   contract violation and are clamped (no access leaves the
 *                   tables).
 *   cos_table, sin_table
 *                   fp32 [max_position, head_dim / 2], row-major, 16-byte
 *                   aligned (an engine's precomputed rotary cache).
 * The arithmetic is fp32 with one rounding to the pool dtype at the end.
 * Slots must be distinct; overlapping slots are undefined.
 */
pa_status pa_rope_kv_store(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const void* k_new,
                           const void* v_new, const int32_t* positions, const int64_t* slot_mapping,
                           int64_t num_rows, const float* cos_table, const float* sin_table, int32_t max_position,
                           void* q_out, void* stream);

/*
 * Decode split plan.  The key range of each request is cut into consecutive
 * pieces of split_tokens keys; each (request, piece, block of KV heads) is one
 * unit of work, and a second kernel merges the pieces by log-sum-exp weights
 * (the online softmax of the Triton backend in the Mini-SGLang README,
 * yangyonggit fork, Reference Attention Backends, cut into independent
 * pieces).  pa_decode_split_tokens returns the piece length the library
 * chooses from the host-side sizes alone (a multiple of 64, at most 2048).
 * Every decode call takes a split_tokens argument: 0 means "this automatic
 * choice", any other value must be a multiple of 64 in [64, 2048].  The
 * result depends on the split only through floating-point rounding.
 *
 * pa_decode_heads_per_block returns how many neighbouring KV heads one unit
 * serves for these sizes (1, 2 or 4, a divisor of num_kv_heads; 0 for invalid
 * sizes): large batches take several heads per unit, whose loads then cover
 * neighbouring slices of the same K/V rows, and shorter automatic pieces
 * (at most 2048 / heads keys).  The choice depends only on these three sizes,
 * never on split_tokens, and changes no result beyond floating-point
 * rounding; every decode call (plain, cascade own keys, mixed) uses it.
 */
int32_t pa_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len);
int32_t pa_decode_heads_per_block(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                                  int32_t split_tokens);

/*
 * Bytes of device workspace pa_decode needs for these sizes and split_tokens
 * (0 = the automatic plan); 0 on invalid sizes.  Layout:
 * fp32 partial outputs [num_seqs, num_q_heads, S, head_dim] followed (at a
 * 256-byte boundary) by fp32 log2-sum-exp values [num_seqs, num_q_heads, S],
 * S = ceil(max_seq_len / split_tokens), and, when S > 1, (at a 256-byte
 * boundary) the order in which the partial kernel takes the pieces, int32
 * [S * num_seqs, 4], written by a one-work-group kernel that pa_decode_partial
 * launches first on large batches.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t split_tokens);

/*
 * pa_decode: out[b, h, :] = softmax(scale * K_b,g q[b, h, :]) V_b,g over the
 * seq_lens[b] keys of request b, g = h / (num_q_heads / num_kv_heads).
 *   q     [num_seqs, num_q_heads, head_dim], pool dtype, 16-byte aligned
 *   out   [num_seqs, num_q_heads, head_dim], pool dtype (bf16 outputs are
 *         rounded once, to nearest even, from fp32 accumulation)
 *   page_table [num_seqs, pt_stride]; pt_stride * page_size >= max_seq_len
 *   max_seq_len: host-side upper bound of seq_lens (sizes the grid; no
 *         device read)
 *   workspace: >= pa_decode_workspace_bytes(...) bytes, 256-byte aligned;
 *         its contents need no initialisation and are clobbered.
 * A request with seq_len 0 gets a zero row.  Requires num_q_heads a multiple
 * of num_kv_heads with group size 1..8 (fp32: group * head_dim <= 512).
 * Enqueues pa_decode_partial then pa_decode_combine.
 */
pa_status pa_decode(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                    const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t max_seq_len, float scale, int32_t split_tokens,
                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc: pa_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, result and kernels as pa_decode, without the
 * workspace: the split partials go to a buffer of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds in static device memory,
 * one copy per GPU, kept from the loading of the library's code on that GPU
 * until the process ends.  The call itself allocates and frees nothing.
 *   - A call whose partials would need more than PA_NOALLOC_SCRATCH_BYTES
 *     (pa_decode_workspace_bytes(...) for the same sizes) returns
 *     PA_ERR_SCRATCH and launches nothing.  The Qwen3-8B-shaped batch of 256
 *     requests of up to 8192 keys needs about 32 MiB.
 *   - The buffer needs no initialisation and keeps whatever the last call
 *     left in it.
 *   - All calls on one GPU share its buffer: two calls that can overlap on
 *     one GPU (other streams, other host threads) race and give wrong rows.
 *     Serialise them, or use pa_decode with a workspace of each caller's own.
 *   - The stream must belong to the current device (PA_ERR_UNSUPPORTED
 *     otherwise); the buffer's address on a device is looked up on the first
 *     call made there.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, float scale, int32_t split_tokens,
                            void* out, void* stream);

/*
 * The two stages of pa_decode, callable one at a time (same arguments).
 * pa_decode_partial (on large batches a one-work-group kernel that writes
 * the order of the pieces into the workspace, then the partial kernel)
 * writes, for every request with more than one piece, the
 * normalised output and log2-sum-exp of each piece into the workspace, and
 * writes `out` directly for requests with exactly one piece.
 * pa_decode_combine merges the pieces into `out` for requests with more than
 * one piece and writes zero rows for requests with seq_len 0.
 */
pa_status pa_decode_partial(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, float scale, int32_t split_tokens,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_decode_combine(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, float scale, int32_t split_tokens,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_extend: request b has n_b = q_indptr[b+1] - q_indptr[b] new tokens
 * whose K/V rows are already stored, after a cached prefix of
 * p_b = seq_lens[b] - n_b keys.  Its new token i (absolute position p_b + i)
 * attends keys 0 .. p_b + i:
 *   out[q_indptr[b] + i, h, :] = softmax(scale * K q) V over those keys.
 *   q, out     [q_indptr[num_seqs], num_q_heads, head_dim], bf16, 16-byte
 *              aligned; q_indptr int32 [num_seqs + 1], non-decreasing
 *   max_q_len  host-side upper bound of n_b; max_seq_len of seq_lens.
 *   split_tokens
 *              keys per piece when the keys are split: 0 = the automatic
 *              choice (pa_extend_workspace_bytes tells whether it splits),
 *              else a multiple of 64; a value >= max_seq_len means no split.
 *              The automatic plan splits only batches with few work items
 *              (fewer than 1024 blocks of 128 / G tokens x KV heads x
 *              requests) and long keys: a handful of requests whose chunks
 *              attend long cached prefixes.
 *   workspace  pa_extend_workspace_bytes(...) bytes, 256-byte aligned, when
 *              the keys are split (NULL and 0 bytes allowed otherwise).
 *              Layout: fp32 partial outputs [num_seqs * max_q_len,
 *              num_q_heads, NP, head_dim] (row r of the first axis: query
 *              row r), then (256-byte aligned) fp32 log2-sum-exp
 *              [num_seqs * max_q_len, num_q_heads, NP],
 *              NP = ceil(max_seq_len / split).  Clobbered; no initialisation.
 * With split keys a second kernel merges the pieces of each row by
 * log-sum-exp weights (each piece a row reads holds at least one key it sees).
 * bf16 pools only, head_dim 128 or 64, group size 1 .. 8.  Scores and the
 * output are accumulated in fp32; softmax weights are rounded to bf16 before
 * the weighted sum of V (matrix-core inputs).
 */
size_t pa_extend_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t split_tokens);
pa_status pa_extend(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                    const int32_t* q_indptr, const int32_t* page_table, int32_t pt_stride,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t max_q_len,
                    int32_t max_seq_len, float scale, int32_t split_tokens, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cascade (prefix-aware) decode.  The requests are cut into consecutive
 * groups: group j is requests group_starts[j] .. group_starts[j+1] - 1
 * (group_starts int32 [num_groups + 1], device, non-decreasing, from 0 to
 * num_seqs, so every request is in exactly one group; a request that shares
 * nothing is a group of its own with shared_len 0).  The first
 * shared_lens[b] keys of request b (int32 [num_seqs], device) are keys
 * 0 .. shared_lens[b] - 1 of its group's prefix pages, prefix_page_table row
 * j (int32 [num_groups, prefix_pt_stride], device); they must be the same
 * pages as the first entries of the request's own page_table row.
 *
 * The result is that of pa_decode with the same q, page_table and seq_lens,
 * up to floating-point rounding.  Three kernels are enqueued:
 *   1. per (group, KV head, key piece of prefix_piece_keys keys): every
 *      member's query heads of the KV head against the group's prefix keys,
 *      on the matrix cores (each tile of shared K/V is read once per group);
 *      on large batches one more work-group of this kernel (or, with no
 *      prefix pass, a kernel of its own) writes the order in which kernel 2
 *      takes its pieces into the workspace;
 *   2. per (request, KV head, piece of split_tokens keys): the request's own
 *      keys shared_lens[b] .. seq_lens[b] - 1, as in pa_decode_partial;
 *   3. per (request, query head): merge of both sets of pieces by
 *      log-sum-exp weights.
 * Scores and the output accumulate in fp32; in the first kernel the softmax
 * weights are rounded to bf16 before the weighted sum of V.
 *
 *   max_group_size      host-side upper bound of the group sizes (> 0 when
 *                       num_groups > 0; <= num_seqs)
 *   max_shared_len      host-side upper bound of shared_lens;
 *                       prefix_pt_stride * page_size >= max_shared_len.  A
 *                       shared_len above it is a contract violation: the keys
 *                       beyond the bound are then left out (no access leaves
 *                       the page tables).  0 (or num_groups 0) runs the plain
 *                       decode through kernels 2 and 3.
 *   prefix_piece_keys   keys per piece of kernel 1: 0 = automatic
 *                       (pa_cascade_piece_keys), else a positive multiple of
 *                       64.
 *   split_tokens        as for pa_decode.
 *   k_new, v_new, slot_mapping, num_new_rows
 *                       optional (NULL, NULL, NULL, 0): the step's new K/V
 *                       rows, stored exactly as pa_kv_store would store them
 *                       (same layout, alignment and slot contract), by the
 *                       same launch that writes the work order of kernel 2
 *                       (one launch fewer in the step).  They are stored
 *                       before kernel 2 reads any key; the new rows must not
 *                       land on pages holding shared keys (a radix cache
 *                       writes a new token to a page of its own request).
 *   workspace           >= pa_decode_cascade_workspace_bytes(...) bytes,
 *                       256-byte aligned, clobbered.  Layout: fp32 partial
 *                       outputs [num_seqs, num_q_heads, NP + S, head_dim],
 *                       then (at a 256-byte boundary) fp32 log2-sum-exp
 *                       values [num_seqs, num_q_heads, NP + S], where
 *                       NP = ceil(max_shared_len / prefix_piece_keys) pieces
 *                       of kernel 1 come first and S = ceil(max_seq_len /
 *                       split_tokens) pieces of kernel 2 follow; then, when
 *                       S > 1, the work order of kernel 2 as for pa_decode.
 * bf16 pools only, head_dim 128 or 64, group size (num_q_heads /
 * num_kv_heads) 1 .. 8.  A request with seq_len 0 gets a zero row.
 */
int32_t pa_cascade_piece_keys(int32_t num_groups, int32_t max_group_size, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t max_shared_len);
size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len, int32_t split_tokens,
                                         int32_t num_groups, int32_t max_group_size, int32_t max_shared_len,
                                         int32_t prefix_piece_keys);
pa_status pa_decode_cascade(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, const int32_t* group_starts,
                            int32_t num_groups, int32_t max_group_size, const int32_t* prefix_page_table,
                            int32_t prefix_pt_stride, const int32_t* shared_lens, int32_t max_shared_len,
                            float scale, int32_t split_tokens, int32_t prefix_piece_keys, const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_new_rows, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The stages of pa_decode_cascade, one kernel each, callable one at a time on
 * one workspace (same arguments; each validates them all):
 *   _order    the work order of kernel 2 (a one-work-group kernel; nothing
 *             when kernel 2 runs without one, i.e. on small batches), and
 *             the store of the new rows when they are given (in the same
 *             launch); the other stages ignore the new rows;
 *   _prefix   kernel 1 alone (nothing when there is no shared prefix);
 *   _suffix   kernel 2: reads the work order _order wrote;
 *   _combine  kernel 3: after both _prefix and _suffix.
 * _order must precede _suffix; _prefix writes other parts of the workspace
 * than _order and _suffix and reads nothing they write, so it may run
 * concurrently with them on another stream, with _combine after all three.
 * _suffix reads the step's new rows, so it follows their store; _prefix reads
 * only the keys below each request's shared length, so it may even run
 * beside the store when no new row lands on those prefix pages (a radix
 * cache writes a new token to a page of its own request).  Called as
 * pa_decode_cascade without new rows, the work order is written by one extra
 * work-group of kernel 1 instead (one launch fewer); with new rows, the
 * order-and-store launch comes first.  A work order written for another batch gives wrong rows but
 * no access outside the requests' pages.
 */
pa_status pa_decode_cascade_prefix(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                                   const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_seq_len, const int32_t* group_starts,
                                   int32_t num_groups, int32_t max_group_size,
                                   const int32_t* prefix_page_table, int32_t prefix_pt_stride,
                                   const int32_t* shared_lens, int32_t max_shared_len, float scale,
                                   int32_t split_tokens, int32_t prefix_piece_keys, const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_new_rows, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);
pa_status pa_decode_cascade_suffix(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                                   const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_seq_len, const int32_t* group_starts,
                                   int32_t num_groups, int32_t max_group_size,
                                   const int32_t* prefix_page_table, int32_t prefix_pt_stride,
                                   const int32_t* shared_lens, int32_t max_shared_len, float scale,
                                   int32_t split_tokens, int32_t prefix_piece_keys, const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_new_rows, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);
pa_status pa_decode_cascade_combine(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                                    const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                                    int32_t num_seqs, int32_t max_seq_len, const int32_t* group_starts,
                                    int32_t num_groups, int32_t max_group_size,
                                    const int32_t* prefix_page_table, int32_t prefix_pt_stride,
                                    const int32_t* shared_lens, int32_t max_shared_len, float scale,
                                    int32_t split_tokens, int32_t prefix_piece_keys, const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_new_rows, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);
pa_status pa_decode_cascade_order(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                                  const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t max_seq_len, const int32_t* group_starts,
                                  int32_t num_groups, int32_t max_group_size,
                                  const int32_t* prefix_page_table, int32_t prefix_pt_stride,
                                  const int32_t* shared_lens, int32_t max_shared_len, float scale,
                                  int32_t split_tokens, int32_t prefix_piece_keys, const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_new_rows, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * pa_verify: the result of pa_extend (same arguments and semantics) for
 * requests whose chunks are short, as in the verification of drafted tokens:
 * max_q_len * (num_q_heads / num_kv_heads) <= 32.  The keys of each request
 * are split into pieces handled by separate work-groups, each reading its
 * keys once for all rows of the chunk and all query heads of a KV head; a
 * second kernel merges the pieces.
 *   split_tokens: keys per piece (the last piece of a request shorter), a
 *              multiple of 64 in [64, 2048]; 0: the automatic choice, 1536,
 *              or max_seq_len rounded up to a multiple of 64 when that is
 *              smaller (one piece per request).
 *   workspace: pa_verify_workspace_bytes(...) bytes, 256-byte aligned
 *              (0 bytes and NULL allowed when one piece covers max_seq_len).
 *              Layout: fp32 partial outputs [num_seqs, max_q_len,
 *              num_q_heads, S, head_dim], then (256-byte aligned) fp32
 *              log2-sum-exp [num_seqs, max_q_len, num_q_heads, S],
 *              S = ceil(max_seq_len / split), split = split_tokens or the
 *              automatic choice.
 * Chunks longer than max_q_len are a contract violation (their extra rows
 * are not computed).  bf16 pools only, head_dim 128 or 64, group size
 * 1 .. 8.  Softmax weights are rounded to bf16 before the weighted sum of V.
 */
size_t pa_verify_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t split_tokens);
pa_status pa_verify(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* q_indptr,
                    const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t max_q_len, int32_t max_seq_len, float scale, int32_t split_tokens, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_attend_mixed: the result of pa_extend (same q, q_indptr, page_table,
 * seq_lens, out) for a batch that mixes decode requests (one new row) with
 * chunked-prefill or verify chunks (several new rows).  Requests with exactly
 * one new row go through the split-K decode kernels (their keys are split
 * over many work-groups), the others through the matrix-core extend kernel;
 * requests with no new row (q_indptr[b+1] == q_indptr[b], seq_len 0) are
 * padding and produce nothing.  Enqueues three kernels: decode partial,
 * extend (only if max_q_len > 1), combine.
 *   split_tokens, workspace, workspace_bytes: as for pa_decode, sized by
 *                   pa_decode_workspace_bytes(num_seqs, num_q_heads,
 *                   num_kv_heads, head_dim, max_seq_len, split_tokens).
 *   max_q_len, max_seq_len: host-side bounds; the grids and the split plan
 *                   depend only on them, so a captured call can be replayed
 *                   with other device-side contents within the same bounds.
 * bf16 pools only, head_dim 128 or 64, group size 1 .. 8.
 */
pa_status pa_attend_mixed(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* q_indptr,
                          const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t max_q_len, int32_t max_seq_len, float scale, int32_t split_tokens, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_check_batch: debug check of the device-resident values every other call
 * takes on trust.  Enqueues kernels that clear *flags (one uint32 in device
 * memory) and then OR into it:
 *   PA_CHECK_SEQ_LEN        a seq_len outside [0, max_seq_len]
 *   PA_CHECK_Q_INDPTR       q_indptr[0] != 0, or a chunk n_b = q_indptr[b+1] -
 *                           q_indptr[b] outside [0, min(seq_len, max_q_len)]
 *                           (only when q_indptr is given)
 *   PA_CHECK_PAGE_ID        a page id outside [0, num_pages) among the
 *                           ceil(seq_len / page_size) pages a request uses
 *   PA_CHECK_SLOT_RANGE     a slot >= num_pages * page_size (only when
 *                           slot_mapping is given)
 *   PA_CHECK_SLOT_DUPLICATE a live slot given twice (pairwise comparison:
 *                           meant for debugging, not every step)
 * It reads only page_table, seq_lens, q_indptr and slot_mapping -- never a
 * pool page -- so it is safe to run on the very inputs it is meant to catch.
 * The caller reads *flags after synchronising the stream; 0 means none found.
 * q_indptr and slot_mapping may be NULL (those checks are skipped).
 */
enum {
  PA_CHECK_SEQ_LEN = 1u,
  PA_CHECK_Q_INDPTR = 2u,
  PA_CHECK_PAGE_ID = 4u,
  PA_CHECK_SLOT_RANGE = 8u,
  PA_CHECK_SLOT_DUPLICATE = 16u
};
pa_status pa_check_batch(const pa_kv_pool* pool, const int32_t* page_table, int32_t pt_stride,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len, const int32_t* q_indptr,
                         int32_t max_q_len, const int64_t* slot_mapping, int64_t num_rows, uint32_t* flags,
                         void* stream);

/*
 * pa_check_cascade: the same kind of debug check for the group description
 * of pa_decode_cascade (whose kernels take it on trust).  Clears *flags, then
 * ORs into it:
 *   PA_CHECK_GROUP_STARTS   group_starts[0] != 0, group_starts[num_groups] !=
 *                           num_seqs, a decreasing step, or a group larger
 *                           than max_group_size
 *   PA_CHECK_SHARED_LEN     a shared_len outside [0, min(seq_len,
 *                           max_shared_len)] (a shared_len above
 *                           max_shared_len would make the cascade leave keys
 *                           out)
 *   PA_CHECK_PREFIX_PAGE    a page holding a request's shared keys that is
 *                           not its group's prefix page at that position, or
 *                           a prefix page id outside [0, num_pages)
 * It reads only the tables, never a pool page.  With num_groups 0 it only
 * clears *flags.  The caller reads *flags after synchronising the stream.
 */
enum {
  PA_CHECK_GROUP_STARTS = 32u,
  PA_CHECK_SHARED_LEN = 64u,
  PA_CHECK_PREFIX_PAGE = 128u
};
pa_status pa_check_cascade(const pa_kv_pool* pool, const int32_t* page_table, int32_t pt_stride,
                           const int32_t* seq_lens, int32_t num_seqs, const int32_t* group_starts,
                           int32_t num_groups, int32_t max_group_size, const int32_t* prefix_page_table,
                           int32_t prefix_pt_stride, const int32_t* shared_lens, int32_t max_shared_len,
                           uint32_t* flags, void* stream);

/*
 * pa_gather: copy the first seq_lens[b] tokens of every request, in logical
 * order, to contiguous k_out / v_out rows starting at row out_offsets[b]
 * (int64 [num_seqs + 1], device).  k_out, v_out: [out_offsets[num_seqs],
 * num_kv_heads, head_dim], pool dtype.  Bit-exact.  Test and calibration
 * helper.
 */
pa_status pa_gather(const pa_kv_pool* pool, const int32_t* page_table, int32_t pt_stride,
                    const int32_t* seq_lens, const int64_t* out_offsets, int32_t num_seqs,
                    int32_t max_seq_len, void* k_out, void* v_out, void* stream);

/*
 * pa_stream_read: read `bytes` (a multiple of 16) of device memory at src
 * (16-byte aligned) with nontemporal 16-byte vector loads (streamed past
 * the caches; each work-group reads its own contiguous run) and OR a nonzero digest
 * of them into *sink (a uint32 in device memory; the value has no meaning
 * beyond keeping the loads live).  Calibration helper: the read-only HBM
 * rate this device reaches, the ceiling the streaming kernels (decode,
 * verify) are measured against beside the 8 TB/s peak.
 */
pa_status pa_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */

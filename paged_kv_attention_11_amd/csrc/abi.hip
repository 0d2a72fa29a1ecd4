// C ABI of the paged-attention library: host-side validation and dispatch.
// Every argument is checked before the first HIP call; a call that fails
// validation launches nothing.  The library allocates nothing and never
// synchronises; its only state is the per-device address of the static
// scratch buffer of pa_decode_noalloc.
#include <limits.h>

#include <algorithm>
#include <mutex>

#include "pagedattn.h"
#include "internal.h"

// Scratch memory of pa_decode_noalloc, for callers that cannot allocate
// device memory.  Every GPU the library runs on holds its own copy of the
// array from the moment the code object is loaded there until the process
// ends.  In host code `scratch` is only a stand-in for the symbol: its device
// address is looked up once per device (scratch_address) and only that
// address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (which must be the
// device of `stream`), looked up on the first call on that device.
pa_status scratch_address(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return PA_ERR_HIP;
    if (sdev != dev) return PA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

using pa::kMaxGroup;
using pa::kMaxSplitTokens;
using pa::kSplitQuantum;

constexpr float kLog2e = 1.4426950408889634f;

#ifndef PA_DECODE_CACHED_PIECES
#define PA_DECODE_CACHED_PIECES 1
#endif
#ifndef PA_PLAN_XCD_CLASSES
#define PA_PLAN_XCD_CLASSES 1
#endif

// Automatic split plan: the longest piece (a multiple of 64, at most
// kMaxSplitTokens for decode, kVerifyMaxSplit for verify) that still gives
// about kTargetUnits work-groups, i.e. two rounds of a full chip at the
// decode kernel's occupancy; when no piece length gets there the batch
// cannot fill the chip anyway, and pieces of 256 keys (fewer work-groups,
// less to merge) are fastest.  Measured on one MI355X: Qwen3-0.6B-shaped
// decode (64 requests x 8 KV heads, <= 2048 keys) 53 us at 256 against 58 us
// at 512; Qwen2.5-0.5B-shaped (32 x 2, <= 640 keys) 16.3 us at 256 against
// 18.7 us at 64; Qwen3-8B-shaped radix batch (256 x 8, <= 8192 keys, in the
// work order below) each request's own keys 403 us at 2048, 406 at 1536,
// 412 at 1024 and 432 at 512.
constexpr int64_t kTargetUnits = 4096;
constexpr int kSmallBatchSplit = 256;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int elem_bytes(int32_t dtype) { return dtype == PA_BF16 ? 2 : 4; }

pa_status check_pool(const pa_kv_pool* pool) {
  if (!pool) return PA_ERR_NULL;
  if (pool->dtype != PA_F32 && pool->dtype != PA_BF16) return PA_ERR_DTYPE;
  if (pool->num_pages <= 0 || pool->page_size <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0)
    return PA_ERR_SHAPE;
  if (!pool->k_pool || !pool->v_pool) return PA_ERR_NULL;
  if ((pool->page_size & (pool->page_size - 1)) != 0 || pool->page_size > 256) return PA_ERR_UNSUPPORTED;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (pool->num_pages > (int64_t)INT_MAX / pool->page_size) return PA_ERR_SHAPE;
  if (!aligned(pool->k_pool, 16) || !aligned(pool->v_pool, 16)) return PA_ERR_SHAPE;
  return PA_OK;
}

pa_status hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// hb: KV heads per work-group (decode; 1 for verify).  A work-group then
// covers hb heads of a piece, so the longest piece is kMaxSplitTokens / hb
// keys: the same key-head rows per work-group as one head of the longest
// piece.
int32_t auto_split(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t max_split, int hb = 1) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return kSplitQuantum;
  const int64_t units = (int64_t)num_seqs * (num_kv_heads / hb);
  for (int64_t split = max_split / hb; split >= kSplitQuantum; split -= kSplitQuantum)
    if (units * ((max_seq_len + split - 1) / split) >= kTargetUnits) return (int32_t)split;
  // too small to fill the chip: 256-key pieces, or one piece if shorter
  const int64_t one = (max_seq_len + kSplitQuantum - 1) / kSplitQuantum * kSplitQuantum;
  return (int32_t)(one < kSmallBatchSplit ? one : kSmallBatchSplit);
}

// KV heads per decode work-group.  The four waves of a work-group serve hb
// neighbouring KV heads (4 / hb waves each) of the same keys, so their loads
// cover neighbouring slices of the same K/V rows at about the same time;
// pieces are then at most kMaxSplitTokens / hb keys.  Measured on one MI355X
// on the Qwen3-8B-shaped radix batch (8 KV heads, each request's own keys,
// in the work order), microseconds per launch: one head, 2048-key pieces 402;
// two heads, 1024/1536/2048 keys 384/381/386; four heads, 512/768/1024/1536
// keys 394/389/380/407.  The plain decode of the same batch, which reads the
// shared prefix pages of a group through the L2 of the XCDs that run its
// head blocks, took 495 us with one head, 471-475 with two and 486-494 with
// four (its head blocks then spread over four XCDs instead of two).  The
// automatic split therefore takes pairs of heads when num_kv_heads is even
// and the batch fills the chip with full pieces (1024 keys), else one head,
// where small batches keep the most work-groups; that choice depends on the
// batch like the split itself.  With an explicit split the choice depends
// only on the split and num_kv_heads (the most heads, up to four, with
// split * hb <= kMaxSplitTokens), so a request's result has the same bits in
// any batch.
int decode_heads_per_block(int32_t split_tokens, int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len) {
  if (split_tokens) {
    for (int hb = 4; hb > 1; hb >>= 1)
      if (num_kv_heads % hb == 0 && (int64_t)split_tokens * hb <= kMaxSplitTokens) return hb;
    return 1;
  }
  if (num_kv_heads % 2 == 0 && auto_split(num_seqs, num_kv_heads, max_seq_len, kMaxSplitTokens, 2) * 2 >=
                                   kMaxSplitTokens)
    return 2;
  return 1;
}

// The split of a call: split_tokens if valid (a multiple of 64 in
// [64, max_split]), the automatic choice for 0, -1 otherwise.
int32_t resolve_split(int32_t split_tokens, int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                      int32_t max_split = kMaxSplitTokens, int hb = 1) {
  if (split_tokens == 0) return auto_split(num_seqs, num_kv_heads, max_seq_len, max_split, hb);
  const bool ok = split_tokens >= kSplitQuantum && split_tokens <= max_split && split_tokens % kSplitQuantum == 0;
  return ok ? split_tokens : -1;
}

// The decode split: resolve_split at the batch's heads per work-group.
int32_t resolve_decode_split(int32_t split_tokens, int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len) {
  return resolve_split(split_tokens, num_seqs, num_kv_heads, max_seq_len, kMaxSplitTokens,
                       decode_heads_per_block(0, num_seqs, num_kv_heads, max_seq_len));
}

// The verify split: pieces of split_tokens keys (a multiple of 64 in [64,
// kVerifyMaxSplit]), or automatically (0) of kVerifyAutoSplit keys, one
// piece when every request is shorter.  Each verify work-group streams its
// keys at about the same rate however many share the chip, so fewer, longer
// pieces -- fewer partials to write and merge, fewer work-groups to set up --
// are faster until the work-groups no longer fill the chip.  Measured on one
// MI355X (us per call, 32/8 heads, D = 128, 6 rows per request; pieces of
// 256 / 512 / 1024 / 1536 / 2048 keys): 64 requests of 2048 keys 139 / 116 /
// 102 / 97 / 105; 32 of 8192 keys 258 / 218 / 196 / 189 / 175; 256 of 1030
// keys 276 / 240 / 216 / 178 / 177; 16 of 512..16384 log-uniform 116 / 80 /
// 77 / 71 / 67; 48 of 256..8192 log-uniform 145 / 100 / 84 / 85 / 87; 128 of
// 706 keys 96 / 85 / 63 / 65 / 64; the Qwen3-8B-shaped verify workload 134
// at 1024, 124-127 at 1536, 130 at 2048.  Pieces of equal length within a
// request (ceil(L / 2048) of them, no short last piece) were slower on the
// verify workload (129-132 us) and on four of the six batches above.
constexpr int32_t kVerifyAutoSplit = 1536;
int32_t resolve_verify_split(int32_t split_tokens, int32_t max_seq_len) {
  if (split_tokens == 0) {
    const int64_t one = ((int64_t)(max_seq_len > 0 ? max_seq_len : 1) + kSplitQuantum - 1) / kSplitQuantum * kSplitQuantum;
    return (int32_t)(one < kVerifyAutoSplit ? one : kVerifyAutoSplit);
  }
  return resolve_split(split_tokens, 0, 1, max_seq_len, pa::kVerifyMaxSplit);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Work order of the decode partial kernel (a plan kernel lists the pieces
// that exist, longest first).  The plan kernel is one more launch of a few
// microseconds, so it is used only on grids of at least kPlanMinBlocks
// (request, KV head, piece) units, whatever the heads per work-group (a grid
// of 4096 work-groups of two or four heads each ran 20-25% slower in grid
// order than in the work order on the Qwen3-8B-shaped radix batch); the
// workspace always has room for it when there is more than one piece per
// request.
constexpr int64_t kPlanMinBlocks = 6144;

size_t plan_bytes(int32_t num_seqs, int64_t S) { return S > 1 ? align256((size_t)num_seqs * S * 16) : 0; }

bool use_plan(int32_t num_seqs, int32_t num_kv_heads, int64_t S) {
  return S > 1 && (int64_t)num_seqs * num_kv_heads * S >= kPlanMinBlocks;
}

size_t workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                       int32_t split) {
  const int64_t S = (max_seq_len + split - 1) / split;
  const size_t rows = (size_t)num_seqs * num_q_heads * S;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float)) + plan_bytes(num_seqs, S);
}

// Shared validation of the three decode calls; fills `a` on success.
pa_status prepare_decode(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                         const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                         int32_t num_seqs, int32_t max_seq_len, float scale, int32_t split_tokens,
                         void* out, void* workspace, size_t ws_bytes, pa::DecodeArgs& a,
                         bool check_workspace = true) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_seq_len < 0 || pt_stride < 0 || num_q_heads <= 0) return PA_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (pool->dtype == PA_F32 && G * pool->head_dim > 512) return PA_ERR_UNSUPPORTED;
  if ((int64_t)pt_stride * pool->page_size < max_seq_len) return PA_ERR_SHAPE;
  const int32_t split = resolve_decode_split(split_tokens, num_seqs, pool->num_kv_heads, max_seq_len);
  if (split < 0) return PA_ERR_SHAPE;
  const int hb = decode_heads_per_block(split_tokens, num_seqs, pool->num_kv_heads, max_seq_len);
  const int64_t S = (max_seq_len + split - 1) / split;
  if ((int64_t)num_seqs * pool->num_kv_heads * S > (int64_t)INT_MAX) return PA_ERR_SHAPE;
  if (num_seqs > 0) {
    if (!q || !page_table || !seq_lens || !out) return PA_ERR_NULL;
    if (!aligned(q, 16)) return PA_ERR_SHAPE;
    const size_t need = workspace_bytes(num_seqs, num_q_heads, pool->head_dim, max_seq_len, split);
    if (check_workspace && ws_bytes < need) return PA_ERR_WORKSPACE;
    if (check_workspace && S > 0 && (!workspace || !aligned(workspace, 256))) return PA_ERR_WORKSPACE;
  }
  const size_t rows = (size_t)num_seqs * num_q_heads * S;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.q = q;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.o_part = (float*)workspace;
  a.lse = workspace ? (float*)((char*)workspace + align256(rows * pool->head_dim * sizeof(float))) : nullptr;
  a.out = out;
  a.pt_stride = pt_stride;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.log2_page = ilog2(pool->page_size);
  a.key_begin = nullptr;
  a.q_indptr = nullptr;
  a.split_tokens = split;
  a.max_splits = (int32_t)S;
  a.piece_offset = 0;
  a.ws_pieces = (int32_t)S;
  a.always_partial = 0;
  a.heads_per_block = hb;
  a.group_lens = nullptr;
  a.group_piece_keys = 1;
  a.bf16 = pool->dtype == PA_BF16;
  a.scale_log2 = scale * kLog2e;
  a.cached_keys = PA_DECODE_CACHED_PIECES < 0 ? INT_MAX : split * PA_DECODE_CACHED_PIECES;
  a.plan = workspace && use_plan(num_seqs, pool->num_kv_heads, S)
               ? (int4*)((char*)workspace + align256(rows * pool->head_dim * sizeof(float)) +
                         align256(rows * sizeof(float)))
               : nullptr;
  return PA_OK;
}

// The work order's inputs for the partial kernel described by `a`.
pa::PlanArgs plan_args(const pa::DecodeArgs& a) {
  pa::PlanArgs p;
  p.plan = a.plan;
  p.seq_lens = a.seq_lens;
  p.key_begin = a.key_begin;
  p.q_indptr = a.q_indptr;
  p.num_seqs = a.num_seqs;
  p.split_tokens = a.split_tokens;
  p.max_splits = a.max_splits;
  p.always_partial = a.always_partial;
  // Request ranges whose full pieces each go to one XCD per head block (see
  // the work order): every neighbouring request reads pages it shares with
  // others through one L2.  Not for a cascade's own keys, which share none.
  const int nb = a.num_kv_heads / a.heads_per_block;
  int g = 8, x = nb;
  while (x) {
    const int t = g % x;
    g = x;
    x = t;
  }
  p.xcd_classes = PA_PLAN_XCD_CLASSES && !a.key_begin ? 8 / g : 1;
  return p;
}

// The partial kernel, after its work order when it has one.
pa_status enqueue_partial(const pa::DecodeArgs& a, hipStream_t stream) {
  pa_status st = hip_status(pa::launch_decode_plan(plan_args(a), stream));
  if (st != PA_OK) return st;
  return hip_status(pa::launch_decode_partial(a, stream));
}

// Shared-prefix pass of the cascade decode: keys per piece.  The plan aims
// at about 256 work-groups of the matrix-core kernel, each looping over the
// tiles of its piece, rather than many short work-groups that each pay the
// prologue and write partials (on the Qwen3-8B-shaped radix workload: 512-key
// pieces 28 us, 256-key 27 us, 128-key 38 us, 64-key 72 us).
constexpr int kPrefixTile = 64;   // keys per tile of the matrix-core kernel
constexpr int kPrefixRows = 128;  // query rows per work-group of that kernel
constexpr int64_t kPrefixTargetUnits = 256;

int64_t prefix_row_blocks(int32_t max_group_size, int32_t G) {
  const int tok = kPrefixRows / G;
  return (max_group_size + tok - 1) / tok;
}

int32_t auto_piece_keys(int32_t num_groups, int32_t max_group_size, int32_t G, int32_t num_kv_heads,
                        int32_t max_shared_len) {
  const int64_t units = (int64_t)num_groups * num_kv_heads * prefix_row_blocks(max_group_size, G);
  if (units <= 0 || max_shared_len <= 0) return kPrefixTile;
  const int64_t want = (kPrefixTargetUnits + units - 1) / units;
  int64_t pk = (max_shared_len + want - 1) / want;
  pk = (pk + kPrefixTile - 1) / kPrefixTile * kPrefixTile;
  return (int32_t)(pk < kPrefixTile ? kPrefixTile : pk);
}

int32_t resolve_piece_keys(int32_t piece_keys, int32_t num_groups, int32_t max_group_size, int32_t G,
                           int32_t num_kv_heads, int32_t max_shared_len) {
  if (piece_keys == 0) return auto_piece_keys(num_groups, max_group_size, G, num_kv_heads, max_shared_len);
  return (piece_keys > 0 && piece_keys % kPrefixTile == 0) ? piece_keys : -1;
}

// Workspace of the cascade decode: rows of (prefix pieces + suffix pieces).
size_t cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                               int32_t split, int32_t max_shared_len, int32_t piece_keys) {
  const int64_t S = (max_seq_len + split - 1) / split;
  const int64_t NP = (max_shared_len + piece_keys - 1) / piece_keys;
  const size_t rows = (size_t)num_seqs * num_q_heads * (S + NP);
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float)) + plan_bytes(num_seqs, S);
}

// Split extend.  The extend kernel's items are (token block, request, KV
// head); a batch with fewer than kExtendTargetItems of them (a few requests
// whose chunks attend long cached prefixes) leaves most of the chip idle, so
// the automatic plan also cuts the keys into pieces, merged afterwards by a
// combine kernel: enough pieces to reach the target, each at least
// kExtendMinPiece keys (a shorter piece pays its prologue for too few tiles).
constexpr int64_t kExtendTargetItems = 1024;  // two rounds of two work-groups per compute unit
constexpr int kExtendMinPiece = 512;
constexpr int kExtendTile = 64;

// Keys per piece for these sizes: 0 = not split (one piece), -1 = invalid
// split_tokens.  An explicit split_tokens (a multiple of 64) is taken as is;
// one at or above max_seq_len means no split.
int32_t resolve_extend_split(int32_t split_tokens, int32_t num_seqs, int32_t max_q_len, int G, int32_t num_kv_heads,
                             int32_t max_seq_len) {
  if (split_tokens < 0 || split_tokens % kExtendTile != 0) return -1;
  if (split_tokens > 0) return split_tokens >= max_seq_len ? 0 : split_tokens;
  const int64_t tok = 128 / G;
  const int64_t items = (max_q_len + tok - 1) / tok * (int64_t)num_kv_heads * num_seqs;
  if (items <= 0 || items >= kExtendTargetItems || max_seq_len < 2 * kExtendMinPiece) return 0;
  int64_t np = (kExtendTargetItems + items - 1) / items;
  np = std::min<int64_t>(np, max_seq_len / kExtendMinPiece);
  if (np <= 1) return 0;
  int64_t split = (max_seq_len + np - 1) / np;
  split = (split + kExtendTile - 1) / kExtendTile * kExtendTile;
  return split >= max_seq_len ? 0 : (int32_t)split;
}

size_t extend_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads, int32_t head_dim,
                              int32_t max_seq_len, int32_t split) {
  if (split <= 0) return 0;
  const int64_t NP = (max_seq_len + split - 1) / split;
  const size_t rows = (size_t)num_seqs * max_q_len * num_q_heads * NP;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}

}  // namespace

extern "C" {

const char* pa_version(void) { return "pagedattn 0.1.0 gfx950"; }

const char* pa_status_string(int32_t s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "bad or inconsistent sizes";
    case PA_ERR_DTYPE: return "unsupported dtype";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, group size or page size";
    case PA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_SCRATCH: return "call needs more than the library's static scratch buffer holds";
    default: return "unknown status";
  }
}

pa_status pa_kv_store(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int64_t num_rows, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_rows < 0) return PA_ERR_SHAPE;
  if (num_rows == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return PA_ERR_SHAPE;
  pa::StoreArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.num_rows = num_rows;
  a.row_chunks = pool->num_kv_heads * pool->head_dim * elem_bytes(pool->dtype) / 16;
  return hip_status(pa::launch_kv_store(a, (hipStream_t)stream));
}

pa_status pa_rope_kv_store(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const void* k_new,
                           const void* v_new, const int32_t* positions, const int64_t* slot_mapping,
                           int64_t num_rows, const float* cos_table, const float* sin_table, int32_t max_position,
                           void* q_out, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_rows < 0 || num_q_heads < 0 || max_position <= 0) return PA_ERR_SHAPE;
  if (num_rows == 0) return PA_OK;
  if (!k_new || !v_new || !positions || !slot_mapping || !cos_table || !sin_table) return PA_ERR_NULL;
  if (num_q_heads > 0 && (!q || !q_out)) return PA_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(cos_table, 16) || !aligned(sin_table, 16))
    return PA_ERR_SHAPE;
  if (num_q_heads > 0 && (!aligned(q, 16) || !aligned(q_out, 16))) return PA_ERR_SHAPE;
  if (num_rows * (num_q_heads + 2 * (int64_t)pool->num_kv_heads) * pool->head_dim > ((int64_t)1 << 50))
    return PA_ERR_SHAPE;
  pa::RopeArgs a;
  a.q = q;
  a.q_out = q_out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.positions = positions;
  a.slot_mapping = slot_mapping;
  a.cos_table = cos_table;
  a.sin_table = sin_table;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.num_rows = num_rows;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.max_position = max_position;
  a.bf16 = pool->dtype == PA_BF16;
  return hip_status(pa::launch_rope_store(a, (hipStream_t)stream));
}

int32_t pa_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len) {
  return resolve_decode_split(0, num_seqs, num_kv_heads, max_seq_len);
}

int32_t pa_decode_heads_per_block(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                                  int32_t split_tokens) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_seq_len < 0) return 0;
  if (resolve_decode_split(split_tokens, num_seqs, num_kv_heads, max_seq_len) < 0) return 0;
  return decode_heads_per_block(split_tokens, num_seqs, num_kv_heads, max_seq_len);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t split_tokens) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0)
    return 0;
  const int32_t split = resolve_decode_split(split_tokens, num_seqs, num_kv_heads, max_seq_len);
  if (split < 0) return 0;
  return workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, split);
}

pa_status pa_decode_partial(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, float scale, int32_t split_tokens,
                            void* out, void* workspace, size_t workspace_bytes_, void* stream) {
  pa::DecodeArgs a;
  pa_status st = prepare_decode(pool, q, num_q_heads, page_table, pt_stride, seq_lens, num_seqs,
                                max_seq_len, scale, split_tokens, out, workspace, workspace_bytes_, a);
  if (st != PA_OK || num_seqs == 0) return st;
  return enqueue_partial(a, (hipStream_t)stream);
}

pa_status pa_decode_combine(const pa_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, float scale, int32_t split_tokens,
                            void* out, void* workspace, size_t workspace_bytes_, void* stream) {
  pa::DecodeArgs a;
  pa_status st = prepare_decode(pool, q, num_q_heads, page_table, pt_stride, seq_lens, num_seqs,
                                max_seq_len, scale, split_tokens, out, workspace, workspace_bytes_, a);
  if (st != PA_OK || num_seqs == 0) return st;
  return hip_status(pa::launch_decode_combine(a, (hipStream_t)stream));
}

pa_status pa_decode(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* page_table,
                    int32_t pt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                    float scale, int32_t split_tokens, void* out, void* workspace,
                    size_t workspace_bytes_, void* stream) {
  pa::DecodeArgs a;
  pa_status st = prepare_decode(pool, q, num_q_heads, page_table, pt_stride, seq_lens, num_seqs,
                                max_seq_len, scale, split_tokens, out, workspace, workspace_bytes_, a);
  if (st != PA_OK || num_seqs == 0) return st;
  st = enqueue_partial(a, (hipStream_t)stream);
  if (st != PA_OK) return st;
  // one piece per request: the partial kernel wrote every row (zero rows too)
  if (a.max_splits <= 1) return PA_OK;
  return hip_status(pa::launch_decode_combine(a, (hipStream_t)stream));
}

pa_status pa_decode_noalloc(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* page_table,
                            int32_t pt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                            float scale, int32_t split_tokens, void* out, void* stream) {
  // host-side checks first: the sizes, then whether the partials fit
  pa::DecodeArgs a;
  pa_status st = prepare_decode(pool, q, num_q_heads, page_table, pt_stride, seq_lens, num_seqs, max_seq_len,
                                scale, split_tokens, out, nullptr, 0, a, /*check_workspace=*/false);
  if (st != PA_OK || num_seqs == 0) return st;
  const size_t need = workspace_bytes(num_seqs, num_q_heads, pool->head_dim, max_seq_len, a.split_tokens);
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address((hipStream_t)stream, &ws);
  if (st != PA_OK) return st;
  // the same plan and kernels as pa_decode, on the static buffer
  st = prepare_decode(pool, q, num_q_heads, page_table, pt_stride, seq_lens, num_seqs, max_seq_len, scale,
                      split_tokens, out, ws, PA_NOALLOC_SCRATCH_BYTES, a);
  if (st != PA_OK) return st;
  st = enqueue_partial(a, (hipStream_t)stream);
  if (st != PA_OK) return st;
  if (a.max_splits <= 1) return PA_OK;
  return hip_status(pa::launch_decode_combine(a, (hipStream_t)stream));
}

size_t pa_extend_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t split_tokens) {
  if (num_seqs < 0 || max_q_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  const int32_t split =
      resolve_extend_split(split_tokens, num_seqs, max_q_len, num_q_heads / num_kv_heads, num_kv_heads, max_seq_len);
  if (split < 0) return 0;
  return extend_workspace_bytes(num_seqs, max_q_len, num_q_heads, head_dim, max_seq_len, split);
}

pa_status pa_extend(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* q_indptr,
                    const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t max_q_len, int32_t max_seq_len, float scale, int32_t split_tokens,
                    void* out, void* workspace, size_t workspace_bytes_, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (pool->dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || max_q_len < 0 || max_seq_len < 0 || pt_stride < 0 || num_q_heads <= 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G < 1 || G > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (max_q_len > max_seq_len) return PA_ERR_SHAPE;
  if ((int64_t)pt_stride * pool->page_size < max_seq_len) return PA_ERR_SHAPE;
  const int32_t split = resolve_extend_split(split_tokens, num_seqs, max_q_len, G, pool->num_kv_heads, max_seq_len);
  if (split < 0) return PA_ERR_SHAPE;
  const int64_t NP = split ? (max_seq_len + split - 1) / split : 1;
  const int64_t qblocks = (max_q_len + 128 / G - 1) / (128 / G);
  if (qblocks * NP * pool->num_kv_heads * num_seqs > (int64_t)INT_MAX) return PA_ERR_SHAPE;
  if ((int64_t)num_seqs * max_q_len * num_q_heads * NP > (int64_t)INT_MAX) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_q_len == 0) return PA_OK;
  if (!q || !q_indptr || !page_table || !seq_lens || !out) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return PA_ERR_SHAPE;
  const size_t need = extend_workspace_bytes(num_seqs, max_q_len, num_q_heads, pool->head_dim, max_seq_len, split);
  if (NP > 1 && (workspace_bytes_ < need || !workspace || !aligned(workspace, 256))) return PA_ERR_WORKSPACE;
  pa::ExtendArgs a = {};
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.q = q;
  a.q_indptr = q_indptr;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.pt_stride = pt_stride;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.log2_page = ilog2(pool->page_size);
  a.max_q_len = max_q_len;
  a.num_pieces = (int32_t)NP;
  a.piece_keys = NP > 1 ? split : 0;
  if (NP > 1) {
    const size_t rows = (size_t)num_seqs * max_q_len * num_q_heads * NP;
    a.o_part = (float*)workspace;
    a.lse = (float*)((char*)workspace + align256(rows * pool->head_dim * sizeof(float)));
  }
  a.scale_log2 = scale * kLog2e;
  return hip_status(pa::launch_extend(a, (hipStream_t)stream));
}

int32_t pa_cascade_piece_keys(int32_t num_groups, int32_t max_group_size, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t max_shared_len) {
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return kPrefixTile;
  return auto_piece_keys(num_groups, max_group_size, num_q_heads / num_kv_heads, num_kv_heads,
                         max_shared_len);
}

size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len, int32_t split_tokens,
                                         int32_t num_groups, int32_t max_group_size, int32_t max_shared_len,
                                         int32_t prefix_piece_keys) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      num_groups < 0 || max_group_size < 0 || max_shared_len < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int32_t split = resolve_decode_split(split_tokens, num_seqs, num_kv_heads, max_seq_len);
  const int32_t pk = resolve_piece_keys(prefix_piece_keys, num_groups, max_group_size,
                                        num_q_heads / num_kv_heads, num_kv_heads, max_shared_len);
  if (split < 0 || pk < 0) return 0;
  return cascade_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, split, max_shared_len, pk);
}

}  // extern "C"

namespace {

// Stages: the shared-prefix pass, the own-keys pass, the merge, and the own-keys
// pass's work order (with the store of the step's new rows when they are
// given).  Called together (pa_decode_cascade) without new rows, the work
// order is written by one extra work-group of the shared-prefix pass; called
// one at a time, each stage is one kernel, so the shared-prefix pass may run
// on another stream beside the work order and the own-keys pass.
enum : unsigned { kStagePrefix = 1, kStageSuffix = 2, kStageCombine = 4, kStageOrder = 8, kStageAll = 15 };

// The cascade decode's validation, plan and the enqueueing of the selected
// stages (all three for pa_decode_cascade).
pa_status cascade_impl(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* page_table,
                       int32_t pt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                       const int32_t* group_starts, int32_t num_groups, int32_t max_group_size,
                       const int32_t* prefix_page_table, int32_t prefix_pt_stride, const int32_t* shared_lens,
                       int32_t max_shared_len, float scale, int32_t split_tokens, int32_t prefix_piece_keys,
                       const void* k_new, const void* v_new, const int64_t* slot_mapping, int64_t num_new_rows,
                       void* out, void* workspace, size_t workspace_bytes_, void* stream, unsigned stages) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (pool->dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || max_seq_len < 0 || pt_stride < 0 || num_q_heads <= 0 || num_groups < 0 ||
      max_group_size < 0 || prefix_pt_stride < 0 || max_shared_len < 0 || num_new_rows < 0)
    return PA_ERR_SHAPE;
  if (num_new_rows > 0) {  // the step's new rows, stored by the work-order stage
    if (!k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return PA_ERR_SHAPE;
  }
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G < 1 || G > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if ((int64_t)pt_stride * pool->page_size < max_seq_len) return PA_ERR_SHAPE;
  if ((int64_t)prefix_pt_stride * pool->page_size < max_shared_len) return PA_ERR_SHAPE;
  if (max_group_size > num_seqs) return PA_ERR_SHAPE;
  const int32_t split = resolve_decode_split(split_tokens, num_seqs, pool->num_kv_heads, max_seq_len);
  const int hb = decode_heads_per_block(split_tokens, num_seqs, pool->num_kv_heads, max_seq_len);
  const int32_t pk = resolve_piece_keys(prefix_piece_keys, num_groups, max_group_size, G, pool->num_kv_heads,
                                        max_shared_len);
  if (split < 0 || pk < 0) return PA_ERR_SHAPE;
  const int64_t S = (max_seq_len + split - 1) / split;
  const int64_t NP = (max_shared_len + pk - 1) / pk;
  if ((int64_t)num_seqs * pool->num_kv_heads * S > (int64_t)INT_MAX) return PA_ERR_SHAPE;
  if ((int64_t)num_groups * pool->num_kv_heads * prefix_row_blocks(max_group_size, G) * NP > (int64_t)INT_MAX)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!q || !page_table || !seq_lens || !out || !workspace) return PA_ERR_NULL;
  const bool prefix_pass = num_groups > 0 && max_group_size > 0 && NP > 0;
  if (prefix_pass && (!group_starts || !prefix_page_table || !shared_lens)) return PA_ERR_NULL;
  if (!aligned(q, 16)) return PA_ERR_SHAPE;
  const size_t need =
      cascade_workspace_bytes(num_seqs, num_q_heads, pool->head_dim, max_seq_len, split, max_shared_len, pk);
  if (workspace_bytes_ < need || !aligned(workspace, 256)) return PA_ERR_WORKSPACE;

  const size_t rows = (size_t)num_seqs * num_q_heads * (S + NP);
  float* o_part = (float*)workspace;
  float* lse = (float*)((char*)workspace + align256(rows * pool->head_dim * sizeof(float)));
  const hipStream_t hs = (hipStream_t)stream;

  // pass 2 (each request's own keys [shared_len, seq_len)) and pass 3 (the merge)
  pa::DecodeArgs a = {};
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.q = q;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.key_begin = prefix_pass ? shared_lens : nullptr;
  a.o_part = o_part;
  a.lse = lse;
  a.out = out;
  a.pt_stride = pt_stride;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.log2_page = ilog2(pool->page_size);
  a.split_tokens = split;
  a.max_splits = (int32_t)S;
  a.piece_offset = (int32_t)NP;
  a.ws_pieces = (int32_t)(S + NP);
  a.always_partial = 1;
  a.heads_per_block = hb;
  a.group_lens = prefix_pass ? shared_lens : nullptr;
  a.group_piece_keys = pk;
  a.cached_keys = 0;  // (the own keys are all read nontemporally)
  a.bf16 = 1;
  a.scale_log2 = scale * kLog2e;
  a.plan = use_plan(num_seqs, pool->num_kv_heads, S)
               ? (int4*)((char*)lse + align256(rows * sizeof(float)))
               : nullptr;
  // The work order of pass 2 (when it has one) and the store of the step's
  // new rows (when given) in one launch.  Called together without new rows,
  // one extra work-group of pass 1 writes the order instead.
  const bool store_rows = num_new_rows > 0;
  const bool order_in_prefix = !store_rows && prefix_pass && (stages & kStagePrefix) && (stages & kStageOrder);
  if ((stages & kStageOrder) && !order_in_prefix) {  // no-op without an order or rows
    if (store_rows) {
      pa::StoreArgs sa;
      sa.k_new = k_new;
      sa.v_new = v_new;
      sa.slot_mapping = slot_mapping;
      sa.k_pool = pool->k_pool;
      sa.v_pool = pool->v_pool;
      sa.num_rows = num_new_rows;
      sa.row_chunks = pool->num_kv_heads * pool->head_dim * elem_bytes(pool->dtype) / 16;
      st = hip_status(pa::launch_decode_plan_store(plan_args(a), sa, hs));
    } else {
      st = hip_status(pa::launch_decode_plan(plan_args(a), hs));
    }
    if (st != PA_OK) return st;
  }
  // pass 1: each group's shared pages, all members' queries in one tile, and
  // (all stages in one call, no new rows) the work order of pass 2
  if (prefix_pass && (stages & kStagePrefix)) {
    pa::ExtendArgs e = {};
    e.k_pool = pool->k_pool;
    e.v_pool = pool->v_pool;
    e.q = q;
    e.q_indptr = group_starts;
    e.page_table = prefix_page_table;
    e.seq_lens = shared_lens;
    e.o_part = o_part;
    e.lse = lse;
    e.pt_stride = prefix_pt_stride;
    e.num_seqs = num_groups;
    e.num_q_heads = num_q_heads;
    e.num_kv_heads = pool->num_kv_heads;
    e.head_dim = pool->head_dim;
    e.log2_page = ilog2(pool->page_size);
    e.max_q_len = max_group_size;
    e.max_keys = max_shared_len;
    e.piece_keys = pk;
    e.num_pieces = (int32_t)NP;
    e.ws_pieces = (int32_t)(S + NP);
    e.scale_log2 = scale * kLog2e;
    e.plan = plan_args(a);  // its extra work-group writes pass 2's work order
    if (!order_in_prefix) e.plan.plan = nullptr;
    st = hip_status(pa::launch_prefix(e, hs));
    if (st != PA_OK) return st;
  }

  if (stages & kStageSuffix) {
    st = hip_status(pa::launch_decode_partial(a, hs));
    if (st != PA_OK) return st;
  }
  if (stages & kStageCombine) return hip_status(pa::launch_decode_combine(a, hs));
  return PA_OK;
}

}  // namespace

extern "C" {

#define PA_CASCADE_PARAMS                                                                                   \
  const pa_kv_pool *pool, const void *q, int32_t num_q_heads, const int32_t *page_table, int32_t pt_stride, \
      const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len, const int32_t *group_starts,          \
      int32_t num_groups, int32_t max_group_size, const int32_t *prefix_page_table, int32_t prefix_pt_stride, \
      const int32_t *shared_lens, int32_t max_shared_len, float scale, int32_t split_tokens,                 \
      int32_t prefix_piece_keys, const void *k_new, const void *v_new, const int64_t *slot_mapping,          \
      int64_t num_new_rows, void *out, void *workspace, size_t workspace_bytes_, void *stream
#define PA_CASCADE_ARGS                                                                                    \
  pool, q, num_q_heads, page_table, pt_stride, seq_lens, num_seqs, max_seq_len, group_starts, num_groups, \
      max_group_size, prefix_page_table, prefix_pt_stride, shared_lens, max_shared_len, scale, split_tokens, \
      prefix_piece_keys, k_new, v_new, slot_mapping, num_new_rows, out, workspace, workspace_bytes_, stream

pa_status pa_decode_cascade(PA_CASCADE_PARAMS) { return cascade_impl(PA_CASCADE_ARGS, kStageAll); }
pa_status pa_decode_cascade_prefix(PA_CASCADE_PARAMS) { return cascade_impl(PA_CASCADE_ARGS, kStagePrefix); }
pa_status pa_decode_cascade_suffix(PA_CASCADE_PARAMS) { return cascade_impl(PA_CASCADE_ARGS, kStageSuffix); }
pa_status pa_decode_cascade_combine(PA_CASCADE_PARAMS) { return cascade_impl(PA_CASCADE_ARGS, kStageCombine); }
pa_status pa_decode_cascade_order(PA_CASCADE_PARAMS) { return cascade_impl(PA_CASCADE_ARGS, kStageOrder); }

#undef PA_CASCADE_PARAMS
#undef PA_CASCADE_ARGS

pa_status pa_attend_mixed(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* q_indptr,
                          const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t max_q_len, int32_t max_seq_len, float scale, int32_t split_tokens, void* out,
                          void* workspace, size_t workspace_bytes_, void* stream) {
  pa::DecodeArgs a;
  pa_status st = prepare_decode(pool, q, num_q_heads, page_table, pt_stride, seq_lens, num_seqs, max_seq_len,
                                scale, split_tokens, out, workspace, workspace_bytes_, a);
  if (st != PA_OK) return st;
  if (pool->dtype != PA_BF16) return PA_ERR_DTYPE;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G < 1 || G > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (max_q_len < 0 || max_q_len > max_seq_len) return PA_ERR_SHAPE;
  const int64_t qblocks = (max_q_len + 128 / G - 1) / (128 / G);
  if (qblocks * pool->num_kv_heads * num_seqs > (int64_t)INT_MAX) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!q_indptr) return PA_ERR_NULL;
  if (!aligned(out, 16)) return PA_ERR_SHAPE;
  a.q_indptr = q_indptr;
  a.always_partial = 0;
  const hipStream_t hs = (hipStream_t)stream;
  // requests with one new row: split-K decode; the others: matrix-core tiles
  st = enqueue_partial(a, hs);
  if (st != PA_OK) return st;
  if (max_q_len > 1) {
    pa::ExtendArgs e = {};
    e.k_pool = pool->k_pool;
    e.v_pool = pool->v_pool;
    e.q = q;
    e.q_indptr = q_indptr;
    e.page_table = page_table;
    e.seq_lens = seq_lens;
    e.out = out;
    e.pt_stride = pt_stride;
    e.num_seqs = num_seqs;
    e.num_q_heads = num_q_heads;
    e.num_kv_heads = pool->num_kv_heads;
    e.head_dim = pool->head_dim;
    e.log2_page = ilog2(pool->page_size);
    e.max_q_len = max_q_len;
    e.num_pieces = 1;
    e.skip_single = 1;
    e.scale_log2 = scale * kLog2e;
    st = hip_status(pa::launch_extend(e, hs));
    if (st != PA_OK) return st;
  }
  return hip_status(pa::launch_decode_combine(a, hs));
}

size_t pa_verify_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t split_tokens) {
  if (num_seqs < 0 || max_q_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0)
    return 0;
  const int32_t split = resolve_verify_split(split_tokens, max_seq_len);
  if (split < 0) return 0;
  const int64_t S = (max_seq_len + split - 1) / split;
  const size_t rows = (size_t)num_seqs * max_q_len * num_q_heads * (S > 1 ? S : 0);
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}

pa_status pa_verify(const pa_kv_pool* pool, const void* q, int32_t num_q_heads, const int32_t* q_indptr,
                    const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t max_q_len, int32_t max_seq_len, float scale, int32_t split_tokens, void* out,
                    void* workspace, size_t workspace_bytes_, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (pool->dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || max_q_len < 0 || max_seq_len < 0 || pt_stride < 0 || num_q_heads <= 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G < 1 || G > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_q_len * G > 32) return PA_ERR_UNSUPPORTED;  // rows of one matrix-core tile pair
  if (max_q_len > max_seq_len) return PA_ERR_SHAPE;
  if ((int64_t)pt_stride * pool->page_size < max_seq_len) return PA_ERR_SHAPE;
  const int32_t split = resolve_verify_split(split_tokens, max_seq_len);
  if (split < 0) return PA_ERR_SHAPE;
  const int64_t S = (max_seq_len + split - 1) / split;
  if ((int64_t)num_seqs * pool->num_kv_heads * S > (int64_t)INT_MAX) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_q_len == 0 || max_seq_len == 0) return PA_OK;
  if (!q || !q_indptr || !page_table || !seq_lens || !out) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return PA_ERR_SHAPE;
  const size_t need = pa_verify_workspace_bytes(num_seqs, max_q_len, num_q_heads, pool->num_kv_heads,
                                                pool->head_dim, max_seq_len, split);
  if (S > 1 && (workspace_bytes_ < need || !workspace || !aligned(workspace, 256))) return PA_ERR_WORKSPACE;
  const size_t rows = (size_t)num_seqs * max_q_len * num_q_heads * (S > 1 ? S : 0);
  pa::VerifyArgs a = {};
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.q = q;
  a.q_indptr = q_indptr;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.o_part = S > 1 ? (float*)workspace : nullptr;
  a.lse = S > 1 ? (float*)((char*)workspace + align256(rows * pool->head_dim * sizeof(float))) : nullptr;
  a.pt_stride = pt_stride;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.log2_page = ilog2(pool->page_size);
  a.max_q_len = max_q_len;
  a.split_tokens = split;
  a.max_splits = (int32_t)S;
  a.scale_log2 = scale * kLog2e;
  return hip_status(pa::launch_verify(a, (hipStream_t)stream));
}

pa_status pa_check_batch(const pa_kv_pool* pool, const int32_t* page_table, int32_t pt_stride,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len, const int32_t* q_indptr,
                         int32_t max_q_len, const int64_t* slot_mapping, int64_t num_rows, uint32_t* flags,
                         void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || pt_stride < 0 || max_seq_len < 0 || max_q_len < 0 || num_rows < 0) return PA_ERR_SHAPE;
  if (!flags) return PA_ERR_NULL;
  if (!aligned(flags, 4)) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!page_table || !seq_lens)) return PA_ERR_NULL;
  if (num_rows > 0 && !slot_mapping) return PA_ERR_NULL;
  pa::CheckArgs a;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.q_indptr = q_indptr;
  a.slot_mapping = num_rows > 0 ? slot_mapping : nullptr;
  a.flags = flags;
  a.num_pages = pool->num_pages;
  a.num_rows = num_rows;
  a.pt_stride = pt_stride;
  a.num_seqs = num_seqs;
  a.max_seq_len = max_seq_len;
  a.max_q_len = max_q_len;
  a.page_size = pool->page_size;
  return hip_status(pa::launch_check(a, (hipStream_t)stream));
}

pa_status pa_check_cascade(const pa_kv_pool* pool, const int32_t* page_table, int32_t pt_stride,
                           const int32_t* seq_lens, int32_t num_seqs, const int32_t* group_starts,
                           int32_t num_groups, int32_t max_group_size, const int32_t* prefix_page_table,
                           int32_t prefix_pt_stride, const int32_t* shared_lens, int32_t max_shared_len,
                           uint32_t* flags, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || pt_stride < 0 || num_groups < 0 || max_group_size < 0 || prefix_pt_stride < 0 ||
      max_shared_len < 0)
    return PA_ERR_SHAPE;
  if (!flags) return PA_ERR_NULL;
  if (!aligned(flags, 4)) return PA_ERR_SHAPE;
  if (num_seqs > 0 && num_groups > 0 &&
      (!page_table || !seq_lens || !group_starts || !prefix_page_table || !shared_lens))
    return PA_ERR_NULL;
  pa::CascadeCheckArgs a;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.group_starts = group_starts;
  a.prefix_page_table = prefix_page_table;
  a.shared_lens = shared_lens;
  a.flags = flags;
  a.num_pages = pool->num_pages;
  a.pt_stride = pt_stride;
  a.prefix_pt_stride = prefix_pt_stride;
  a.num_seqs = num_seqs;
  a.num_groups = num_groups;
  a.max_group_size = max_group_size;
  a.max_shared_len = max_shared_len;
  a.page_size = pool->page_size;
  return hip_status(pa::launch_check_cascade(a, (hipStream_t)stream));
}

pa_status pa_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0) return PA_ERR_SHAPE;
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return PA_ERR_NULL;
  if (!aligned(src, 16) || bytes % 16 != 0 || !aligned(sink, 4)) return PA_ERR_SHAPE;
  return hip_status(pa::launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

pa_status pa_gather(const pa_kv_pool* pool, const int32_t* page_table, int32_t pt_stride,
                    const int32_t* seq_lens, const int64_t* out_offsets, int32_t num_seqs,
                    int32_t max_seq_len, void* k_out, void* v_out, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_seq_len < 0 || pt_stride < 0) return PA_ERR_SHAPE;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if ((int64_t)pt_stride * pool->page_size < max_seq_len) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_seq_len == 0) return PA_OK;
  if (!page_table || !seq_lens || !out_offsets || !k_out || !v_out) return PA_ERR_NULL;
  if (!aligned(k_out, 16) || !aligned(v_out, 16)) return PA_ERR_SHAPE;
  pa::GatherArgs a;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out_offsets = out_offsets;
  a.k_out = k_out;
  a.v_out = v_out;
  a.pt_stride = pt_stride;
  a.num_seqs = num_seqs;
  a.max_seq_len = max_seq_len;
  a.log2_page = ilog2(pool->page_size);
  a.row_chunks = pool->num_kv_heads * pool->head_dim * elem_bytes(pool->dtype) / 16;
  return hip_status(pa::launch_gather(a, (hipStream_t)stream));
}

}  // extern "C"

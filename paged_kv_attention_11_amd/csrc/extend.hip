// Paged extend attention for gfx950 matrix cores: a chunk of new tokens per
// request (a chunked-prefill piece, or the k+1 tokens of a speculative
// verification) attends the request's cached prefix and, causally, the chunk
// itself, reading K/V straight from the pages.
//
// What is computed (Mini-SGLang README, yangyonggit fork, sections Reference
// Attention Backends -- causal attention with the prefix-cache offset -- and
// Speculative Decoding -- the target model checks all drafted tokens in one
// parallel prefill; nanollmserve README, section v0.7 Chunked Prefill):
//   request b, n_b new tokens after p_b cached keys; new token i (absolute
//   position p_b + i) attends keys j <= p_b + i.
//
// The same kernel (PREFIX mode) computes the shared-prefix pass of the
// cascade decode: its rows are the members of a request group times their
// query heads, its keys the group's shared pages, and it writes split-softmax
// partials that the decode combine kernel merges with each member's own keys.
// On large batches one more work-group of that pass writes the work order of
// the decode kernel that takes the own keys next (plan.h).
//
// Design (FlashAttention-2 style tiling written for the CDNA4 matrix core):
//  * Work-group = 4 waves = 128 query rows = (128 / G) tokens (or group
//    members) x all G query heads of one KV head, so every K/V tile staged in
//    LDS serves G heads (for G = 3, 5, 6, 7 the last 128 mod G rows idle).
//  * Per wave: 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in
//    registers), so each lane owns one query row of the score tile and the
//    softmax needs only one cross-lane exchange (lane ^ 32).  The output is
//    also accumulated transposed, O^T += V^T P^T, so the rescale factor of a
//    query row is lane-local and P goes from the score accumulator to the
//    B operand without leaving registers.
//  * K and V are copied straight from the pages into an LDS ring of 32-key
//    half-tiles with direct-to-LDS loads, a tile ahead, one barrier per
//    64-key tile; two work-groups per compute unit (registers cut to 2 waves
//    per SIMD).  V stays in row layout and is read into the A operand with
//    transposing LDS reads.
//  * Software pipeline over half-tiles: while the vector units run the
//    online softmax of half h, the matrix cores take the scores of half h+1
//    and the PV product of half h-1, interleaved instruction by instruction.
//  * Work-groups are renumbered so that each XCD runs whole (request, head)
//    groups, which read the same keys from its L2.
//  * Key tiles entirely above the diagonal are never visited; only tiles that
//    cross it (or a row's key limit) are masked.
//  * Softmax in fp32 (base 2, scale folded with log2 e); P is rounded to bf16
//    for the matrix core; O accumulates in fp32 and is rounded once.
#include "device.h"
#include "mfma_tile.h"
#include "internal.h"
#include "plan.h"

namespace pa {

namespace {

using namespace tile;

// Work-group shape of the two uses of the kernel.  Every wave owns 32 query
// rows and the waves of a work-group share one LDS ring of K/V.  Both uses
// run 4 waves, two work-groups per compute unit and two waves per SIMD (the
// register budget).  On the Qwen3-8B-shaped chunked-prefill workload an
// earlier, unpipelined version of this kernel measured 251 us with 8 waves
// (256 rows, half the K/V bytes per FLOP) against 243 us with 4: the tile
// traffic is not what bounds the kernel.  The shared-prefix pass needs no
// more: a group of 16 requests x 4 heads is 64 rows.
#ifndef PA_EXTEND_NW
#define PA_EXTEND_NW 4
#endif
template <bool PREFIX>
struct Shape {
  static constexpr int kWaves = PREFIX ? 4 : PA_EXTEND_NW;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRows = kWaves * 32;
};

// Largest row sum (one lane's 16 weights) the usual path of the online
// softmax accepts against its reference; beyond it the reference moves.
constexpr float kMaxRowSum = 65536.0f;

__device__ __forceinline__ int shfl_xor_i(int x, int mask) {
  return __builtin_amdgcn_ds_bpermute((__lane_id() ^ mask) << 2, x);
}

// PREFIX = false: extend (chunk of new tokens, causal after the prefix);
//   SPLIT = true: its keys cut into pieces, partials to the workspace.
// PREFIX = true:  shared-prefix pass of the cascade decode.
template <int D, int G, bool PREFIX, bool SPLIT = false>
__global__ __launch_bounds__(Shape<PREFIX>::kThreads, 2) void mfma_attn_kernel(const ExtendArgs p) {
  using C = ExtCfg<D>;
  using SH = Shape<PREFIX>;
  constexpr int kThreads = SH::kThreads, kWaves = SH::kWaves;
  constexpr int TOK = SH::kRows / G;  // tokens (or group members) per work-group
  constexpr int KSTEPS = C::KSTEPS, DT = C::DT, PPR = C::PPR;
  constexpr int HB = 32 / C::RPB;  // 1 KB DMA blocks per half-tile and tensor
  constexpr int NH = HB / kWaves;  // of them per wave
  static_assert(NH >= 1 && HB % kWaves == 0, "half-tile does not split over the waves");
  constexpr int kHalfBytes = 32 * PPR * 16;

  __shared__ uint4 s_k[4][32 * PPR];
  __shared__ uint4 s_v[4][32 * PPR];
  __shared__ int32_t s_pages[kPageCap];
  __shared__ int32_t s_red[2][kWaves];

  if constexpr (PREFIX) {
    // the extra work-group: the work order of the decode partial kernel
    // that takes each request's own keys next
    if (p.plan.plan && blockIdx.x == gridDim.x - 1) {
      build_decode_plan<SH::kThreads>(p.plan);
      return;
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query row within the wave
  const int half = lane >> 5;
  const int row = wave * 32 + col;  // rows are (head, token/member) with token fastest
  const int hq = row / TOK;
  // when G does not divide the work-group's rows, the last G * TOK .. kRows - 1
  // are padding (no query head): never loaded, never written
  const bool head_ok = hq < G;

  // ---- extend: the requests that run work-groups here (more than one row,
  // or one when single rows are not skipped) first, in order of decreasing
  // key count when there are at most 64 of them, the others after them;
  // with their row ranges, once per work-group (batches of at most
  // kRankMax requests; larger batches keep the request order).
  constexpr int kRankMax = PREFIX ? 1 : kThreads;
  __shared__ int32_t s_req[4][kRankMax];  // at position r: request, first row, rows, keys
  __shared__ int32_t s_cnt[kWaves];
  bool ranked = false;
  int n_active = 0;
  if constexpr (!PREFIX) {
    ranked = p.num_seqs <= kRankMax;
    if (ranked) {
      int rj = 0, nj = 0, lj = 0;
      bool act = false;
      if (tid < p.num_seqs) {
        rj = p.q_indptr[tid];
        nj = p.q_indptr[tid + 1] - rj;
        lj = p.seq_lens[tid];
        act = nj > 1 || (nj == 1 && !p.skip_single);
      }
      // stable partition: active requests first
      const uint64_t bal = __ballot(act);
      const int below = __popcll(bal & ((1ull << lane) - 1));
      if (lane == 0) s_cnt[wave] = __popcll(bal);
      __syncthreads();
      int before = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int c = s_cnt[w];
        before += w < wave ? c : 0;
        n_active += c;
      }
      if (tid < p.num_seqs) {
        const int pos = act ? before + below : n_active + (tid - before - below);
        s_req[0][pos] = tid;
        s_req[1][pos] = rj;
        s_req[2][pos] = nj;
        s_req[3][pos] = lj;
      }
      __syncthreads();
      if (n_active > 1 && n_active <= 64) {  // uniform
        if (wave == 0) {
          int rb = 0, rr = 0, rn = 0, cost = INT_MIN;
          if (lane < n_active) {
            rb = s_req[0][lane];
            rr = s_req[1][lane];
            rn = s_req[2][lane];
            cost = s_req[3][lane];
          }
          int myrank = 0;  // ties keep the partition order
          for (int i = 0; i < n_active; ++i) {  // uniform loop
            const int ci = __builtin_amdgcn_readlane(cost, i);
            const int rank = __popcll(__ballot(cost > ci)) + __popcll(__ballot(cost == ci) & ((1ull << i) - 1));
            if (lane == i) myrank = rank;
          }
          if (lane < n_active) {
            s_req[0][myrank] = rb;
            s_req[1][myrank] = rr;
            s_req[2][myrank] = rn;
            s_req[3][myrank] = cost;
          }
        }
        __syncthreads();
      }
    }
  }

  // ---- the work-group's items.  Extend: logical item ids are (token block
  // qb, request rank, KV head g) with qb fastest and heaviest (latest)
  // first, so consecutive ids of one (request, head) read the same keys.
  // The ids are split into 8 contiguous ranges, one per XCD (work-group i
  // runs on XCD i mod 8); the W work-groups of an XCD take its range in
  // rounds of W, alternating direction, so that a work-group pairs heavy
  // items with light ones.  A grid of one work-group per item takes one
  // round.  Shared-prefix pass: one item per work-group.
  const int xcd = blockIdx.x % 8, kx = blockIdx.x / 8;
  const int wx = ((int)gridDim.x - xcd + 7) / 8;  // work-groups on this XCD
  for (int item = 0;; ++item) {
  int g, q_row, vis_lim, k_begin, k_end, min_vis, piece = 0;
  bool qvalid, has_keys;
  const int32_t* pt;
  if constexpr (!PREFIX) {
    const int qblocks = (p.max_q_len + TOK - 1) / TOK;
    const int NP = SPLIT ? p.num_pieces : 1;  // key pieces per block
    const int total = qblocks * NP * p.num_kv_heads * p.num_seqs;
    const int q8 = total / 8, r8 = total % 8;
    const int nx = q8 + (xcd < r8 ? 1 : 0);
    const int start = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
    const int within = item * wx + ((item & 1) ? wx - 1 - kx : kx);
    if (within >= nx) break;  // uniform
    int bid = start + within;
    const int qb = qblocks - 1 - (bid % qblocks);
    bid /= qblocks;
    if constexpr (SPLIT) {
      piece = bid % NP;
      bid /= NP;
    }
    const int rk = bid % p.num_seqs;
    g = bid / p.num_seqs;
    int b, r0, n, L;
    if (ranked) {
      if (rk >= n_active) {
        // the rest of this head's ids are inactive requests too: go on at
        // the round that reaches the next head's first id
        const int next = (g + 1) * qblocks * NP * p.num_seqs - start;
        if (next >= nx) break;
        item = max(item, next / wx - 1);
        continue;
      }
      b = s_req[0][rk];
      r0 = s_req[1][rk];
      n = s_req[2][rk];
      L = s_req[3][rk];
    } else {
      b = rk;
      r0 = p.q_indptr[b];
      n = p.q_indptr[b + 1] - r0;
      L = p.seq_lens[b];
    }
    const int i0 = qb * TOK;
    if (i0 >= n || (n == 1 && p.skip_single)) continue;  // uniform
    const int prefix = L - n;
    const int kend_blk = prefix + min(i0 + TOK, n);  // keys this block can see
    // piece `piece` of the block's keys (the whole range when not split)
    k_begin = SPLIT ? piece * p.piece_keys : 0;
    if (SPLIT && k_begin >= kend_blk) continue;  // uniform: the block sees no key of this piece
    k_end = SPLIT ? min(k_begin + p.piece_keys, kend_blk) : kend_blk;
    const int ti = i0 + (row % TOK);
    qvalid = head_ok && ti < n;
    q_row = r0 + ti;
    vis_lim = prefix + (qvalid ? ti : (n - 1));  // padding rows mask like the last token
    min_vis = prefix + i0;
    has_keys = true;  // split: decided at the end (rows that see none of the piece write nothing)
    pt = p.page_table + (int64_t)b * p.pt_stride;
  } else {
    // work-group: key piece sp of row block rb of (group j, KV head g)
    if (item > 0) break;
    const int rblocks = (p.max_q_len + TOK - 1) / TOK;
    int bid = blockIdx.x;
    piece = bid % p.num_pieces;
    bid /= p.num_pieces;
    const int rb = bid % rblocks;
    bid /= rblocks;
    g = bid % p.num_kv_heads;
    const int j = bid / p.num_kv_heads;
    const int m_begin = p.q_indptr[j];
    const int gsize = p.q_indptr[j + 1] - m_begin;
    const int m0 = rb * TOK;
    if (m0 >= gsize) break;
    const int mi = m0 + (row % TOK);
    qvalid = head_ok && mi < gsize;
    q_row = m_begin + (qvalid ? mi : m0);
    // clamped so that no key beyond the group's page-table rows is addressed
    const int shared = qvalid ? min(p.seq_lens[q_row], p.max_keys) : 0;
    vis_lim = shared - 1;
    k_begin = piece * p.piece_keys;
    has_keys = qvalid && shared > k_begin;
    // block-wide largest and smallest key limits of the valid rows
    int mx = qvalid ? shared : 0, mn = qvalid ? shared : 0x7fffffff;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      mx = max(mx, shfl_xor_i(mx, m));
      mn = min(mn, shfl_xor_i(mn, m));
    }
    if (lane == 0) {
      s_red[0][wave] = mx;
      s_red[1][wave] = mn;
    }
    __syncthreads();
    mx = s_red[0][0];
    mn = s_red[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      mx = max(mx, s_red[0][w]);
      mn = min(mn, s_red[1][w]);
    }
    if (k_begin >= mx) break;  // no row of the block reads this piece (uniform)
    k_end = min(k_begin + p.piece_keys, mx);
    min_vis = mn - 1;
    pt = p.page_table + (int64_t)j * p.pt_stride;
  }
  const int ntiles = (k_end - k_begin + kKT - 1) / kKT;

  uint4 qreg[KSTEPS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)q_row * p.num_q_heads + (int64_t)g * G + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qreg[ks] = qvalid ? *(const uint4*)(qp + ks * 16 + half * 8) : make_uint4(0, 0, 0, 0);
    // Retire the query loads here, once: after this the registers' last
    // writer is not a memory load, so the loop below carries no wait for them.
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = __builtin_bit_cast(u32x4_t, qreg[ks]);
      asm volatile("" : "+v"(v));
      qreg[ks] = __builtin_bit_cast(uint4, v);
    }
  }

  const int sh = p.log2_page;
  const int pmask = (1 << sh) - 1;
  const int64_t row_stride = (int64_t)p.num_kv_heads * D;  // elements per slot
  const uint16_t* kbase = (const uint16_t*)p.k_pool + (int64_t)g * D;
  const uint16_t* vbase = (const uint16_t*)p.v_pool + (int64_t)g * D;
  const uint32_t k_lds0 = lds_addr(&s_k[0][0]), v_lds0 = lds_addr(&s_v[0][0]);
  const int npages = ((k_end - 1) >> sh) + 1;

  // Page ids of the window of kPageCap pages starting at page `first` into
  // LDS; entries past the block's last page are not read.
  int pwin = k_begin >> sh;
  auto stage_pages = [&](int first) {
    for (int i = tid; i < kPageCap; i += kThreads)
      if (first + i < npages) s_pages[i] = pt[first + i];
  };

  // K/V ring: each tensor holds four 32-key half-tiles, half j of tile t in
  // slot (2t + j) mod 4.  A half is NH 1 KB blocks per wave, one
  // direct-to-LDS load each; lane l of block hb loads piece l mod PPR of key
  // hb RPB + l / PPR of the half, from the swizzled position.  Keys past the
  // block's range are clamped to its last key (a real row; masked out of the
  // softmax).
  int hkey[NH];
  uint32_t kpiece[NH], vpiece[NH];  // byte offsets inside a pool row
#pragma unroll
  for (int m = 0; m < NH; ++m) {
    hkey[m] = (wave * NH + m) * C::RPB + lane / PPR;
    kpiece[m] = (uint32_t)(((lane % PPR) ^ k_swz<D>(hkey[m])) * 16);
    vpiece[m] = (uint32_t)(((lane % PPR) ^ v_swz<D>(hkey[m])) * 16);
  }
  const uint32_t row_bytes = (uint32_t)row_stride * 2u;
  const char* const kb8 = (const char*)kbase;
  const char* const vb8 = (const char*)vbase;
  // byte offsets of the pool rows one half reads: the page lookups first,
  // then one 32 x 32 -> 64-bit product per block
  auto half_rows = [&](int t, int j, uint64_t* off) __attribute__((always_inline)) {
    int kk[NH], pg[NH];
#pragma unroll
    for (int m = 0; m < NH; ++m) kk[m] = min(k_begin + t * kKT + j * 32 + hkey[m], k_end - 1);
#pragma unroll
    for (int m = 0; m < NH; ++m) pg[m] = s_pages[(kk[m] >> sh) - pwin];
#pragma unroll
    for (int m = 0; m < NH; ++m) off[m] = (uint64_t)(uint32_t)((pg[m] << sh) | (kk[m] & pmask)) * row_bytes;
  };
  auto dma_half = [&](const bool is_v, const uint64_t* off, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NH; ++m) {
      const uint32_t lds = (is_v ? v_lds0 : k_lds0) + slot * kHalfBytes + (wave * NH + m) * 1024;
      dma16_unordered(lds, (is_v ? vb8 + vpiece[m] : kb8 + kpiece[m]) + off[m]);
    }
  };
  // Row offsets of halves (t, 1) and (t + 1, 0), computed when their K was
  // issued and used again for their V a tile later.
  uint64_t c1[NH], c0[NH];

  // Issued right after the barrier that opens tile t (of parity u), to land
  // by the next one: V(t, 1), K(t+1, 1), V(t+1, 0)
  // and K(t+2, 0).  Their slots are the four the steps of tile t do not
  // read, so the loads past the last tile (clamped keys, never read) are
  // issued too and the issue has no branch.
  auto slide_window = [&](int t) __attribute__((always_inline)) {
    const int kmax = min(k_begin + (t + 2) * kKT + 31, k_end - 1);  // no key looked up now is larger
    if ((kmax >> sh) - pwin >= kPageCap) {  // block-uniform and rare
      pwin = (k_begin + t * kKT + 32) >> sh;  // the smallest key looked up now
      stage_pages(pwin);
      __syncthreads();
    }
  };
  auto issue_after = [&](int t, const int u) __attribute__((always_inline)) {
    uint64_t n1[NH], n0[NH];
    half_rows(t + 1, 1, n1);
    half_rows(t + 2, 0, n0);
    dma_half(true, c1, (2 * u + 1) & 3);
    dma_half(false, n1, (2 * u + 3) & 3);
    dma_half(true, c0, (2 * u + 2) & 3);
    dma_half(false, n0, (2 * u) & 3);
#pragma unroll
    for (int m = 0; m < NH; ++m) {
      c1[m] = n1[m];
      c0[m] = n0[m];
    }
  };

  f32x16_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_ref = -INFINITY;  // reference maximum of this row's raw scores
  float l_run = 0.f;        // this lane's half of the running sum
  const float sl2 = p.scale_log2;

  // Per-lane LDS byte offsets inside a half-tile slot, computed once.  K
  // piece (2 ks + half) ^ (key mod PPR) of key col sits at koff[ks]; the
  // transposing V read of step (k2, r) and head-dim block i sits at
  // 16 k2 PPR 16 + 8 r PPR 16 + voff[i].  With a compile-time slot the rest
  // of each LDS address is an instruction's immediate offset.
  uint32_t koff[KSTEPS], voff[DT];
  {
    const int ck = col & (PPR - 1);
    const int kb = col * PPR * 16 + 16 * (half ^ (ck & 1));
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) koff[ks] = kb + 32 * (ks ^ (ck >> 1));
    const int j = lane & 15, g1 = (lane >> 4) & 1;
    const int sv = v_swz<D>(4 * half + (j >> 2));  // the keys read here, mod 8
    const int pl = (4 * half + (j >> 2)) * PPR * 16 + 8 * (j & 1) + 16 * ((2 * g1 + ((j >> 1) & 1)) ^ (sv & 3));
#pragma unroll
    for (int i = 0; i < DT; ++i) voff[i] = pl + 64 * (i ^ (sv >> 2));
  }
  const char* const k_lds = (const char*)&s_k[0][0];
  const char* const v_lds = (const char*)&s_v[0][0];

  // S^T = K Q^T for the 32 keys of one half-tile slot (the first k-step
  // accumulates onto the inline constant 0)
  auto qk = [&](const int slot) __attribute__((always_inline)) {
    const char* kp = k_lds + slot * kHalfBytes;
    f32x16_t sc = mfma32(*(const uint4*)(kp + koff[0]), qreg[0], f32x16_t{});
#pragma unroll
    for (int ks = 1; ks < KSTEPS; ++ks) sc = mfma32(*(const uint4*)(kp + koff[ks]), qreg[ks], sc);
    return sc;
  };
  // O^T += V^T P^T for one half-tile slot.  The A operand is read transposed
  // out of row-major V: lane (group of 16, j) reads keys 16 k2 + 8 r +
  // 4 half + j/4, head-dims d0 + 4 (j mod 4) .. +3 and receives
  // V[4 keys][d0 + j].
  auto pv = [&](const uint4* pb, const int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const char* vp = v_lds + slot * kHalfBytes + k2 * 16 * PPR * 16 + voff[i];
        const uint2 x0 = lds_read_tr16(vp);
        const uint2 x1 = lds_read_tr16(vp + 8 * PPR * 16);
        o[i] = mfma32(make_uint4(x0.x, x0.y, x1.x, x1.y), pb[k2], o[i]);
      }
  };

  // ---- prologue: page ids; K(0, *), K(1, 0) and V(0, 0) in, the V slot of
  // the (empty) half before the first zeroed; scores of half (0, 0)
  stage_pages(pwin);
  for (int i = tid; i < 32 * PPR; i += kThreads) s_v[3][i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  {
    uint64_t h00[NH];
    half_rows(0, 0, h00);
    half_rows(0, 1, c1);
    half_rows(1, 0, c0);  // clamped keys when there is one tile
    dma_half(false, h00, 0);
    dma_half(false, c1, 1);
    dma_half(true, h00, 0);
    if (ntiles > 1) dma_half(false, c0, 2);
  }
  vm_wait<0>();
  __syncthreads();
  f32x16_t s_cur = qk(0);
  uint4 pp[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};  // P of the previous half
  __syncthreads();  // K slot 0 is refilled next

  // One pipeline step on half (t, j), whose scores are in s_cur: its online
  // softmax on the vector units while the matrix cores take the next half's
  // scores (K slot kslot) and the previous half's product (V slot vslot).
  //
  // Weights are taken against a per-row reference m_ref, not the running
  // maximum: any reference gives the same normalised result as long as the
  // weights stay in range.  The usual path therefore skips the row maximum
  // and only checks the row sum it forms anyway: a sum above 2^16 (or not
  // finite -- the first half, when no reference exists yet) sends the wave
  // to the exact path, which moves the reference to the row maximum,
  // rescales O and the sum (after the previous half's product, weighted
  // against the old reference) and forms the weights again.  A row with no
  // visible key yet takes reference 0; its weights are exp2(-inf) = 0.
  auto step = [&](const bool masked, const int t, const int j, const int kslot, const int vslot)
                  __attribute__((always_inline)) {
    if (masked) {  // block-uniform; only on halves that reach past a row's last key
      const int kb = k_begin + t * kKT + j * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb + 8 * (r >> 2) + 4 * half + (r & 3) > vis_lim) s_cur[r] = -INFINITY;
    }
    constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
    // weights against reference m, rounded for the product; the row sum
    // (this lane's half) takes them as rounded
    auto weigh = [&](float m, uint4& w0, uint4& w1) __attribute__((always_inline)) {
      const float mb = -m * sl2;
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(s_cur[r], sl2, mb));
      w0 = make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
      w1 = make_uint4(pack2(e[8], e[9]), pack2(e[10], e[11]), pack2(e[12], e[13]), pack2(e[14], e[15]));
      float sum = dot2_bf16(w0.x, kOnes, 0.f);
      sum = dot2_bf16(w0.y, kOnes, sum);
      sum = dot2_bf16(w0.z, kOnes, sum);
      sum = dot2_bf16(w0.w, kOnes, sum);
      sum = dot2_bf16(w1.x, kOnes, sum);
      sum = dot2_bf16(w1.y, kOnes, sum);
      sum = dot2_bf16(w1.z, kOnes, sum);
      return dot2_bf16(w1.w, kOnes, sum);
    };
    uint4 pc0, pc1;
    float ls = weigh(m_ref, pc0, pc1);

    // matrix-core work, the two chains alternating: k-step k of the next
    // half's scores, then product step k of the previous half (head-dim
    // block k / 2, 16-key step k mod 2)
    static_assert(KSTEPS == 2 * DT, "one product step per score k-step");
    const char* kp = k_lds + kslot * kHalfBytes;
    f32x16_t s_nxt;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const uint4 ka = *(const uint4*)(kp + koff[k]);
      s_nxt = k == 0 ? mfma32(ka, qreg[0], f32x16_t{}) : mfma32(ka, qreg[k], s_nxt);
      const int i = k >> 1, k2 = k & 1;
      const char* vp = v_lds + vslot * kHalfBytes + k2 * 16 * PPR * 16 + voff[i];
      const uint2 x0 = lds_read_tr16(vp);
      const uint2 x1 = lds_read_tr16(vp + 8 * PPR * 16);
      o[i] = mfma32(make_uint4(x0.x, x0.y, x1.x, x1.y), pp[k2], o[i]);
    }
    // Order: the operands of the first two MFMA pairs, then each MFMA
    // followed by the LDS reads (three per pair, issued two pairs ahead) and
    // the vector work that fit under it.
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // vector ALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // vector ALU
    }
    // the weights are formed before the (rare) exact path below
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, pc0)), "v"(__builtin_bit_cast(u32x4_t, pc1)), "v"(ls));
    if (__ballot(!(ls <= kMaxRowSum)) != 0) {  // wave-uniform
      float mx = s_cur[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
      {  // lanes l and l ^ 32 hold the two halves of a row: swap and take both
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      float m_new = fmaxf(m_ref, mx);
      if (m_new == -INFINITY) m_new = 0.f;  // no visible key yet
      const float alpha = fast_exp2((m_ref - m_new) * sl2);  // 0 when there was no reference
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      ls = weigh(m_ref, pc0, pc1);
    }
    l_run += ls;
    pp[0] = pc0;
    pp[1] = pc1;
    s_cur = s_nxt;
  };

  for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + u;
      if (t >= ntiles) break;
      slide_window(t);
      issue_after(t, u);
      const int kt0 = k_begin + t * kKT;
      // half (t, 0): scores of (t, 1), product of (t - 1, 1)
      step(kt0 + 31 > min_vis, t, 0, 2 * u + 1, (2 * u + 3) & 3);
      // half (t, 1): scores of (t + 1, 0) (unused after the last tile),
      // product of (t, 0)
      step(kt0 + kKT - 1 > min_vis, t, 1, (2 * u + 2) & 3, 2 * u);
      // this tile's DMA has landed everywhere and its slots' readers are done
      vm_wait<0>();
      __syncthreads();
    }
  }
  pv(pp, (2 * ntiles - 1) & 3);  // product of the last half

  // ---- normalise and write this lane's row
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if constexpr (!PREFIX) {
    if constexpr (SPLIT) {
      // split keys: the piece's normalised output and log2-sum-exp, merged
      // by extend_combine_kernel
      if (qvalid && vis_lim >= k_begin) {
        const float inv = 1.f / l_tot;
        const int64_t part_row = ((int64_t)q_row * p.num_q_heads + (int64_t)g * G + hq) * p.num_pieces + piece;
        float* op = p.o_part + part_row * D;
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d = i * 32 + 8 * q4 + 4 * half;
            *(float4*)(op + d) = make_float4(o[i][4 * q4 + 0] * inv, o[i][4 * q4 + 1] * inv,
                                             o[i][4 * q4 + 2] * inv, o[i][4 * q4 + 3] * inv);
          }
        if (half == 0) p.lse[part_row] = m_ref * sl2 + __log2f(l_tot);
      }
    } else if (qvalid) {
    const float inv = 1.f / l_tot;
    uint16_t* op = (uint16_t*)p.out + ((int64_t)q_row * p.num_q_heads + (int64_t)g * G + hq) * D;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = i * 32 + 8 * q4 + 4 * half;
        uint2 w;
        w.x = pack2(o[i][4 * q4 + 0] * inv, o[i][4 * q4 + 1] * inv);
        w.y = pack2(o[i][4 * q4 + 2] * inv, o[i][4 * q4 + 3] * inv);
        *(uint2*)(op + d) = w;
      }
    }
  } else {
    // the combine kernel reads this piece for a member only if the member
    // has keys in it
    if (has_keys) {
    const float inv = 1.f / l_tot;
    const int64_t wrow = ((int64_t)q_row * p.num_q_heads + (int64_t)g * G + hq) * p.ws_pieces + piece;
    float* op = p.o_part + wrow * D;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = i * 32 + 8 * q4 + 4 * half;
        *(float4*)(op + d) = make_float4(o[i][4 * q4 + 0] * inv, o[i][4 * q4 + 1] * inv,
                                         o[i][4 * q4 + 2] * inv, o[i][4 * q4 + 3] * inv);
      }
    if (half == 0) p.lse[wrow] = m_ref * sl2 + __log2f(l_tot);
    }
  }
  __syncthreads();  // the next item refills the LDS
  }  // items
}

// Split extend: one wave per (request b, row i < max_q_len, query head)
// merges the key pieces of that row (workspace row: query row r0 + i, head).  Row i of request b sees
// p_b + i + 1 keys, so it has ceil((p_b + i + 1) / piece_keys) pieces, each
// with at least one visible key (written by the extend kernel); their
// log-sum-exps are read one per lane and the partial outputs in batches of
// eight independent loads.
template <int D>
__global__ __launch_bounds__(256) void extend_combine_kernel(const ExtendArgs p) {
  constexpr int EPL = D / 64;
  constexpr int BATCH = 8;
  constexpr int kFew = 8;  // rows of at most this many pieces take the one-round-trip path
  const int lane = threadIdx.x & 63;
  const int64_t R = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.num_seqs * p.max_q_len * p.num_q_heads;
  if (R >= rows) return;
  const int hq = (int)(R % p.num_q_heads);
  const int64_t bi = R / p.num_q_heads;
  const int i = (int)(bi % p.max_q_len);
  const int b = (int)(bi / p.max_q_len);
  const int r0 = p.q_indptr[b];
  const int n = p.q_indptr[b + 1] - r0;
  if (i >= n) return;
  const int vis = p.seq_lens[b] - n + i + 1;  // keys row i sees
  const int ns = min((vis + p.piece_keys - 1) / p.piece_keys, p.num_pieces);
  const int64_t wrow = ((int64_t)(r0 + i) * p.num_q_heads + hq) * p.num_pieces;  // the row's pieces
  const float* lse = p.lse + wrow;
  const float* op = p.o_part + wrow * D + lane * EPL;
  uint16_t* out = (uint16_t*)p.out + ((int64_t)(r0 + i) * p.num_q_heads + hq) * D + lane * EPL;

  if (ns > 0 && ns <= kFew) {
    // every load issued at once: the log-sum-exps (lane k: piece k) and the
    // partial outputs do not depend on each other, so the merge waits for
    // one memory round trip instead of two.  Same order of operations as
    // the general path below.
    const float l = lane < ns ? lse[lane] : -INFINITY;
    float v[kFew][EPL];
#pragma unroll
    for (int k = 0; k < kFew; ++k) {
      if (k < ns) {  // uniform
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[k][e] = op[(int64_t)k * D + e];
      }
    }
    const float M = wave_max(l);
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    if (M != -INFINITY) {
      const float w = (lane < ns && l != -INFINITY) ? fast_exp2(l - M) : 0.f;
      const float wsum = wave_sum(w);
#pragma unroll
      for (int k = 0; k < kFew; ++k) {
        if (k < ns) {  // uniform
          const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[e] = wk > 0.f ? fmaf(wk, v[k][e], o[e]) : o[e];
        }
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] /= wsum;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = (uint16_t)f32_to_bf16_bits(o[e]);
    return;
  }

  float M = -INFINITY;
  for (int c = 0; c < ns; c += 64) M = fmaxf(M, lse[min(c + lane, ns - 1)]);
  M = wave_max(M);
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  if (ns > 0 && M != -INFINITY) {
    float wsum = 0.f;
    for (int c = 0; c < ns; c += 64) {
      const float l = lse[min(c + lane, ns - 1)];
      const float w = (c + lane < ns && l != -INFINITY) ? fast_exp2(l - M) : 0.f;
      wsum += w;
      const int cnt = min(64, ns - c);
      for (int j0 = 0; j0 < cnt; j0 += BATCH) {
        float wk[BATCH], v[BATCH][EPL];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const int j = min(j0 + k, cnt - 1);  // clamped: a real piece, weight zero below
          wk[k] = j0 + k < cnt ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j))
                               : 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[k][e] = op[(int64_t)(c + j) * D + e];
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k)
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[e] = wk[k] > 0.f ? fmaf(wk[k], v[k][e], o[e]) : o[e];
      }
    }
    wsum = wave_sum(wsum);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] /= wsum;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = (uint16_t)f32_to_bf16_bits(o[e]);
}

template <int D, int G, bool PREFIX, bool SPLIT>
hipError_t launch_g(const ExtendArgs& a, hipStream_t stream) {
  constexpr int TOK = Shape<PREFIX>::kRows / G;
  const int64_t blocks_per = (a.max_q_len + TOK - 1) / TOK;
  int64_t blocks = blocks_per * a.num_kv_heads * a.num_seqs * a.num_pieces;
  if (blocks == 0) return hipSuccess;
  if (!PREFIX) {
    // Up to four chip-fulls of items, one work-group per item: the
    // dispatcher balances them as slots free up.  Beyond that (typically a
    // batch of mostly single-row requests, whose items are empty), two
    // work-groups per compute unit (what fits at once, a multiple of the 8
    // XCDs) each take their share of the items and skip the empty ones
    // without a launch each.
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t cap = (int64_t)(2 * cus) / 8 * 8;
    if (cap >= 8 && blocks > 4 * cap) blocks = cap;
  }
  if (PREFIX && a.plan.plan) ++blocks;  // the work-group that writes the decode work order
  hipLaunchKernelGGL((mfma_attn_kernel<D, G, PREFIX, SPLIT>), dim3((unsigned)blocks), dim3(Shape<PREFIX>::kThreads),
                     0, stream, a);
  hipError_t e = hipGetLastError();
  if (!SPLIT || e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.num_seqs * a.max_q_len * a.num_q_heads;
  hipLaunchKernelGGL((extend_combine_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool PREFIX, bool SPLIT>
hipError_t launch_d(const ExtendArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<D, 1, PREFIX, SPLIT>(a, stream);
    case 2: return launch_g<D, 2, PREFIX, SPLIT>(a, stream);
    case 3: return launch_g<D, 3, PREFIX, SPLIT>(a, stream);
    case 4: return launch_g<D, 4, PREFIX, SPLIT>(a, stream);
    case 5: return launch_g<D, 5, PREFIX, SPLIT>(a, stream);
    case 6: return launch_g<D, 6, PREFIX, SPLIT>(a, stream);
    case 7: return launch_g<D, 7, PREFIX, SPLIT>(a, stream);
    case 8: return launch_g<D, 8, PREFIX, SPLIT>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream) {
  const bool split = a.num_pieces > 1;
  if (a.head_dim == 128) return split ? launch_d<128, false, true>(a, stream) : launch_d<128, false, false>(a, stream);
  if (a.head_dim == 64) return split ? launch_d<64, false, true>(a, stream) : launch_d<64, false, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefix(const ExtendArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128, true, false>(a, stream);
  if (a.head_dim == 64) return launch_d<64, true, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

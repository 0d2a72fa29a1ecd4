// Parallel verification of drafted tokens: every request brings a short
// chunk of n new rows (k drafted tokens + 1, a handful) that attends its whole
// cached context causally.  The target model verifies the k tokens in one
// parallel prefill rather than k decodes (Mini-SGLang README, yangyonggit
// fork, section Speculative Decoding), so the rows of a request are few and
// its keys many: the work is shaped like decode, not like prefill.
//
// Design:
//  * Split-K like decode: work-group = (piece s of split_tokens keys,
//    request b, KV head or pair of KV heads); the pieces are merged by
//    verify_combine_kernel with log-sum-exp weights.  Pieces are dispatched
//    longest first (longest_first_piece).
//  * The n rows x G query heads of (b, g) (at most 32, row = i G + h) are
//    the N dimension of two 16-row matrix-core tiles, so each K/V byte is
//    read once for all of them: S^T = K Q^T with v_mfma_f32_16x16x32_bf16,
//    and O^T += V^T P^T with the same instruction over a chunk's 32 keys,
//    whose B operand (keys x rows) is the two score tiles' accumulators side
//    by side, so P never leaves registers.
//  * Each wave streams its own 32-key chunks of the piece (chunk c to wave
//    c mod W of the head's W waves) with its own online softmax; the W
//    partial results of a head are merged through LDS at the end, so the key
//    loop has no work-group barrier.  A chunk's K and V rows are loaded whole
//    (16-byte pieces, a load instruction covering four 256-byte rows) into
//    registers with nontemporal loads one chunk ahead, written to the wave's
//    own LDS slot and read back in the operand layouts (V^T with the
//    transposing LDS read).  Within a wave the slot needs no barrier: a
//    wave's LDS instructions execute in the order it issues them.
//  * Row (token i, head h) sees keys <= L - n + i; only the chunks that
//    reach past L - n are masked.
#include "device.h"
#include "internal.h"
#include "mfma_tile.h"

namespace pa {

namespace {

using namespace tile;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = kTileThreads;
constexpr float kSlack = 8.0f;  // log2 units: rescale only when the maximum grows by more

__device__ __forceinline__ f32x4_t mfma16_k32(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Longest-first work order for batches of at most 64 requests: position
// `pos` of a KV-head block takes every full piece (split_tokens keys) first,
// piece index slowest, then the shorter last pieces by decreasing key count
// (ties in request order).  Returns false past the last existing piece: the
// grid covers every possible piece (max_splits per request), and the
// work-groups with nothing to do all come at the end of the dispatch order
// instead of holding slots between the others.  On the Qwen3-8B-shaped
// verify workload (64 requests, 1024-key pieces) 135-140 us in this order
// against 148-154 us with the existing pieces taken piece index slowest
// regardless of length.  Lane j holds request j; every lane of the wave
// calls this.
__device__ __forceinline__ bool longest_first_piece(const VerifyArgs& p, int pos, int lane, int& s, int& b) {
  int nfull = 0, rem = -1;
  if (lane < p.num_seqs && p.q_indptr[lane + 1] - p.q_indptr[lane] > 0) {
    const int lj = p.seq_lens[lane];
    nfull = lj / p.split_tokens;
    rem = lj - nfull * p.split_tokens;
    if (rem == 0) rem = -1;  // no shorter last piece
  }
  s = -1;
  b = 0;
  int before = 0;  // full pieces of the lower piece indices
  for (int sp = 0; sp < p.max_splits; ++sp) {  // uniform loop
    const uint64_t have = __ballot(nfull > sp);
    const int c = __popcll(have);
    if (c == 0) break;
    if (pos < before + c) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(have >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)have, 0u));
      s = sp;
      b = __builtin_ctzll(__ballot(nfull > sp && below == pos - before));
      break;
    }
    before += c;
  }
  if (s < 0) {
    const int q = pos - before;  // rank among the last pieces
    int rank = 0;                // this lane's rank
    for (int i = 0; i < p.num_seqs; ++i) {  // uniform loop
      const int ri = __builtin_amdgcn_readlane(rem, i);
      rank += (ri > rem || (ri == rem && i < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(rem >= 0 && rank == q);
    if (hit == 0) return false;  // uniform: past the last existing piece
    b = __builtin_ctzll(hit);
    s = __builtin_amdgcn_readlane(nfull, b);
  }
  return true;
}

// HP: KV heads per work-group (1 or 2): the four waves serve HP heads, 4 / HP
// waves each, so with two the loads of a key's two head slices (512
// contiguous bytes of its pool row) are issued at about the same time.
template <int D, int G, int HP>
__global__ __launch_bounds__(kThreads, 2) void verify_kernel(const VerifyArgs p) {
  using C = ExtCfg<D>;
  constexpr int PPR = C::PPR;
  constexpr int KS = D / 32;         // k-steps of S^T
  constexpr int DC = D / 16;         // 16-wide head-dim tiles of O^T
  constexpr int WPH = 4 / HP;        // waves per KV head
  constexpr int CK = 32;             // keys per chunk
  constexpr int KPL = 64 / PPR;      // keys per load instruction (whole rows)
  constexpr int NV = CK / KPL;       // K (and V) loads per lane per chunk
  constexpr int SLOT = 2 * CK * PPR;  // uint4 per wave: a K and a V chunk, or its O^T (32 rows x D fp32) at the end
  static_assert(HP == 1 || HP == 2, "bad shape");
  static_assert(SLOT * 16 == 32 * D * 4, "slot holds a wave's O^T");

  __shared__ uint4 s_buf[kThreads / 64][SLOT];
  __shared__ int32_t s_pages[kVerifyMaxSplit];  // a piece's page ids (one key per page at page size 1)
  __shared__ float s_m[kThreads / 64][32];
  __shared__ float s_l[kThreads / 64][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int hh = wave / WPH;  // head of the block
  const int sw = wave % WPH;  // this wave's share of the chunks

  // work-group -> (piece s, request b, KV head block); the KV head block is
  // the fastest index, so each XCD gets the same share of every piece
  const int nhb = p.num_kv_heads / HP;
  const int gb = blockIdx.x % nhb;
  const int g = gb * HP + hh;
  const int pos = blockIdx.x / nhb;
  int s, b;
  if (p.num_seqs <= 64) {
    if (!longest_first_piece(p, pos, lane, s, b)) return;  // uniform
  } else {
    s = pos / p.num_seqs;
    b = pos - s * p.num_seqs;
  }
  const int r0 = p.q_indptr[b];
  const int n = p.q_indptr[b + 1] - r0;
  const int L = p.seq_lens[b];
  const int k_begin = s * p.split_tokens;
  if (n <= 0 || k_begin >= L) return;  // uniform over the work-group
  const int k_end = min(k_begin + p.split_tokens, L);
  const int prefix = L - n;
  const int nq = min(n, p.max_q_len);
  const int ns = (L + p.split_tokens - 1) / p.split_tokens;
  const int nch = (k_end - k_begin + CK - 1) / CK;

  // ---- queries: row = i * G + h in two 16-row tiles; this lane supplies row
  // 16 rt + l16 of tile rt's B operand, head dims 32 ks + 8 grp .. + 7
  uint4 qreg[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = rt * 16 + l16;
    const int i = row / G, h = row % G;
    const bool ok = i < nq;
    const uint16_t* qp =
        (const uint16_t*)p.q + ((int64_t)(r0 + (ok ? i : 0)) * p.num_q_heads + (int64_t)g * G + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[rt][ks] = ok ? *(const uint4*)(qp + 32 * ks + 8 * grp) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = __builtin_bit_cast(u32x4_t, qreg[rt][ks]);
      asm volatile("" : "+v"(v));
      qreg[rt][ks] = __builtin_bit_cast(uint4, v);
    }

  // ---- page ids of the piece (at most kVerifyMaxSplit keys, so pages)
  const int sh = p.log2_page;
  const int pmask = (1 << sh) - 1;
  const int pg0 = k_begin >> sh;
  const int npg = ((k_end - 1) >> sh) - pg0 + 1;
  {
    const int32_t* pt = p.page_table + (int64_t)b * p.pt_stride + pg0;
    for (int i = tid; i < npg; i += kThreads) s_pages[i] = pt[i];
  }
  __syncthreads();

  const uint32_t row_bytes = (uint32_t)p.num_kv_heads * D * 2u;
  const char* const kb8 = (const char*)p.k_pool + (int64_t)g * D * 2;
  const char* const vb8 = (const char*)p.v_pool + (int64_t)g * D * 2;
  // byte offset of a key's pool row; keys past the piece are clamped to its
  // last key (a real row, masked out of the softmax)
  auto row_off = [&](int key) __attribute__((always_inline)) {
    const int kk = min(key, k_end - 1);
    const int32_t page = s_pages[(kk >> sh) - pg0];
    return (uint64_t)(uint32_t)((page << sh) | (kk & pmask)) * row_bytes;
  };
  // Chunk c's K and V, whole rows: load m covers keys m KPL .. + KPL - 1, lane
  // l piece l % PPR of key m KPL + l / PPR.  Past the wave's last chunk every
  // key clamps to the piece's last key: the loads are issued anyway (one row,
  // the values never used), so that no load sits under a branch -- the
  // compiler's waits would then also count the next chunk's loads.
  uint4 kreg[NV], vreg[NV];
  auto load_kv = [&](int c) __attribute__((always_inline)) {
    const int kb = k_begin + c * CK;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const uint64_t off = row_off(kb + m * KPL + lane / PPR) + 16 * (lane % PPR);
      kreg[m] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(kb8 + off)));
      vreg[m] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(vb8 + off)));
    }
  };
  // the wave's LDS slot: K rows (pieces XOR key mod PPR), then V rows
  uint4* const kslot = &s_buf[wave][0];
  uint4* const slot = &s_buf[wave][CK * PPR];

  f32x4_t o[DC][2];  // O^T tile (dc, rt): lane holds d = 16 dc + 4 grp + r of row 16 rt + l16
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) o[dc][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-INFINITY, -INFINITY};  // raw-score reference maximum of this lane's rows
  float l_run[2] = {0.f, 0.f};              // this lane's part of the row sums
  const float sl2 = p.scale_log2;
  const float slack = kSlack / sl2;

  load_kv(sw);
  for (int c = sw; c < nch; c += WPH) {
    // this chunk into the wave's slot, row = key, swizzled as the reads below
    // expect
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int kr = m * KPL + lane / PPR;
      kslot[kr * PPR + ((lane % PPR) ^ k_swz<D>(kr))] = kreg[m];
      slot[kr * PPR + ((lane % PPR) ^ v_swz<D>(kr))] = vreg[m];
    }
    load_kv(c + WPH);  // the next chunk of this wave, loaded meanwhile
    asm volatile("" ::: "memory");  // the slot's stores stay before its reads

    // ---- S^T: tile (j, rt), lane holds keys 16 j + 4 grp + r of row 16 rt + l16
    f32x4_t sacc[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        sacc[j][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int kr = 16 * j + l16;
          sacc[j][rt] = mfma16_k32(kslot[kr * PPR + ((4 * ks + grp) ^ k_swz<D>(kr))], qreg[rt][ks], sacc[j][rt]);
        }
      }

    // ---- causal mask and the keys past the piece, on the last chunks only
    const int kt0 = k_begin + c * CK;
    if (kt0 + CK - 1 > prefix || kt0 + CK > k_end) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int i = (rt * 16 + l16) / G;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kt0 + 16 * j + 4 * grp + r;
            if (key > prefix + i || key >= k_end) sacc[j][rt][r] = -INFINITY;
          }
      }
    }

    // ---- online softmax per row tile; the four lane groups hold the row's keys
    uint2 pb[2][2];  // P^T B operands: keys 16 j + 4 grp .. + 3 of row 16 rt + l16
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][rt][0], sacc[0][rt][1]), fmaxf(sacc[0][rt][2], sacc[0][rt][3])),
                       fmaxf(fmaxf(sacc[1][rt][0], sacc[1][rt][1]), fmaxf(sacc[1][rt][2], sacc[1][rt][3])));
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      if (__ballot(mx > m_ref[rt] + slack) != 0) {
        const float m_new = fmaxf(m_ref[rt], mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_ref[rt] - m_new) * sl2);
        m_ref[rt] = m_new;
        l_run[rt] *= alpha;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) o[dc][rt] *= alpha;
      }
      const float mb = m_ref[rt] == -INFINITY ? 0.f : -m_ref[rt] * sl2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = fast_exp2(fmaf(sacc[j][rt][r], sl2, mb));
          l_run[rt] += e[r];
        }
        pb[j][rt] = make_uint2(pack2(e[0], e[1]), pack2(e[2], e[3]));
      }
    }

    // ---- O^T += V^T P^T: lane (grp, l16) addresses key 16 j + 4 grp + l16/4,
    // dims 16 dc + 4 (l16 % 4) .. + 3, and receives V[4 keys][16 dc + l16]
    {
      const char* vb = (const char*)slot;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int d = 16 * dc + 4 * (l16 & 3);
        const int lp = d >> 3;
        const int within = (d & 4) ? 8 : 0;
        uint2 x[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kr = 16 * j + 4 * grp + (l16 >> 2);
          x[j] = lds_read_tr16(vb + (kr * PPR + (lp ^ v_swz<D>(kr))) * 16 + within);
        }
        // one 32-key product: k-elements 0..3 of lane group grp are keys
        // 4 grp + r, 4..7 keys 16 + 4 grp + r, in A and in B alike
        const uint4 a = make_uint4(x[0].x, x[0].y, x[1].x, x[1].y);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          o[dc][rt] = mfma16_k32(a, make_uint4(pb[0][rt].x, pb[0][rt].y, pb[1][rt].x, pb[1][rt].y), o[dc][rt]);
      }
    }
    asm volatile("" ::: "memory");  // and before the next chunk's stores
  }

  // ---- merge the WPH waves of each head: reference maxima and sums per row,
  // then each wave sums its share of the O^T tiles
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    l_run[rt] += shfl_xor_f(l_run[rt], 16);
    l_run[rt] += shfl_xor_f(l_run[rt], 32);
    if (grp == 0) {
      s_m[wave][rt * 16 + l16] = m_ref[rt];
      s_l[wave][rt * 16 + l16] = l_run[rt];
    }
  }
  {
    f32x4_t* ob = (f32x4_t*)kslot;  // the whole slot, K and V parts
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) ob[(dc * 2 + rt) * 64 + lane] = o[dc][rt];
  }
  __syncthreads();

  float M[2], inv[2], lse[2], wgt[2][WPH];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = rt * 16 + l16;
    float mw[WPH];
    M[rt] = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPH; ++w) {
      mw[w] = s_m[hh * WPH + w][row];
      M[rt] = fmaxf(M[rt], mw[w]);
    }
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < WPH; ++w) {
      wgt[rt][w] = mw[w] == -INFINITY ? 0.f : fast_exp2((mw[w] - M[rt]) * sl2);
      Lt += wgt[rt][w] * s_l[hh * WPH + w][row];
    }
    const bool seen = M[rt] != -INFINITY;  // false: no key of this piece is visible to the row
    inv[rt] = seen ? 1.f / Lt : 0.f;
    lse[rt] = seen ? M[rt] * sl2 + __log2f(Lt) : -INFINITY;
  }

  // tiles bi = 2 dc + rt with bi mod WPH == sw
  const int64_t head0 = (int64_t)g * G;
#pragma unroll
  for (int bi = 0; bi < 2 * DC; ++bi) {
    if (bi % WPH != sw) continue;  // wave-uniform
    const int dc = bi >> 1, rt = bi & 1;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < WPH; ++w) acc += wgt[rt][w] * ((const f32x4_t*)&s_buf[hh * WPH + w][0])[bi * 64 + lane];
    const int row = rt * 16 + l16;
    const int i = row / G, h = row % G;
    if (i >= nq) continue;
    const int d = 16 * dc + 4 * grp;
    const float iv = inv[rt];
    if (ns == 1) {
      uint16_t* op = (uint16_t*)p.out + ((int64_t)(r0 + i) * p.num_q_heads + head0 + h) * D;
      *(uint2*)(op + d) = make_uint2(pack_bf16x2(acc[0] * iv, acc[1] * iv), pack_bf16x2(acc[2] * iv, acc[3] * iv));
    } else {
      const int64_t wr = (((int64_t)b * p.max_q_len + i) * p.num_q_heads + head0 + h) * p.max_splits + s;
      *(float4*)(p.o_part + wr * D + d) = make_float4(acc[0] * iv, acc[1] * iv, acc[2] * iv, acc[3] * iv);
      if (dc == 0 && grp == 0) p.lse[wr] = lse[rt];
    }
  }
}

// One wave per (request b, row i < max_q_len, query head): merge the pieces
// of rows whose request has more than one piece; pieces the row cannot see
// carry lse = -inf and get weight zero.
template <int D>
__global__ __launch_bounds__(256) void verify_combine_kernel(const VerifyArgs p) {
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
  if (i >= p.q_indptr[b + 1] - r0) return;
  const int L = p.seq_lens[b];
  const int ns = min((L + p.split_tokens - 1) / p.split_tokens, p.max_splits);
  if (ns <= 1) return;  // written by the partial kernel
  const float* lse = p.lse + R * p.max_splits;
  const float* op = p.o_part + R * p.max_splits * D + lane * EPL;
  uint16_t* out = (uint16_t*)p.out + ((int64_t)(r0 + i) * p.num_q_heads + hq) * D + lane * EPL;

  if (ns <= kFew) {
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
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < ns; c += 64) {
      const float l = lse[min(c + lane, ns - 1)];
      const float w = (c + lane < ns && l != -INFINITY) ? fast_exp2(l - M) : 0.f;
      wsum += w;
      const int cnt = min(64, ns - c);
      for (int j0 = 0; j0 < cnt; j0 += BATCH) {
        float wk[BATCH], v[BATCH][EPL];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const int j = min(j0 + k, cnt - 1);
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

template <int D, int G>
hipError_t launch_g(const VerifyArgs& a, hipStream_t stream) {
  const bool pairs = a.num_kv_heads % 2 == 0;
  const int64_t blocks = (int64_t)a.num_seqs * (a.num_kv_heads / (pairs ? 2 : 1)) * a.max_splits;
  if (blocks == 0) return hipSuccess;
  if (pairs)
    hipLaunchKernelGGL((verify_kernel<D, G, 2>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((verify_kernel<D, G, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits <= 1) return e;
  const int64_t rows = (int64_t)a.num_seqs * a.max_q_len * a.num_q_heads;
  hipLaunchKernelGGL((verify_combine_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const VerifyArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<D, 1>(a, stream);
    case 2: return launch_g<D, 2>(a, stream);
    case 3: return launch_g<D, 3>(a, stream);
    case 4: return launch_g<D, 4>(a, stream);
    case 5: return launch_g<D, 5>(a, stream);
    case 6: return launch_g<D, 6>(a, stream);
    case 7: return launch_g<D, 7>(a, stream);
    case 8: return launch_g<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

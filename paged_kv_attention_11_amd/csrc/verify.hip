// Parallel verification of drafted tokens: every request brings a short
// chunk of n new rows (k drafted tokens + 1, a handful) that attends its whole
// cached context causally.  The target model verifies the k tokens in one
// parallel prefill rather than k decodes (Mini-SGLang README, yangyonggit
// fork, section Speculative Decoding), so the rows of a request are few and
// its keys many: the work is shaped like decode, not like prefill.
//
// Design:
//  * Split-K like decode: work-group = (piece s of split_tokens keys,
//    request b, KV head g), piece index slowest; the pieces are merged by
//    verify_combine_kernel with log-sum-exp weights.
//  * The n rows x G query heads of (b, g) (at most 32) are packed into the
//    N dimension of 16x16 matrix-core tiles, two halves of 16 rows, so each
//    K/V byte is read once for all of them.
//  * K and V tiles of 64 keys come from the pages straight into an LDS ring
//    (the extend kernel's pipeline), with nontemporal loads: each tile is
//    read by one work-group only.  Wave w takes row half w % 2 and head-dim
//    half w / 2: it computes the scores of its 16 rows over the whole tile,
//    S^T = K Q^T with v_mfma_f32_16x16x32_bf16, and its half of their output,
//    O^T += V^T P^T with v_mfma_f32_16x16x16_bf16, whose B operand (keys x
//    rows) is exactly the score accumulator's layout, so P never leaves
//    registers; V^T is read with the transposing LDS read.
//  * The two waves of a row half hold identical running maxima and sums and
//    disjoint output columns: nothing is merged between waves at the end.
//  * Row (token i, head h) sees keys <= L - n + i; only the tiles that reach
//    past L - n are masked.
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
__device__ __forceinline__ f32x4_t mfma16_k16(const uint2& a, const uint2& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                   c, 0, 0, 0);
}

// LDS ring depth: kVStages - 1 tiles in flight per work-group.  Two stages
// (64 KB for D = 128) let two work-groups share a compute unit, which hides
// more latency than a third stage in one work-group (190 vs 237 us on the
// Qwen3-8B-shaped verify workload).
#ifndef PA_VERIFY_STAGES
#define PA_VERIFY_STAGES 2
#endif
constexpr int kVStages = PA_VERIFY_STAGES;
#ifndef PA_VERIFY_TILE
#define PA_VERIFY_TILE 64
#endif
constexpr int kVT = PA_VERIFY_TILE;  // keys per tile

// HP: KV heads per work-group (1 or 2).  With two, a tile holds half the
// keys of both heads of the pair, row key * 2 + head (a key's two head slices
// are 512 contiguous bytes of its pool row), and wave w serves head w / 2 over
// all head dims instead of one head's half.
template <int D, int G, int HP>
__global__ __launch_bounds__(kThreads) void verify_kernel(const VerifyArgs p) {
  using C = ExtCfg<D>;
  constexpr int VT = kVT / HP;         // keys per tile
  constexpr int TR = VT * HP;          // tile rows: (key, head) pairs
  constexpr int PPR = C::PPR, NDMA = TR * PPR / kThreads;  // DMA loads per thread per tile and tensor
  static_assert(NDMA >= 1 && TR * PPR % kThreads == 0 && VT % 16 == 0, "bad tile");
  constexpr int KS = D / 32;           // 32-wide head-dim steps of S^T
  constexpr int DCW = D / 16 * HP / 2;  // 16-wide output chunks per wave
  constexpr int NJ = VT / 16;          // 16-key slices of a tile
  static_assert(DCW >= 1 && (HP == 1 || HP == 2), "bad shape");

  __shared__ uint4 s_k[kVStages][TR * PPR];
  __shared__ uint4 s_v[kVStages][TR * PPR];
  __shared__ int32_t s_pages[kPageCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int rh = wave & 1;                 // row half: rows 16 rh .. 16 rh + 15
  const int dg = HP == 1 ? wave >> 1 : 0;  // head-dim half of the output (one head per work-group)
  const int hh = HP == 1 ? 0 : wave >> 1;  // head of the pair (two per work-group)

  // work-group -> (piece s, request b, KV head g).  Pieces are taken piece
  // index slowest; the KV head is fastest, so each XCD (work-group i runs on
  // XCD i mod 8) gets the same share of every piece.  In a batch of at most
  // 64 requests split into at most 8 pieces, work-group p of a head takes
  // the p-th piece that exists (requests are of different lengths, so later
  // piece indices exist for fewer of them): the work-groups with nothing to
  // do come last in the dispatch order instead of holding slots between the
  // others (181 -> 168 us on the Qwen3-8B-shaped verify workload).  With
  // more pieces that tail of empty work-groups grows long enough to cost
  // more than it saves (256-key pieces: 211 -> 245 us), and the plain order
  // is kept.
  const int nhb = p.num_kv_heads / HP;
  const int gb = blockIdx.x % nhb;  // head block: heads gb * HP .. + HP - 1
  const int g = gb * HP + hh;       // this wave's KV head
  const int pos = blockIdx.x / nhb;
  int s, b;
  if (p.num_seqs <= 64 && p.max_splits <= 8) {
    int ns = 0;  // lane j: pieces of request j
    if (lane < p.num_seqs) {
      const int nj = p.q_indptr[lane + 1] - p.q_indptr[lane];
      const int lj = p.seq_lens[lane];
      ns = nj > 0 ? (lj + p.split_tokens - 1) / p.split_tokens : 0;
    }
    s = -1;
    b = 0;
    int before = 0;  // existing pieces of the lower piece indices
    for (int sp = 0; sp < p.max_splits; ++sp) {  // uniform loop
      const bool has = ns > sp;
      const uint64_t have = __ballot(has);
      const int c = __popcll(have);
      if (pos < before + c) {
        // the request whose piece sp is the (pos - before)-th that exists:
        // the lane with that many existing pieces below it
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(have >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)have, 0u));
        s = sp;
        b = __builtin_ctzll(__ballot(has && below == pos - before));
        break;
      }
      before += c;
    }
    if (s < 0) return;  // uniform: past the last existing piece
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
  const int nq = min(n, p.max_q_len);  // rows computed (more than max_q_len breaks the contract)
  const int ns = (L + p.split_tokens - 1) / p.split_tokens;
  const int ntiles = (k_end - k_begin + VT - 1) / VT;

  // ---- queries: row = i * G + h; this lane supplies row 16 rh + l16 of the
  // B operand, head dims 32 ks + 8 grp .. + 7
  uint4 qreg[KS];
  {
    const int row = rh * 16 + l16;
    const int i = row / G, h = row % G;
    const bool ok = i < nq;
    const uint16_t* qp =
        (const uint16_t*)p.q + ((int64_t)(r0 + (ok ? i : 0)) * p.num_q_heads + (int64_t)g * G + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = ok ? *(const uint4*)(qp + 32 * ks + 8 * grp) : make_uint4(0, 0, 0, 0);
  }
  // retire the query loads once, so the key loop carries no wait for them
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t v = __builtin_bit_cast(u32x4_t, qreg[ks]);
    asm volatile("" : "+v"(v));
    qreg[ks] = __builtin_bit_cast(uint4, v);
  }

  // ---- page ids of the piece (split_tokens <= 1024 keys: at most 1024 pages)
  const int sh = p.log2_page;
  const int pmask = (1 << sh) - 1;
  const int pg0 = k_begin >> sh;
  const int npg = ((k_end - 1) >> sh) - pg0 + 1;
  {
    const int32_t* pt = p.page_table + (int64_t)b * p.pt_stride + pg0;
    for (int i = tid; i < npg; i += kThreads) s_pages[i] = pt[i];
  }
  __syncthreads();

  const int64_t row_stride = (int64_t)p.num_kv_heads * D;
  const uint16_t* kbase = (const uint16_t*)p.k_pool + (int64_t)gb * HP * D;  // the block's first head
  const uint16_t* vbase = (const uint16_t*)p.v_pool + (int64_t)gb * HP * D;

  // DMA of tile t into ring slot sb; keys past the piece are clamped to its
  // last key (a real row, masked out of the softmax)
  auto issue_tile = [&](int t, int sb) {
    const int pc = lane % PPR;
#pragma unroll
    for (int m = 0; m < NDMA; ++m) {
      const int blk = wave * NDMA + m;
      const int row = blk * C::RPB + lane / PPR;  // (key, head) pair of the tile
      const int kk = min(k_begin + t * VT + row / HP, k_end - 1);
      const int32_t page = s_pages[(kk >> sh) - pg0];
      const int64_t off = ((int64_t)((page << sh) | (kk & pmask))) * row_stride + (row % HP) * D;
      dma16_nt(lds_addr(&s_k[sb][blk * 64]), kbase + off + (pc ^ k_swz<D>(row)) * 8);
      dma16_nt(lds_addr(&s_v[sb][blk * 64]), vbase + off + (pc ^ v_swz<D>(row)) * 8);
    }
  };

  f32x4_t o[DCW];  // O^T chunk dc = dg * DCW + c: lane holds d = 16 dc + 4 grp + r, row 16 rh + l16
#pragma unroll
  for (int c = 0; c < DCW; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // raw-score reference maximum of this lane's row
  float l_run = 0.f;        // this lane's part of the row sum
  const float sl2 = p.scale_log2;
  const float slack = kSlack / sl2;

  // ---- prologue: tiles 0 .. kVStages - 2 in flight, tile 0 landed
  for (int t = 0; t < kVStages - 1 && t < ntiles; ++t) issue_tile(t, t);
  wait_next<kVStages, NDMA>(min(kVStages - 2, ntiles - 1));
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t % kVStages;
    if (t + kVStages - 1 < ntiles) issue_tile(t + kVStages - 1, (t + kVStages - 1) % kVStages);

    // ---- S^T of the whole tile for this row half: slice j, lane holds keys
    // 16 j + 4 grp + r of row 16 rh + l16
    f32x4_t sacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int row_l = (16 * j + l16) * HP + hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = s_k[buf][row_l * PPR + ((4 * ks + grp) ^ k_swz<D>(row_l))];
        sacc[j] = mfma16_k32(a, qreg[ks], sacc[j]);
      }
    }

    // ---- causal mask and the keys past the piece, on the last tiles only
    const int kt0 = k_begin + t * VT;
    if (kt0 + VT - 1 > prefix || kt0 + VT > k_end) {
      const int i = (rh * 16 + l16) / G;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt0 + 16 * j + 4 * grp + r;
          if (key > prefix + i || key >= k_end) sacc[j][r] = -INFINITY;
        }
    }

    // ---- online softmax: row maximum over this lane's keys and the lanes
    // holding the same row (lane ^ 16, lane ^ 32)
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[j][0], sacc[j][1]), fmaxf(sacc[j][2], sacc[j][3])));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (__ballot(mx > m_ref + slack) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_ref - m_new) * sl2);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < DCW; ++c) o[c] *= alpha;
    }
    uint2 pb[NJ];  // P^T B operands: keys 16 j + 4 grp .. + 3 of row 16 rh + l16
    {
      const float mb = m_ref == -INFINITY ? 0.f : -m_ref * sl2;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = fast_exp2(fmaf(sacc[j][r], sl2, mb));
          l_run += e[r];
        }
        pb[j] = make_uint2(pack2(e[0], e[1]), pack2(e[2], e[3]));
      }
    }

    // ---- O^T += V^T P^T for this wave's head dims: lane (grp, l16) addresses
    // key 16 j + 4 grp + l16/4, dims 16 dc + 4 (l16 % 4) .. + 3, and receives
    // V[4 keys][16 dc + l16]
    {
      const char* vb = (const char*)&s_v[buf][0];
#pragma unroll
      for (int c = 0; c < DCW; ++c) {
        const int d = 16 * (dg * DCW + c) + 4 * (l16 & 3);
        const int lp = d >> 3;
        const int within = (d & 4) ? 8 : 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int kr = (16 * j + 4 * grp + (l16 >> 2)) * HP + hh;  // tile row of the key for this head
          const uint2 x = lds_read_tr16(vb + (kr * PPR + (lp ^ v_swz<D>(kr))) * 16 + within);
          o[c] = mfma16_k16(x, pb[j], o[c]);
        }
      }
    }

    // tiles issued after t + 1: min(kVStages - 2, ntiles - 2 - t)
    wait_next<kVStages, NDMA>(min(kVStages - 2, ntiles - 2 - t));
    __syncthreads();
  }

  // ---- write this wave's columns of its valid rows
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  const int row = rh * 16 + l16;
  const int i = row / G, h = row % G;
  if (i >= nq) return;
  const bool seen = m_ref != -INFINITY;  // false: no key of this piece is visible to the row
  const float inv = seen ? 1.f / l_run : 0.f;
  const int64_t head = (int64_t)g * G + h;
  if (ns == 1) {
    uint16_t* op = (uint16_t*)p.out + ((int64_t)(r0 + i) * p.num_q_heads + head) * D;
#pragma unroll
    for (int c = 0; c < DCW; ++c) {
      const int d = 16 * (dg * DCW + c) + 4 * grp;
      *(uint2*)(op + d) = make_uint2(pack_bf16x2(o[c][0] * inv, o[c][1] * inv),
                                     pack_bf16x2(o[c][2] * inv, o[c][3] * inv));
    }
  } else {
    const int64_t wr = (((int64_t)b * p.max_q_len + i) * p.num_q_heads + head) * p.max_splits + s;
    float* op = p.o_part + wr * D;
#pragma unroll
    for (int c = 0; c < DCW; ++c) {
      const int d = 16 * (dg * DCW + c) + 4 * grp;
      *(float4*)(op + d) = make_float4(o[c][0] * inv, o[c][1] * inv, o[c][2] * inv, o[c][3] * inv);
    }
    if (dg == 0 && grp == 0) p.lse[wr] = seen ? m_ref * sl2 + __log2f(l_run) : -INFINITY;
  }
}

// One wave per (request b, row i < max_q_len, query head): merge the pieces
// of rows whose request has more than one piece; pieces the row cannot see
// carry lse = -inf and get weight zero.
template <int D>
__global__ __launch_bounds__(256) void verify_combine_kernel(const VerifyArgs p) {
  constexpr int EPL = D / 64;
  constexpr int BATCH = 8;
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
  uint16_t* out = (uint16_t*)p.out + ((int64_t)(r0 + i) * p.num_q_heads + hq) * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = (uint16_t)f32_to_bf16_bits(o[e]);
}

#ifndef PA_VERIFY_HEAD_PAIRS
#define PA_VERIFY_HEAD_PAIRS 1
#endif

template <int D, int G>
hipError_t launch_g(const VerifyArgs& a, hipStream_t stream) {
  const bool pairs = PA_VERIFY_HEAD_PAIRS && a.num_kv_heads % 2 == 0;
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

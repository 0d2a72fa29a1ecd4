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
//
// Design (FlashAttention-2 style tiling written for the CDNA4 matrix core):
//  * Work-group = 4 waves = 128 query rows = (128 / G) tokens (or group
//    members) x all G query heads of one KV head, so every K/V tile staged in
//    LDS serves G heads.
//  * Per wave: 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in
//    registers), so each lane owns one query row of the score tile and the
//    softmax needs only one cross-lane exchange (lane ^ 32).  The output is
//    also accumulated transposed, O^T += V^T P^T, so the rescale factor of a
//    query row is lane-local and P goes from the score accumulator to the
//    B operand without leaving registers.
//  * K and V tiles (64 keys) are copied straight from the pages into an LDS
//    ring with direct-to-LDS loads one tile ahead, two work-groups per
//    compute unit (registers cut to 2 waves per SIMD); V stays in row
//    layout and is read into the A operand with transposing LDS reads.
//  * Key tiles entirely above the diagonal are never visited; only tiles that
//    cross it (or a row's key limit) are masked.
//  * Softmax in fp32 (base 2, scale folded with log2 e); P is rounded to bf16
//    for the matrix core; O accumulates in fp32 and is rounded once.
#include "device.h"
#include "mfma_tile.h"
#include "internal.h"

namespace pa {

namespace {

using namespace tile;

constexpr int kThreads = kTileThreads;
constexpr int kRows = 128;  // query rows per work-group

// LDS ring depth and the waves per SIMD the register budget is cut for.  A
// 2-stage ring (64 KB for D = 128) with registers cut to 256 lets two
// work-groups share a compute unit, so one's softmax and LDS traffic overlap
// the other's matrix-core work: 324 -> 260 us on the Qwen3-8B-shaped
// chunked-prefill workload, where a deeper ring in one work-group per CU
// changed nothing.
#ifndef PA_EXTEND_STAGES
#define PA_EXTEND_STAGES 2
#endif
#ifndef PA_EXTEND_WAVES
#define PA_EXTEND_WAVES 2
#endif
constexpr int kEStages = PA_EXTEND_STAGES;

constexpr float kExtRescaleSlack = 8.0f;  // log2 units, as in decode

__device__ __forceinline__ int shfl_xor_i(int x, int mask) {
  return __builtin_amdgcn_ds_bpermute((__lane_id() ^ mask) << 2, x);
}

// PREFIX = false: extend (chunk of new tokens, causal after the prefix).
// PREFIX = true:  shared-prefix pass of the cascade decode.
template <int D, int G, bool PREFIX>
__global__ __launch_bounds__(kThreads, PA_EXTEND_WAVES) void mfma_attn_kernel(const ExtendArgs p) {
  using C = ExtCfg<D>;
  constexpr int TOK = kRows / G;  // tokens (or group members) per work-group
  constexpr int KSTEPS = C::KSTEPS, DT = C::DT, PPR = C::PPR, NDMA = C::NDMA;

  __shared__ uint4 s_k[kEStages][kKT * PPR];
  __shared__ uint4 s_v[kEStages][kKT * PPR];
  __shared__ int32_t s_pages[kPageCap];
  __shared__ int32_t s_red[2][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query row within the wave
  const int half = lane >> 5;
  const int row = wave * 32 + col;  // rows are (head, token/member) with token fastest
  const int hq = row / TOK;

  int g, q_row, vis_lim, k_begin, k_end, min_vis, piece = 0;
  bool qvalid, has_keys;
  const int32_t* pt;
  if constexpr (!PREFIX) {
    // work-group: token block qb of (request b, KV head g); the blocks of one
    // (request, head) are consecutive ids, heaviest (latest) first
    const int qblocks = (p.max_q_len + TOK - 1) / TOK;
    int bid = blockIdx.x;
    const int qb = qblocks - 1 - (bid % qblocks);
    bid /= qblocks;
    g = bid % p.num_kv_heads;
    const int b = bid / p.num_kv_heads;
    const int r0 = p.q_indptr[b];
    const int n = p.q_indptr[b + 1] - r0;
    const int i0 = qb * TOK;
    if (i0 >= n || (n == 1 && p.skip_single)) return;
    const int prefix = p.seq_lens[b] - n;
    k_begin = 0;
    k_end = prefix + min(i0 + TOK, n);  // keys this block can see
    const int ti = i0 + (row % TOK);
    qvalid = ti < n;
    q_row = r0 + ti;
    vis_lim = prefix + (qvalid ? ti : (n - 1));  // padding rows mask like the last token
    min_vis = prefix + i0;
    has_keys = true;
    pt = p.page_table + (int64_t)b * p.pt_stride;
  } else {
    // work-group: key piece sp of row block rb of (group j, KV head g)
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
    if (m0 >= gsize) return;
    const int mi = m0 + (row % TOK);
    qvalid = mi < gsize;
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
    mx = max(max(s_red[0][0], s_red[0][1]), max(s_red[0][2], s_red[0][3]));
    mn = min(min(s_red[1][0], s_red[1][1]), min(s_red[1][2], s_red[1][3]));
    if (k_begin >= mx) return;  // no row of the block reads this piece (uniform)
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
  const int chunk_keys = kPageCap << sh;  // keys covered by one staging of page ids
  const int npages = ((k_end - 1) >> sh) + 1;

  // Page ids of chunk c (pages c*kPageCap ...) into LDS; entries past the
  // block's last page are not read.
  auto stage_pages = [&](int c) {
    const int base = c * kPageCap;
    for (int i = tid; i < kPageCap; i += kThreads)
      if (base + i < npages) s_pages[i] = pt[base + i];
  };

  // DMA of tile t into ring slot sb: each wave fills NDMA 1 KB blocks of K and
  // of V.  Keys past the block's range are clamped to its last key (a real
  // row; masked out of the softmax).
  auto issue_tile = [&](int t, int sb, int chunk) {
    const int pc = lane % PPR;
#pragma unroll
    for (int m = 0; m < NDMA; ++m) {
      const int blk = wave * NDMA + m;
      const int key = blk * C::RPB + lane / PPR;
      const int kk = min(k_begin + t * kKT + key, k_end - 1);
      const int32_t page = s_pages[(kk >> sh) - chunk * kPageCap];
      const int64_t off = ((int64_t)((page << sh) | (kk & pmask))) * row_stride;
      dma16(lds_addr(&s_k[sb][blk * 64]), kbase + off + (pc ^ k_swz<D>(key)) * 8);
      dma16(lds_addr(&s_v[sb][blk * 64]), vbase + off + (pc ^ v_swz<D>(key)) * 8);
    }
  };
  auto chunk_of = [&](int t) { return (k_begin + t * kKT) / chunk_keys; };

  f32x16_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_ref = -INFINITY;  // reference maximum of this row's raw scores
  float l_run = 0.f;        // this lane's half of the running sum
  const float sl2 = p.scale_log2;
  const float slack = kExtRescaleSlack / sl2;  // the same slack in raw-score units

  // ---- prologue: page ids, then tiles 0 .. kEStages - 2 in flight
  int chunk = chunk_of(0);
  stage_pages(chunk);
  __syncthreads();
  for (int t = 0; t < kEStages - 1 && t < ntiles; ++t) {
    const int c = chunk_of(t);
    if (c != chunk) {  // rare: the tile starts the next chunk of page ids
      vm_wait<0>();
      __syncthreads();
      chunk = c;
      stage_pages(chunk);
      __syncthreads();
    }
    issue_tile(t, t, chunk);
  }
  wait_next<kEStages, NDMA>(min(kEStages - 2, ntiles - 1));
  __syncthreads();

  // Per-lane LDS byte offsets inside a tile, computed once.  K piece
  // (2 ks + half) ^ (key mod PPR) of key 32 kt + col sits at
  // 32 kt PPR 16 + koff[ks]; the transposing V read of step (ks, r) and
  // head-dim block i sits at 16 ks PPR 16 + 8 r PPR 16 + voff[i].  Together
  // with a compile-time ring slot the rest of each LDS address is an
  // instruction's immediate offset.
  uint32_t koff[KSTEPS], voff[DT];
  {
    const int ck = col & (PPR - 1);
    const int kb = col * PPR * 16 + 16 * (half ^ (ck & 1));
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) koff[ks] = kb + 32 * (ks ^ (ck >> 1));
    const int j = lane & 15, g1 = (lane >> 4) & 1;
    const int sv = 2 * ((j >> 2) & 3);
    const int pl = (4 * half + (j >> 2)) * PPR * 16 + 8 * (j & 1) + 16 * ((2 * g1 + ((j >> 1) & 1)) ^ (sv & 3));
#pragma unroll
    for (int i = 0; i < DT; ++i) voff[i] = pl + 64 * (i ^ (sv >> 2));
  }
  constexpr int kTileBytes = kKT * PPR * 16;
  const char* const k_lds = (const char*)&s_k[0][0];
  const char* const v_lds = (const char*)&s_v[0][0];

  // One tile; `buf` is a compile-time ring slot in every inlined copy.
  auto tile_step = [&](const int t, const int buf) __attribute__((always_inline)) {
      const int tn = t + kEStages - 1;  // the tile issued now
      if (tn < ntiles) {
        const int c2 = chunk_of(tn);
        if (c2 != chunk) {  // block-uniform and rare: restage page ids
          vm_wait<0>();
          __syncthreads();
          stage_pages(c2);
          chunk = c2;
          __syncthreads();
        }
        issue_tile(tn, (buf + kEStages - 1) % kEStages, chunk);
      }

      // ---- S^T = K Q^T for two 32-key halves of the tile
      f32x16_t s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        // the first step accumulates onto the inline constant 0
        s[kt] = mfma32(*(const uint4*)(k_lds + buf * kTileBytes + kt * 32 * PPR * 16 + koff[0]), qreg[0],
                       f32x16_t{});
#pragma unroll
        for (int ks = 1; ks < KSTEPS; ++ks) {
          const uint4 a = *(const uint4*)(k_lds + buf * kTileBytes + kt * 32 * PPR * 16 + koff[ks]);
          s[kt] = mfma32(a, qreg[ks], s[kt]);
        }
      }

      // ---- mask, only on tiles that reach past some row's last visible key
      const int kt0 = k_begin + t * kKT;
      if (kt0 + kKT - 1 > min_vis) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key > vis_lim) s[kt][r] = -INFINITY;
          }
      }

      // ---- online softmax and O^T += V^T P^T, one 32-key half at a time so
      // that the softmax of a half can overlap the matrix-core work of the
      // other (lane owns one query row; the reference maximum moves only when
      // exceeded by the slack, checked per half)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        if (__ballot(mx > m_ref + slack) != 0) {
          const float m_new = fmaxf(m_ref, mx);
          const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_ref - m_new) * sl2);
          m_ref = m_new;
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < DT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
        }
        // a row with no visible key yet keeps weights exp2(-inf) = 0
        const float mb = m_ref == -INFINITY ? 0.f : -m_ref * sl2;
        uint4 pb[2];  // B operands of this half's two 16-key steps
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          e[r] = fast_exp2(fmaf(s[kt][r], sl2, mb));
          l_run += e[r];
        }
        pb[0] = make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
        pb[1] = make_uint4(pack2(e[8], e[9]), pack2(e[10], e[11]), pack2(e[12], e[13]), pack2(e[14], e[15]));

        // the A operand is read transposed out of row-major V: lane (group of
        // 16, j) reads keys 16ks + 8r + 4*half + j/4, head-dims d0 + 4(j%4) ..
        // +3 and receives V[4 keys][d0 + j]
#pragma unroll
        for (int i = 0; i < DT; ++i) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int ks = 2 * kt + k2;
            const char* vp = v_lds + buf * kTileBytes + ks * 16 * PPR * 16 + voff[i];
            const uint2 x0 = lds_read_tr16(vp);
            const uint2 x1 = lds_read_tr16(vp + 8 * PPR * 16);
            o[i] = mfma32(make_uint4(x0.x, x0.y, x1.x, x1.y), pb[k2], o[i]);
          }
        }
      }

      // tile t+1 must have landed (the tiles issued after it may still be in
      // flight) before the next iteration reads it; the barrier also retires
      // this tile's reads
      wait_next<kEStages, NDMA>(min(kEStages - 2, ntiles - 2 - t));
      __syncthreads();
  };

  for (int t0 = 0; t0 < ntiles; t0 += kEStages) {
#pragma unroll
    for (int u = 0; u < kEStages; ++u) {
      if (t0 + u >= ntiles) break;
      tile_step(t0 + u, u);
    }
  }

  // ---- normalise and write this lane's row
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if constexpr (!PREFIX) {
    if (!qvalid) return;
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
  } else {
    // the combine kernel reads this piece for a member only if the member
    // has keys in it
    if (!has_keys) return;
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

template <int D, int G, bool PREFIX>
hipError_t launch_g(const ExtendArgs& a, hipStream_t stream) {
  constexpr int TOK = kRows / G;
  const int64_t blocks_per = (a.max_q_len + TOK - 1) / TOK;
  const int64_t blocks = blocks_per * a.num_kv_heads * a.num_seqs * (PREFIX ? a.num_pieces : 1);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mfma_attn_kernel<D, G, PREFIX>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool PREFIX>
hipError_t launch_d(const ExtendArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<D, 1, PREFIX>(a, stream);
    case 2: return launch_g<D, 2, PREFIX>(a, stream);
    case 4: return launch_g<D, 4, PREFIX>(a, stream);
    case 8: return launch_g<D, 8, PREFIX>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128, false>(a, stream);
  if (a.head_dim == 64) return launch_d<64, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefix(const ExtendArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128, true>(a, stream);
  if (a.head_dim == 64) return launch_d<64, true>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

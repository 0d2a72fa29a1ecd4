// Paged decode attention for gfx950: one new query token per request attends
// every key of its request through the page table, with grouped-query heads.
//
// What is computed (Mini-SGLang README, yangyonggit fork, section Reference
// Attention Backends: paged gather, GQA by repeat_interleave; nanoSGLang
// README, section Ablation: attention straight from the pages through the
// page table, no per-token copy):
//   out[b,h] = softmax(scale * K_{b,g} q[b,h]) V_{b,g},  g = h / G.
// The triton backend on the same page runs an online (FlashAttention-style)
// softmax per (request, head); this design keeps the online softmax but
// reorganises the work for an HBM-bound gfx950 kernel:
//
//  * Split-K over keys.  Work unit = (request b, block of HB neighbouring KV
//    heads, piece s of split_tokens keys).  decode_partial_kernel writes the
//    piece's normalised output o_s and its log2-sum-exp per query head;
//    decode_combine_kernel merges pieces with weights 2^(lse_s - max lse).  A
//    request with one piece is finished by the partial kernel directly.
//  * GQA sharing.  The waves of a KV head serve all G query heads of it, so
//    every K/V byte is fetched from HBM once per work unit and reused G times
//    from registers.
//  * Loads.  Each wave takes 16 keys per iteration, and every load
//    instruction covers whole 128-byte lines of the key rows.  K is read in
//    an "octet" layout: eight lanes per key, lane o holding 16-byte pieces
//    o, o+8, ... of the key's head row, keys a and a+8 for lane group a;
//    the QK dot product is a packed bf16 dot (v_dot2_f32_bf16) plus a
//    transposing three-step DPP reduction over the octet, after which each
//    lane holds whole dot products of its own (key, head) pairs, so each
//    score is exponentiated once.  (Read-only probes of the Qwen3-8B-shaped
//    radix batch with nontemporal loads: 6.89 TB/s with K in octets against
//    6.19 TB/s with four lanes per key, whose load instructions cover half
//    lines.)  V is read in a "row" layout: D/8 consecutive lanes cover one
//    key's head row with 16-byte loads.  Softmax weights move from the K
//    layout to the V layout through LDS.
//  * Online softmax with a wave-uniform reference maximum.  The reference is
//    raised (and the accumulator rescaled) only when a score exceeds it by
//    more than 2^8 in the exponent, so the common iteration does no cross-lane
//    maximum and no rescale; the result is exact because numerator and
//    denominator carry the same reference.
//  * Key slots of the piece (page_table[t / P] * P + t % P) are computed once
//    per work-group into LDS.
//  * Work order.  On large batches one work-group first lists the pieces
//    that exist, longest first (plan.h), and the partial kernel's
//    work-groups take them in that order.
#include <type_traits>

#include "device.h"
#include "internal.h"
#include "plan.h"

namespace pa {

namespace {

constexpr int kThreads = kDecodeWaves * 64;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <bool BF16, int D, int G>
struct DecodeCfg {
  static constexpr int EPC = BF16 ? 8 : 4;        // elements per 16-byte piece
  static constexpr int CPR = D / EPC;              // pieces per head row
  static constexpr int PPL = CPR / 8;              // K pieces per lane and key (octet layout)
  static constexpr int NK = 2 * PPL;               // K pieces per lane per iteration (two keys)
  static constexpr int VP = (2 * G + 7) / 8 * 8;   // dot products per lane before the octet reduction
  static constexpr int VPL = VP / 8;               // ... and after it
  static constexpr int LPR = CPR;                  // lanes per V row
  static constexpr int RPI = 64 / LPR;             // V rows per load instruction
  static constexpr int NV = kDecodeTokPerIter / RPI;  // V pieces per lane per iteration
  static constexpr int GP = (G + 3) & ~3;          // group padded for float4 LDS reads
  static_assert(PPL >= 1 && CPR % 8 == 0 && RPI >= 1 && NV >= 1, "bad tiling");
};

template <bool BF16, int D, int G>
struct Tile {
  using C = DecodeCfg<BF16, D, G>;
  uint4 k[C::NK];
  uint4 v[C::NV];
};

// QK partial dot product of one 16-byte piece.
template <bool BF16>
__device__ __forceinline__ float dot_piece(const uint4& q, const uint4& k, float acc) {
  if constexpr (BF16) {
    acc = dot2_bf16(q.x, k.x, acc);
    acc = dot2_bf16(q.y, k.y, acc);
    acc = dot2_bf16(q.z, k.z, acc);
    acc = dot2_bf16(q.w, k.w, acc);
  } else {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  }
  return acc;
}

template <bool BF16>
__device__ __forceinline__ void widen_piece(const uint4& v, float* f) {
  if constexpr (BF16) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 1
#endif
constexpr int DEPTH = PA_DECODE_DEPTH;  // tile buffers per wave

// Waves per SIMD the register budget is sized for: one tile buffer, the
// group's accumulators and scores, and a fixed remainder (queries live in LDS).
template <bool BF16, int D, int G>
struct DecodeOcc {
  using C = DecodeCfg<BF16, D, G>;
  static constexpr int kEstVgprs = G * C::EPC + (C::NK + C::NV) * 4 * DEPTH + 2 * G + 36;
  static constexpr int kEst = 512 / kEstVgprs < 1 ? 1 : (512 / kEstVgprs > 8 ? 8 : 512 / kEstVgprs);
  // Corrections where the estimate is too tight or too loose, each checked
  // against the compiler's register report so that no instantiation spills
  // to scratch memory inside the key loop (the loose estimate let the
  // compiler spend the spare registers and lose a wave per SIMD).
  static constexpr int kWaves = (BF16 && G == 8)                ? 2
                                : (BF16 && D == 128 && G == 1)  ? 8
                                : (BF16 && D == 128 && G == 2)  ? 6
                                : (BF16 && D == 128 && G == 3)  ? 4
                                : (BF16 && D == 128 && G == 4)  ? 5
                                : (BF16 && D == 64 && G == 7)   ? 3
                                : (D == 64 && G == 5)           ? 4
                                : (!BF16 && D == 128 && G == 1) ? 5
                                : (!BF16 && D == 64 && G <= 3)  ? (G == 1 ? 8 : 7)
                                : (!BF16 && D == 64 && G == 8)  ? 3
                                                                : kEst;
};
#ifdef PA_DECODE_MIN_WAVES
#define PA_DECODE_WAVES(B, D, G) PA_DECODE_MIN_WAVES
#else
#define PA_DECODE_WAVES(B, D, G) (DecodeOcc<B, D, G>::kWaves)
#endif

typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));

// 16-byte load; NT marks it nontemporal (streamed past the caches).
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* ptr) {
  if constexpr (NT)
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_nt_t*)ptr));
  else
    return *(const uint4*)ptr;
}

// The work order of the partial kernel (plan.h), by one work-group: 256
// threads for batches of at most 256 requests (one request per thread, and
// the loops over the waves of the work-group are short), else 1024.
template <int kPlanThreads>
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const PlanArgs p) {
  build_decode_plan<kPlanThreads>(p);
}

// The work order and the store of the step's new rows in one launch (they
// are independent): work-group 0 writes the order when there is one, the
// other work-groups copy new row i to flat slot slot_mapping[i] of both pools
// (negative slots are padding), one 16-byte piece per lane, as
// kv_store_kernel does.  One launch instead of two takes a kernel and a
// launch gap off the critical path of a decode step.
template <int kPlanThreads>
__global__ __launch_bounds__(kPlanThreads) void decode_plan_store_kernel(const PlanArgs p, const StoreArgs s) {
  int first = 0;
  if (p.plan) {
    if (blockIdx.x == 0) {
      build_decode_plan<kPlanThreads>(p);
      return;
    }
    first = 1;
  }
  const uint4* k_new = (const uint4*)s.k_new;
  const uint4* v_new = (const uint4*)s.v_new;
  uint4* k_pool = (uint4*)s.k_pool;
  uint4* v_pool = (uint4*)s.v_pool;
  const int64_t total = s.num_rows * s.row_chunks;
  const int64_t stride = (int64_t)(gridDim.x - first) * kPlanThreads;
  for (int64_t i = (int64_t)(blockIdx.x - first) * kPlanThreads + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / s.row_chunks;
    const int64_t c = i - row * s.row_chunks;
    const int64_t slot = s.slot_mapping[row];
    if (slot < 0) continue;
    const int64_t dst = slot * s.row_chunks + c;
    k_pool[dst] = k_new[i];
    v_pool[dst] = v_new[i];
  }
}

// Transposing sum over the eight lanes of each octet: value m of lane o
// enters; afterwards lane o holds, at index u, the octet's sum of value
// 8 u + o.  Each step pairs lanes that differ in one bit of o (partners
// o ^ 7, o ^ 2, o ^ 1 in turn), keeps the half of the values whose index
// bit matches that bit of the lane and receives the partner's copy of it.
template <int VP>
__device__ __forceinline__ void octet_reduce(float (&v)[VP], const int o) {
  const bool b2 = (o & 4) != 0, b1 = (o & 2) != 0, b0 = (o & 1) != 0;
  float w[VP / 2], x[VP / 4];
#pragma unroll
  for (int u = 0; u < VP / 8; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lo = v[8 * u + r], hi = v[8 * u + r + 4];
      w[4 * u + r] = (b2 ? hi : lo) + octet_mirror(b2 ? lo : hi);
    }
#pragma unroll
  for (int u = 0; u < VP / 8; ++u)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const float lo = w[4 * u + r], hi = w[4 * u + r + 2];
      x[2 * u + r] = (b1 ? hi : lo) + quad_xor2(b1 ? lo : hi);
    }
#pragma unroll
  for (int u = 0; u < VP / 8; ++u) {
    const float lo = x[2 * u], hi = x[2 * u + 1];
    v[u] = (b0 ? hi : lo) + quad_xor1(b0 ? lo : hi);
  }
}

// NT: the keys are read once per step and nowhere else (each request's own
// keys in the cascade), so they are loaded nontemporally and leave the
// caches to the data that is read again (the groups' shared pages, the
// queries, the partials).
// HB: KV heads per work-group.  Wave w serves KV head (first + w / WPH) and
// takes every WPH-th 16-key block of the piece.  With HB > 1 the waves of a
// work-group read neighbouring head slices of the same key rows at about the
// same time, which streams faster than one head per work-group: read-only
// probes of the Qwen3-8B-shaped batch (8 KV heads, 256-byte head slices of
// 2 KB rows) moved 5.78 TB/s with one head x four waves, 6.09 TB/s with two
// heads x two waves and 6.02-6.06 TB/s with four heads x one wave.
template <bool BF16, int D, int G, bool NT, int HB>
__global__ __launch_bounds__(kThreads, PA_DECODE_WAVES(BF16, D, G)) void decode_partial_kernel(
    const DecodeArgs p) {
  using C = DecodeCfg<BF16, D, G>;
  using T = std::conditional_t<BF16, uint16_t, float>;
  constexpr int EPC = C::EPC, NK = C::NK, NV = C::NV, RPI = C::RPI, LPR = C::LPR, GP = C::GP;
  static_assert(kDecodeWaves % HB == 0, "heads per work-group must divide its waves");
  constexpr int WPH = kDecodeWaves / HB;  // waves per KV head

  __shared__ int32_t s_slot[kMaxSplitTokens];
  __shared__ uint4 s_q[HB * G][C::CPR];
  __shared__ float4 s_p4[kDecodeWaves][kDecodeTokPerIter][GP / 4];
  __shared__ float s_acc[kDecodeWaves][G][D];
  __shared__ float s_m[kDecodeWaves][G];
  __shared__ float s_l[kDecodeWaves][G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, marked wave-uniform so loop control stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Work-group id -> (piece s, request b, KV head block gb of HB heads).
  // Without a plan the piece index is slowest; with one, work-groups
  // i * NB .. (NB = H_kv / HB) take plan entry i.  Either way the head block
  // is fastest, so consecutive ids go to the 8 XCDs in turn and the XCD of a
  // unit is (its rank * NB + gb) mod 8: every XCD gets a fair share of every
  // kind of piece, and with HB = 1 and 8 KV heads every request's head g runs
  // on XCD g, where the pages that requests share (prefix pages) are served
  // from its L2.
  const int nb = p.num_kv_heads / HB;
  int s, b, gb, qrow, t_begin, n_tok;
  bool single;
  if (p.plan) {
    const int i = blockIdx.x / nb;
    gb = blockIdx.x - i * nb;
    const int4 e = p.plan[i];
    b = e.x;
    s = e.y & (kPlanSingle - 1);
    single = (e.y & kPlanSingle) != 0;
    t_begin = e.z;
    n_tok = e.w;
    // no work, or an entry this batch cannot have (an order written for
    // another batch): nothing is read or written.  The key range is checked
    // against the request's length after the slots are staged.
    if (b < 0 || b >= p.num_seqs || s >= p.max_splits || n_tok > p.split_tokens || t_begin < 0 ||
        (int64_t)t_begin + n_tok > ((int64_t)p.pt_stride << p.log2_page))
      return;  // uniform over the work-group
  } else {
    const int units = p.num_seqs * nb;
    s = blockIdx.x / units;
    const int bg = blockIdx.x - s * units;
    gb = bg % nb;
    b = bg / nb;
  }
  // Mixed batch: only requests with one new row, whose query and output row
  // is q_indptr[b].
  qrow = b;
  if (p.q_indptr) {
    qrow = p.q_indptr[b];
    if (p.q_indptr[b + 1] - qrow != 1) return;  // uniform over the work-group
  }
  // This request's key range is [k0, L)
  const int L = p.seq_lens[b];
  const int k0 = p.key_begin ? max(p.key_begin[b], 0) : 0;
  const bool zero_row = s == 0 && L <= 0 && !p.key_begin && !p.always_partial;
  if (!p.plan) {  // piece s covers split_tokens keys of the range
    t_begin = k0 + s * p.split_tokens;
    n_tok = t_begin < L ? min(L - t_begin, p.split_tokens) : 0;
    single = (L - k0 + p.split_tokens - 1) / p.split_tokens == 1 && !p.always_partial;
  }
  if (n_tok <= 0) {
    // a request with no keys gets zero rows here when it has no pieces to
    // merge later (plain decode)
    if (!zero_row) return;  // uniform over the work-group
    const int64_t orow0 = (int64_t)qrow * p.num_q_heads + (int64_t)gb * HB * G;
    for (int idx = threadIdx.x; idx < HB * G * D; idx += kThreads) {
      if constexpr (BF16)
        ((uint16_t*)p.out)[orow0 * D + idx] = 0;
      else
        ((float*)p.out)[orow0 * D + idx] = 0.f;
    }
    return;
  }

  // ---- stage the piece's key slots in LDS
  {
    const int32_t* pt = p.page_table + (int64_t)b * p.pt_stride;
    const int sh = p.log2_page;
    const int pmask = (1 << sh) - 1;
    for (int i = tid; i < n_tok; i += kThreads) {
      const int t = t_begin + i;
      s_slot[i] = (pt[t >> sh] << sh) | (t & pmask);
    }
  }

  // ---- the queries of the block's HB * G heads, staged in LDS (read back per
  // tile as broadcasts)
  const int o8 = lane & 7;   // piece column of the octet (K layout)
  const int a8 = lane >> 3;  // keys a8 and a8 + 8 of the iteration (K layout)
  const int vr = lane / LPR;  // key row within a V load instruction
  const int vc = lane % LPR;  // 16-byte piece within the V row
  {
    const uint4* qb =
        (const uint4*)((const T*)p.q + ((int64_t)qrow * p.num_q_heads + (int64_t)gb * HB * G) * D);
    for (int i = tid; i < HB * G * C::CPR; i += kThreads) (&s_q[0][0])[i] = qb[i];
  }
  const int hw = wave / WPH;               // this wave's head within the block
  const int ks = wave - hw * WPH;          // and its share of the keys
  const int g = gb * HB + hw;              // its KV head
  const uint4(*qw)[C::CPR] = s_q + hw * G;  // its G queries

  const int64_t row_stride = (int64_t)p.num_kv_heads * D;  // elements per slot
  const T* kbase = (const T*)p.k_pool + (int64_t)g * D;
  const T* vbase = (const T*)p.v_pool + (int64_t)g * D;
  const float sl2 = p.scale_log2;

  // the (key, head) pairs of this lane after the octet reduction: value
  // m = 8 u + o8 is head m % G of key 8 (m / G) + a8 (m < 2 G; the rest pad)
  constexpr int VP = C::VP, VPL = C::VPL, PPL = C::PPL;
  // (recomputed where used: cheaper than holding them in registers)
  auto live = [&](int u) __attribute__((always_inline)) { return 8 * u + o8 < 2 * G; };
  auto h_of = [&](int u) __attribute__((always_inline)) { return live(u) ? (8 * u + o8) % G : 0; };
  auto key_of = [&](int u) __attribute__((always_inline)) { return live(u) ? ((8 * u + o8) / G) * 8 + a8 : 0; };

  float m_ref[G];   // wave-uniform reference maximum (log2 domain)
  float l_acc[VPL];  // per-lane partial sum of weights of its pairs (K layout)
  float acc[G][EPC];  // per-lane partial output (V layout)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_ref[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < VPL; ++u) l_acc[u] = 0.f;
  // m_ref of this lane's head for pair u
  auto ref_of = [&](int u) __attribute__((always_inline)) {
    float r = m_ref[0];
#pragma unroll
    for (int h = 1; h < G; ++h) r = h_of(u) == h ? m_ref[h] : r;
    return r;
  };

  __syncthreads();  // s_slot and s_q ready
  if (t_begin < k0 || (int64_t)t_begin + n_tok > L) return;  // (work order only) uniform over the work-group

  // Loads are issued unconditionally: a key index past the piece is clamped to
  // the piece's last key (a real row, so no NaN can enter; its weight is 0).
  // With no branch around the loads the compiler can keep DEPTH-1 tiles in
  // flight (a skipped load would force it to wait for every load).
  // (nt: std::true_type for nontemporal loads)
  auto load_tile = [&](int ib, Tile<BF16, D, G>& tl, auto nt) {
    constexpr bool LNT = decltype(nt)::value;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      const int ik = min(ib + 8 * kg + a8, n_tok - 1);
      const T* kp = kbase + (int64_t)s_slot[ik] * row_stride;
#pragma unroll
      for (int pc = 0; pc < PPL; ++pc) tl.k[kg * PPL + pc] = load16<LNT>(kp + (8 * pc + o8) * EPC);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int iv = min(ib + j * RPI + vr, n_tok - 1);
      tl.v[j] = load16<LNT>(vbase + (int64_t)s_slot[iv] * row_stride + vc * EPC);
    }
  };

  auto compute_tile = [&](int ib, const Tile<BF16, D, G>& tl) {
    // this lane's partial dot products (value kg * G + h: key 8 kg + a8,
    // head h), then whole ones for its own pairs
    float dv[VP];
#pragma unroll
    for (int m = 0; m < VP; ++m) dv[m] = 0.f;
#pragma unroll
    for (int pc = 0; pc < PPL; ++pc) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4 qv = qw[h][8 * pc + o8];
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) dv[kg * G + h] = dot_piece<BF16>(qv, tl.k[kg * PPL + pc], dv[kg * G + h]);
      }
      __builtin_amdgcn_sched_barrier(0);  // one piece's queries in registers at a time
    }
    octet_reduce<VP>(dv, o8);
    float sc[VPL];
    bool over = false;
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const bool valid = live(u) && ib + key_of(u) < n_tok;
      sc[u] = valid ? dv[u] * sl2 : -INFINITY;
      over |= sc[u] > ref_of(u) + kRescaleSlack;
    }
    if (__ballot(over) != 0) {  // rare: raise the reference maximum
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mh = -INFINITY;
#pragma unroll
        for (int u = 0; u < VPL; ++u) mh = h_of(u) == h ? fmaxf(mh, sc[u]) : mh;
        const float mx = fmaxf(m_ref[h], wave_max(mh));
        const float alpha = fast_exp2(m_ref[h] - mx);
        m_ref[h] = mx;
#pragma unroll
        for (int u = 0; u < VPL; ++u) l_acc[u] = h_of(u) == h ? l_acc[u] * alpha : l_acc[u];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha;
      }
    }
    // each (key, head) weight is published by the one lane that holds it
    float* sp = reinterpret_cast<float*>(&s_p4[wave][0][0]);
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const float pw = live(u) ? fast_exp2(sc[u] - ref_of(u)) : 0.f;
      l_acc[u] += pw;
      if (live(u)) sp[key_of(u) * GP + h_of(u)] = pw;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int tv = j * RPI + vr;
      float pv[GP];
#pragma unroll
      for (int h4 = 0; h4 < GP / 4; ++h4) {
        const float4 x = s_p4[wave][tv][h4];
        pv[4 * h4 + 0] = x.x; pv[4 * h4 + 1] = x.y; pv[4 * h4 + 2] = x.z; pv[4 * h4 + 3] = x.w;
      }
      float vf[EPC];
      widen_piece<BF16>(tl.v[j], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(pv[h], vf[e], acc[h][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- main loop: DEPTH tile buffers, DEPTH-1 tiles in flight while one is
  // computed (buffer indices are compile-time after unrolling)
  constexpr int kStep = WPH * kDecodeTokPerIter;
  auto key_loop = [&](auto nt) {
    const int ib0 = ks * kDecodeTokPerIter;
    if (ib0 < n_tok) {  // uniform over the wave
      Tile<BF16, D, G> buf[DEPTH];
#pragma unroll
      for (int k = 0; k < DEPTH - 1; ++k) load_tile(ib0 + k * kStep, buf[k], nt);
      for (int base = ib0; base < n_tok; base += DEPTH * kStep) {
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
          const int cur = base + k * kStep;
          if (cur >= n_tok) break;
          load_tile(cur + (DEPTH - 1) * kStep, buf[(k + DEPTH - 1) % DEPTH], nt);
          compute_tile(cur, buf[k]);
        }
      }
    }
  };
  // Keys from cached_keys on are read nontemporally (all of them when NT):
  // pages shared through a prefix cache are leading pages, which the other
  // requests of a group read again, so the leading keys go through the caches
  // and the rest streams past them.
  if (NT || t_begin >= p.cached_keys)  // uniform over the work-group
    key_loop(std::true_type{});
  else
    key_loop(std::false_type{});

  // ---- reduce within the wave
  float l_w[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = 0.f;
#pragma unroll
    for (int u = 0; u < VPL; ++u) x += live(u) && h_of(u) == h ? l_acc[u] : 0.f;
    l_w[h] = wave_sum(x);
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] += shfl_xor_f(acc[h][e], m);
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) s_acc[wave][h][vc * EPC + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = m_ref[h];
      s_l[wave][h] = l_w[h];
    }
  }
  __syncthreads();

  // ---- merge the waves of each head and write the piece: query head
  // j = hh * G + h of the block (KV head gb * HB + hh) was served by waves
  // hh * WPH .. hh * WPH + WPH - 1
  const int64_t row0 = (int64_t)b * p.num_q_heads + (int64_t)gb * HB * G;     // workspace rows
  const int64_t orow0 = (int64_t)qrow * p.num_q_heads + (int64_t)gb * HB * G;  // output rows
  for (int idx = tid; idx < HB * G * D; idx += kThreads) {
    const int j = idx / D;
    const int d = idx - j * D;
    const int hh = j / G;
    const int h = j - hh * G;
    const int w0 = hh * WPH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPH; ++w) M = fmaxf(M, s_m[w0 + w][h]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < WPH; ++w) {
      const float f = fast_exp2(s_m[w0 + w][h] - M);
      lsum = fmaf(f, s_l[w0 + w][h], lsum);
      o = fmaf(f, s_acc[w0 + w][h][d], o);
    }
    o = o / lsum;
    if (single) {
      if constexpr (BF16)
        ((uint16_t*)p.out)[(orow0 + j) * D + d] = (uint16_t)f32_to_bf16_bits(o);
      else
        ((float*)p.out)[(orow0 + j) * D + d] = o;
    } else {
      const int64_t r = (row0 + j) * p.ws_pieces + p.piece_offset + s;
      p.o_part[r * D + d] = o;
      if (d == 0) p.lse[r] = M + __log2f(lsum);
    }
  }
}

// One wave per (request, query head): merge the request's pieces.  A row of
// the workspace holds, at indices [0, ng), the pieces of the shared-prefix
// pass (cascade decode only) and, from piece_offset on, the ns pieces of the
// request's own key range.  The log-sum-exp values of up to 64 pieces are
// read at once (one per lane), and the partial outputs in batches of eight
// independent loads, so the merge costs a few memory latencies, not one per
// piece.
constexpr int kFewPieces = 16;  // rows of at most this many pieces take the one-round-trip path

template <bool BF16, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeArgs p) {
  constexpr int EPL = D / 64;  // output elements per lane
  constexpr int BATCH = 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads;
  if (row >= rows) return;
  const int b = (int)(row / p.num_q_heads);
  int64_t orow = row;  // output row
  if (p.q_indptr) {
    const int r0 = p.q_indptr[b];
    if (p.q_indptr[b + 1] - r0 != 1) return;  // not a decode request of a mixed batch
    orow = (int64_t)r0 * p.num_q_heads + (row - (int64_t)b * p.num_q_heads);
  }
  const int L = p.seq_lens[b];
  const int k0 = p.key_begin ? max(p.key_begin[b], 0) : 0;
  // both counts are clamped to the pieces the workspace row holds
  const int ns = min(max(L - k0 + p.split_tokens - 1, 0) / p.split_tokens, p.max_splits);
  const int ng =
      p.group_lens ? min((p.group_lens[b] + p.group_piece_keys - 1) / p.group_piece_keys, p.piece_offset) : 0;
  if (ng == 0 && ns == 1 && !p.always_partial) return;  // written by the partial kernel
  const int n = ng + ns;
  const int off = p.piece_offset - ng;  // merged piece i >= ng sits at workspace index i + off
  const float* lse = p.lse + row * p.ws_pieces;
  const float* op = p.o_part + row * p.ws_pieces * D + lane * EPL;

  float res[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) res[e] = 0.f;
  if (n > 0 && n <= kFewPieces) {
    // every load issued at once: the log-sum-exps (lane i: piece i) and the
    // partial outputs of all pieces do not depend on each other, so the merge
    // waits for one memory round trip instead of three.  Same order of
    // operations as the general path below.
    const float l = lane < n ? lse[lane < ng ? lane : lane + off] : -INFINITY;
    float v[kFewPieces][EPL];
#pragma unroll
    for (int k = 0; k < kFewPieces; ++k) {
      if (k < n) {  // uniform
        const float* src = op + (int64_t)(k < ng ? k : k + off) * D;
        if constexpr (EPL == 2) {
          const float2 x = *(const float2*)src;
          v[k][0] = x.x;
          v[k][1] = x.y;
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[k][e] = src[e];
        }
      }
    }
    const float M = wave_max(l);
    if (M != -INFINITY) {
      const float w = (lane < n && l != -INFINITY) ? fast_exp2(l - M) : 0.f;
      const float wsum = wave_sum(w);
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
      for (int k = 0; k < kFewPieces; ++k) {
        if (k < n) {  // uniform
          const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[e] = wk > 0.f ? fmaf(wk, v[k][e], o[e]) : o[e];
        }
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) res[e] = o[e] / wsum;
    }
  } else if (n > 0) {
    // pieces with no visible key (lse = -inf) get weight zero
    float M = -INFINITY;
    for (int c = 0; c < n; c += 64) {
      const int i = min(c + lane, n - 1);
      M = fmaxf(M, lse[i < ng ? i : i + off]);
    }
    M = wave_max(M);
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    float wsum = 0.f;
    if (M != -INFINITY) {
      for (int c = 0; c < n; c += 64) {
        const int i = min(c + lane, n - 1);
        const float l = lse[i < ng ? i : i + off];
        const float w = (c + lane < n && l != -INFINITY) ? fast_exp2(l - M) : 0.f;
        wsum += w;
        const int cnt = min(64, n - c);
        for (int j0 = 0; j0 < cnt; j0 += BATCH) {
          float wk[BATCH], v[BATCH][EPL];
#pragma unroll
          for (int k = 0; k < BATCH; ++k) {
            const int j = min(j0 + k, cnt - 1);  // clamped: a real piece, weight zero below
            const int pi = c + j;
            const float* src = op + (int64_t)(pi < ng ? pi : pi + off) * D;
            wk[k] = j0 + k < cnt ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j))
                                 : 0.f;
            if constexpr (EPL == 2) {
              const float2 x = *(const float2*)src;
              v[k][0] = x.x;
              v[k][1] = x.y;
            } else {
#pragma unroll
              for (int e = 0; e < EPL; ++e) v[k][e] = src[e];
            }
          }
#pragma unroll
          for (int k = 0; k < BATCH; ++k)
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = wk[k] > 0.f ? fmaf(wk[k], v[k][e], o[e]) : o[e];
        }
      }
      wsum = wave_sum(wsum);
#pragma unroll
      for (int e = 0; e < EPL; ++e) res[e] = o[e] / wsum;
    }
  }
  if constexpr (BF16) {
    uint16_t* out = (uint16_t*)p.out + orow * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = (uint16_t)f32_to_bf16_bits(res[e]);
  } else {
    float* out = (float*)p.out + orow * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = res[e];
  }
}

template <bool BF16, int D, int G, bool NT, int HB>
hipError_t launch_partial_k(const DecodeArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.num_seqs * (a.num_kv_heads / HB) * a.max_splits;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_partial_kernel<BF16, D, G, NT, HB>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

template <bool BF16, int D, int G, bool NT>
hipError_t launch_partial_hb(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_kv_heads % a.heads_per_block != 0) return hipErrorInvalidValue;
  switch (a.heads_per_block) {
    case 1: return launch_partial_k<BF16, D, G, NT, 1>(a, stream);
    case 2: return launch_partial_k<BF16, D, G, NT, 2>(a, stream);
    case 4: return launch_partial_k<BF16, D, G, NT, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int D, int G>
hipError_t launch_partial_g(const DecodeArgs& a, hipStream_t stream) {
  // the cascade's own-keys pass (bf16, the group sizes it supports)
  if constexpr (BF16 && (G == 1 || G == 2 || G == 4 || G == 8)) {
    if (a.key_begin) return launch_partial_hb<BF16, D, G, true>(a, stream);
  }
  return launch_partial_hb<BF16, D, G, false>(a, stream);
}

template <bool BF16, int D>
hipError_t launch_partial_d(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  switch (G) {
    case 1: return launch_partial_g<BF16, D, 1>(a, stream);
    case 2: return launch_partial_g<BF16, D, 2>(a, stream);
    case 3: return launch_partial_g<BF16, D, 3>(a, stream);
    case 4: return launch_partial_g<BF16, D, 4>(a, stream);
    default: break;
  }
  if constexpr (BF16 || D == 64) {
    switch (G) {
      case 5: return launch_partial_g<BF16, D, 5>(a, stream);
      case 6: return launch_partial_g<BF16, D, 6>(a, stream);
      case 7: return launch_partial_g<BF16, D, 7>(a, stream);
      case 8: return launch_partial_g<BF16, D, 8>(a, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_plan(const PlanArgs& p, hipStream_t stream) {
  if (!p.plan || p.num_seqs <= 0 || p.max_splits <= 0) return hipSuccess;
  if (p.num_seqs <= 256)
    hipLaunchKernelGGL(decode_plan_kernel<256>, dim3(1), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_plan_kernel<1024>, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_plan_store(const PlanArgs& p, const StoreArgs& s, hipStream_t stream) {
  const bool plan = p.plan && p.num_seqs > 0 && p.max_splits > 0;
  const int64_t total = s.num_rows * s.row_chunks;
  if (!plan && total == 0) return hipSuccess;
  PlanArgs pp = p;
  if (!plan) pp.plan = nullptr;
  const int threads = plan && p.num_seqs > 256 ? 1024 : 256;
  int64_t store_blocks = (total + threads - 1) / threads;
  if (store_blocks > 8192) store_blocks = 8192;
  const dim3 grid((unsigned)(store_blocks + (plan ? 1 : 0)));
  if (threads == 256)
    hipLaunchKernelGGL(decode_plan_store_kernel<256>, grid, dim3(256), 0, stream, pp, s);
  else
    hipLaunchKernelGGL(decode_plan_store_kernel<1024>, grid, dim3(1024), 0, stream, pp, s);
  return hipGetLastError();
}

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim == 128) return launch_partial_d<true, 128>(a, stream);
    if (a.head_dim == 64) return launch_partial_d<true, 64>(a, stream);
  } else {
    if (a.head_dim == 128) return launch_partial_d<false, 128>(a, stream);
    if (a.head_dim == 64) return launch_partial_d<false, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (a.bf16) {
    if (a.head_dim == 128) hipLaunchKernelGGL((decode_combine_kernel<true, 128>), grid, dim3(256), 0, stream, a);
    else if (a.head_dim == 64) hipLaunchKernelGGL((decode_combine_kernel<true, 64>), grid, dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
  } else {
    if (a.head_dim == 128) hipLaunchKernelGGL((decode_combine_kernel<false, 128>), grid, dim3(256), 0, stream, a);
    else if (a.head_dim == 64) hipLaunchKernelGGL((decode_combine_kernel<false, 64>), grid, dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa

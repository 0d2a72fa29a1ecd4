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
// Design (FlashAttention-2 style tiling written for the CDNA4 matrix core):
//  * Work-group = 4 waves = 128 query rows = (128 / G) tokens x all G query
//    heads of one KV head, so every K/V tile staged in LDS serves G heads.
//  * Per wave: 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in
//    registers), so each lane owns one query row of the score tile and the
//    softmax needs only one cross-lane exchange (lane ^ 32).  The output is
//    also accumulated transposed, O^T += V^T P^T, so the rescale factor of a
//    query row is lane-local and P goes from the score accumulator to the
//    B operand without leaving registers.
//  * K tile [64 keys][D] in LDS with 16-byte pieces XOR-swizzled by key; V
//    tile stored transposed [D][64 keys] (transposed in registers on the way
//    in), with the keys of each 16-key group in the order the score
//    accumulator hands them to the B operand.  Two LDS buffers: the next
//    tile's global loads are in flight while the current tile is computed.
//  * Key tiles entirely above the diagonal are never visited; only tiles that
//    cross it are masked.
//  * Softmax in fp32 (base 2, scale folded with log2 e); P is rounded to bf16
//    for the matrix core; O accumulates in fp32 and is rounded once.
#include "device.h"
#include "internal.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kRows = 128;  // query rows per work-group
constexpr int kKT = 64;     // keys per tile

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

template <int D>
struct ExtCfg {
  static constexpr int PPR = D / 8;            // 16-byte pieces per K row
  static constexpr int KSTEPS = D / 16;        // MFMA k-steps over head_dim
  static constexpr int DT = D / 32;            // 32-row tiles of O^T
  static constexpr int K_LOADS = kKT * PPR / kThreads;        // K pieces per thread per tile
  static constexpr int VDG = D / 4;            // V load: groups of 4 head-dim elements
  static constexpr int V_ITEMS = VDG * 8;      // (dim group, 8-key piece) items per tile
  static constexpr int V_PASSES = (V_ITEMS + kThreads - 1) / kThreads;
  static_assert(K_LOADS >= 1, "tile too small");
  static_assert(V_ITEMS % kThreads == 0 || V_ITEMS < kThreads, "bad V split");
};

// Swizzled position (in 16-byte units) of piece `pc` of K row `key`.
template <int D>
__device__ __forceinline__ int k_lds_off(int key, int pc) {
  constexpr int PPR = D / 8;
  return key * PPR + (pc ^ (key & (PPR - 1)));
}
// Swizzled position of key piece `kp` (0..7) of V^T row `d`.
__device__ __forceinline__ int v_lds_off(int d, int kp) { return d * 8 + (kp ^ (d & 7)); }

template <int D>
struct Staged {
  uint4 k[ExtCfg<D>::K_LOADS];
  uint2 v[ExtCfg<D>::V_PASSES][8];
};

// Byte permute (v_perm_b32): result byte i = byte sel[i] of the 8-byte value
// {hi, lo} (lo = bytes 0..3).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
constexpr uint32_t kLoHalves = 0x05040100u;  // {lo.lo16, hi.lo16}
constexpr uint32_t kHiHalves = 0x07060302u;  // {lo.hi16, hi.hi16}

constexpr float kExtRescaleSlack = 8.0f;  // log2 units, as in decode

template <int D, int G>
__global__ __launch_bounds__(kThreads) void extend_kernel(const ExtendArgs p) {
  using C = ExtCfg<D>;
  constexpr int TOK = kRows / G;  // tokens per work-group
  constexpr int KSTEPS = C::KSTEPS, DT = C::DT, PPR = C::PPR;

  __shared__ uint4 s_k[2][kKT * PPR];
  __shared__ uint4 s_v[2][D * 8];
  __shared__ int32_t s_slot[3][kKT];  // flat slots of the keys of tiles t, t+1, t+2

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query row within the wave
  const int half = lane >> 5;

  // ---- work-group coordinates: the token blocks of one (request, KV head)
  // are consecutive ids, heaviest (latest) first
  const int qblocks = (p.max_q_len + TOK - 1) / TOK;
  int bid = blockIdx.x;
  const int qb = qblocks - 1 - (bid % qblocks);
  bid /= qblocks;
  const int g = bid % p.num_kv_heads;
  const int b = bid / p.num_kv_heads;

  const int r0 = p.q_indptr[b];
  const int n = p.q_indptr[b + 1] - r0;
  const int i0 = qb * TOK;
  if (i0 >= n) return;
  const int L = p.seq_lens[b];
  const int prefix = L - n;
  const int kv_len = prefix + min(i0 + TOK, n);  // keys this block can see
  const int ntiles = (kv_len + kKT - 1) / kKT;

  // ---- this lane's query row: rows are (head, token) with token fastest
  const int row = wave * 32 + col;
  const int hq = row / TOK;
  const int ti = i0 + (row % TOK);
  const bool qvalid = ti < n;
  const int tmask = qvalid ? ti : (n - 1);  // padding rows mask like the last token
  const int vis_lim = prefix + tmask;        // last visible key of this row

  uint4 qreg[KSTEPS];
  {
    const uint16_t* qp =
        (const uint16_t*)p.q + ((int64_t)(r0 + ti) * p.num_q_heads + (int64_t)g * G + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qreg[ks] = qvalid ? *(const uint4*)(qp + ks * 16 + half * 8) : make_uint4(0, 0, 0, 0);
  }

  const int32_t* pt = p.page_table + (int64_t)b * p.pt_stride;
  const int sh = p.log2_page;
  const int pmask = (1 << sh) - 1;
  const int64_t row_stride = (int64_t)p.num_kv_heads * D;  // elements per slot
  const uint16_t* kbase = (const uint16_t*)p.k_pool + (int64_t)g * D;
  const uint16_t* vbase = (const uint16_t*)p.v_pool + (int64_t)g * D;

  // Slot of key (t*64 + tid) for the first 64 threads; keys past the block's
  // range are clamped to its last key (a real row; masked out later), so no
  // page-table entry past the request's pages is read.
  auto slot_of = [&](int t) -> int32_t {
    const int kk = min(t * kKT + tid, kv_len - 1);
    return (pt[kk >> sh] << sh) | (kk & pmask);
  };

  // Global loads of tile t into registers; slots come from LDS.
  auto load_tile = [&](int t, Staged<D>& st) {
    const int32_t* sl = s_slot[t % 3];
#pragma unroll
    for (int j = 0; j < C::K_LOADS; ++j) {
      const int idx = j * kThreads + tid;
      st.k[j] = *(const uint4*)(kbase + (int64_t)sl[idx / PPR] * row_stride + (idx % PPR) * 8);
    }
    // V: an item is 4 head-dim elements of the 8 keys forming one transposed
    // piece: keys 16*(kp/2) + 4*(kp%2) + {0,1,2,3,8,9,10,11}.
#pragma unroll
    for (int ps = 0; ps < C::V_PASSES; ++ps) {
      const int item = ps * kThreads + tid;
      if (item >= C::V_ITEMS) break;
      const int dg = item % C::VDG;
      const int kp = item / C::VDG;
      const int k16 = 16 * (kp >> 1) + 4 * (kp & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        st.v[ps][e] = *(const uint2*)(vbase + (int64_t)sl[k16 + (e & 3) + ((e >> 2) << 3)] * row_stride + dg * 4);
    }
  };

  auto store_tile = [&](int buf, const Staged<D>& st) {
#pragma unroll
    for (int j = 0; j < C::K_LOADS; ++j) {
      const int idx = j * kThreads + tid;
      s_k[buf][k_lds_off<D>(idx / PPR, idx % PPR)] = st.k[j];
    }
#pragma unroll
    for (int ps = 0; ps < C::V_PASSES; ++ps) {
      const int item = ps * kThreads + tid;
      if (item >= C::V_ITEMS) break;
      const int dg = item % C::VDG;
      const int kp = item / C::VDG;
      const uint2* x = st.v[ps];
      // transpose 8 keys x 4 dims -> 4 rows (dims) of 8 keys
      uint4 r[4];
      r[0] = make_uint4(perm(x[1].x, x[0].x, kLoHalves), perm(x[3].x, x[2].x, kLoHalves),
                        perm(x[5].x, x[4].x, kLoHalves), perm(x[7].x, x[6].x, kLoHalves));
      r[1] = make_uint4(perm(x[1].x, x[0].x, kHiHalves), perm(x[3].x, x[2].x, kHiHalves),
                        perm(x[5].x, x[4].x, kHiHalves), perm(x[7].x, x[6].x, kHiHalves));
      r[2] = make_uint4(perm(x[1].y, x[0].y, kLoHalves), perm(x[3].y, x[2].y, kLoHalves),
                        perm(x[5].y, x[4].y, kLoHalves), perm(x[7].y, x[6].y, kLoHalves));
      r[3] = make_uint4(perm(x[1].y, x[0].y, kHiHalves), perm(x[3].y, x[2].y, kHiHalves),
                        perm(x[5].y, x[4].y, kHiHalves), perm(x[7].y, x[6].y, kHiHalves));
#pragma unroll
      for (int i = 0; i < 4; ++i) s_v[buf][v_lds_off(dg * 4 + i, kp)] = r[i];
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
  const float slack = kExtRescaleSlack / sl2;  // the same slack in raw-score units

  // ---- prologue: slots of tiles 0 and 1, then tile 0 into LDS
  if (tid < kKT) {
    s_slot[0][tid] = slot_of(0);
    if (ntiles > 1) s_slot[1][tid] = slot_of(1);
  }
  __syncthreads();
  {
    Staged<D> st;
    load_tile(0, st);
    store_tile(0, st);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    Staged<D> st;
    const bool more = (t + 1) < ntiles;
    if (more) load_tile(t + 1, st);
    int32_t next_slot = 0;
    const bool fill = (t + 2) < ntiles && tid < kKT;
    if (fill) next_slot = slot_of(t + 2);

    // ---- S^T = K Q^T for two 32-key halves of the tile
    f32x16_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
      const int key = kt * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const uint4 a = s_k[buf][k_lds_off<D>(key, 2 * ks + half)];
        s[kt] = mfma32(a, qreg[ks], s[kt]);
      }
    }

    // ---- causal mask, only on tiles that cross the diagonal (block-uniform)
    const int kt0 = t * kKT;
    if (kt0 + kKT - 1 > prefix + i0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > vis_lim) s[kt][r] = -INFINITY;
        }
    }

    // ---- online softmax (lane owns one query row, half of the tile's keys);
    // the reference maximum moves only when exceeded by the slack
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (__ballot(mx > m_ref + slack) != 0) {
      const float m_new = fmaxf(m_ref, mx);  // finite: key 0 of tile 0 is visible to every row
      const float alpha = fast_exp2((m_ref - m_new) * sl2);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
    const float mb = -m_ref * sl2;
    uint4 pb[4];  // B operands of the four 16-key steps
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[r] = fast_exp2(fmaf(s[kt][r], sl2, mb));
        l_run += e[r];
      }
      pb[2 * kt + 0] = make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
      pb[2 * kt + 1] =
          make_uint4(pack2(e[8], e[9]), pack2(e[10], e[11]), pack2(e[12], e[13]), pack2(e[14], e[15]));
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int i = 0; i < DT; ++i) {
      const int d = i * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = s_v[buf][v_lds_off(d, 2 * ks + half)];
        o[i] = mfma32(a, pb[ks], o[i]);
      }
    }

    if (more) store_tile(buf ^ 1, st);
    if (fill) s_slot[(t + 2) % 3][tid] = next_slot;
    __syncthreads();
  }

  // ---- normalise and write this lane's row
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  uint16_t* op = (uint16_t*)p.out + ((int64_t)(r0 + ti) * p.num_q_heads + (int64_t)g * G + hq) * D;
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

template <int D, int G>
hipError_t launch_g(const ExtendArgs& a, hipStream_t stream) {
  constexpr int TOK = kRows / G;
  const int64_t qblocks = (a.max_q_len + TOK - 1) / TOK;
  const int64_t blocks = qblocks * a.num_kv_heads * a.num_seqs;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((extend_kernel<D, G>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ExtendArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<D, 1>(a, stream);
    case 2: return launch_g<D, 2>(a, stream);
    case 4: return launch_g<D, 4>(a, stream);
    case 8: return launch_g<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

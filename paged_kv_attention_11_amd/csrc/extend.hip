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

template <int D, int G>
__global__ __launch_bounds__(kThreads) void extend_kernel(const ExtendArgs p) {
  using C = ExtCfg<D>;
  constexpr int TOK = kRows / G;  // tokens per work-group
  constexpr int KSTEPS = C::KSTEPS, DT = C::DT, PPR = C::PPR;

  __shared__ uint4 s_k[2][kKT * PPR];
  __shared__ uint4 s_v[2][D * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // Global loads of one key tile into registers.
  auto load_tile = [&](int t, Staged<D>& st) {
    const int kt0 = t * kKT;
#pragma unroll
    for (int j = 0; j < C::K_LOADS; ++j) {
      const int idx = j * kThreads + tid;
      const int key = idx / PPR;
      const int pc = idx % PPR;
      const int kk = kt0 + key;
      if (kk < kv_len) {
        const int64_t slot = ((int64_t)pt[kk >> sh] << sh) | (kk & pmask);
        st.k[j] = *(const uint4*)(kbase + slot * row_stride + pc * 8);
      } else {
        st.k[j] = make_uint4(0, 0, 0, 0);
      }
    }
    // V: an item is 4 head-dim elements of the 8 keys forming one transposed
    // piece: keys 16*(kp/2) + 4*(kp%2) + {0,1,2,3,8,9,10,11}.
#pragma unroll
    for (int ps = 0; ps < C::V_PASSES; ++ps) {
      const int item = ps * kThreads + tid;
      if (item >= C::V_ITEMS) break;
      const int dg = item % C::VDG;
      const int kp = item / C::VDG;
      const int kbase16 = 16 * (kp >> 1) + 4 * (kp & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = kt0 + kbase16 + (e & 3) + ((e >> 2) << 3);
        if (kk < kv_len) {
          const int64_t slot = ((int64_t)pt[kk >> sh] << sh) | (kk & pmask);
          st.v[ps][e] = *(const uint2*)(vbase + slot * row_stride + dg * 4);
        } else {
          st.v[ps][e] = make_uint2(0, 0);
        }
      }
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
      r[0] = make_uint4((x[0].x & 0xffffu) | (x[1].x << 16), (x[2].x & 0xffffu) | (x[3].x << 16),
                        (x[4].x & 0xffffu) | (x[5].x << 16), (x[6].x & 0xffffu) | (x[7].x << 16));
      r[1] = make_uint4((x[0].x >> 16) | (x[1].x & 0xffff0000u), (x[2].x >> 16) | (x[3].x & 0xffff0000u),
                        (x[4].x >> 16) | (x[5].x & 0xffff0000u), (x[6].x >> 16) | (x[7].x & 0xffff0000u));
      r[2] = make_uint4((x[0].y & 0xffffu) | (x[1].y << 16), (x[2].y & 0xffffu) | (x[3].y << 16),
                        (x[4].y & 0xffffu) | (x[5].y << 16), (x[6].y & 0xffffu) | (x[7].y << 16));
      r[3] = make_uint4((x[0].y >> 16) | (x[1].y & 0xffff0000u), (x[2].y >> 16) | (x[3].y & 0xffff0000u),
                        (x[4].y >> 16) | (x[5].y & 0xffff0000u), (x[6].y >> 16) | (x[7].y & 0xffff0000u));
#pragma unroll
      for (int i = 0; i < 4; ++i) s_v[buf][v_lds_off(dg * 4 + i, kp)] = r[i];
    }
  };

  f32x16_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY;  // running maximum of this row (log2 domain)
  float l_run = 0.f;        // this lane's half of the running sum
  const float sl2 = p.scale_log2;

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

    // ---- mask, online softmax (lane owns one query row, half the keys)
    const int kt0 = t * kKT;
    const bool diag = kt0 + kKT - 1 > prefix + i0;  // tile may cross the diagonal
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[kt][r] * sl2;
        if (diag) {
          const int key = kt0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > vis_lim) v = -INFINITY;
        }
        s[kt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: key 0 of tile 0 is visible to every row
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
    uint4 pb[4];  // B operands of the four 16-key steps
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[r] = fast_exp2(s[kt][r] - m_new);
        lsum += e[r];
      }
      pb[2 * kt + 0] = make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
      pb[2 * kt + 1] =
          make_uint4(pack2(e[8], e[9]), pack2(e[10], e[11]), pack2(e[12], e[13]), pack2(e[14], e[15]));
    }
    l_run = l_run * alpha + lsum;

    // ---- O^T = alpha * O^T + V^T P^T
#pragma unroll
    for (int i = 0; i < DT; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      const int d = i * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = s_v[buf][v_lds_off(d, 2 * ks + half)];
        o[i] = mfma32(a, pb[ks], o[i]);
      }
    }

    if (more) store_tile(buf ^ 1, st);
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

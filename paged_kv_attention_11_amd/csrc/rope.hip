// Rotary position embedding fused with the KV-cache store: the step just
// before attention.  For every live row (slot >= 0) of the step:
//   q_out[n]          = rope(q[n],     positions[n])   all query heads
//   k_pool[slot[n]]   = rope(k_new[n], positions[n])   all KV heads
//   v_pool[slot[n]]   = v_new[n]                       byte copy
// Pairing is half-split: channel i turns with channel i + D/2 (the
// rotate_half convention; nanoSGLang README, section Notable Fixes, records
// the bug of pairing neighbours), by the angle whose cosine and sine the
// caller's tables hold for (position, i).  The store is the KV-cache write of
// "mini-sglang from Scratch", section "How this book works".
//
// One thread owns 16 bytes of a head's first half and the matching 16 bytes
// of its second half (8 bf16 or 4 fp32 pairs), so every load and store is a
// whole 16-byte vector and consecutive threads cover consecutive bytes.  The
// arithmetic is fp32 (a*c - b*s with one fused multiply-add), rounded once to
// the storage format.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

template <bool BF16>
struct RopeCfg {
  static constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
};

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4& v, float* f) {
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

template <bool BF16>
__device__ __forceinline__ uint4 pack(const float* f) {
  if constexpr (BF16) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  } else {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
}

// Nontemporal 16-byte store (streamed past the caches): the rotated rows are
// not read again by this kernel.  On the Qwen3-8B-shaped chunked-prefill
// rows: 18.5 us against 19.4 us with cached stores; nontemporal loads of the
// inputs (which the step producing them leaves in the caches) were slower,
// 22.9 us.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(void* p, const uint4& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), (u32x4_t*)p);
}

// Work item = (row, head slot, vector c of the first half).  Head slots
// [0, Hq) rotate q, [Hq, Hq + Hkv) rotate k into the pool, [Hq + Hkv,
// Hq + 2 Hkv) copy v into the pool.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void rope_store_kernel(const RopeArgs a) {
  using T = std::conditional_t<BF16, uint16_t, float>;
  constexpr int EPV = RopeCfg<BF16>::EPV;
  constexpr int HALF = D / 2;
  constexpr int VPH = HALF / EPV;  // vectors per half head
  const int heads = a.num_q_heads + 2 * a.num_kv_heads;
  const int64_t total = a.num_rows * heads * VPH;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % VPH);
    const int64_t rh = i / VPH;
    const int h = (int)(rh % heads);
    const int64_t n = rh / heads;
    const int64_t slot = a.slot_mapping[n];
    if (slot < 0) continue;  // padding row: nothing read or written
    const int e0 = c * EPV;  // first channel of this thread's pairs
    if (h >= a.num_q_heads + a.num_kv_heads) {  // v: plain copy of both halves
      const int hv = h - a.num_q_heads - a.num_kv_heads;
      const T* src = (const T*)a.v_new + (n * a.num_kv_heads + hv) * D;
      T* dst = (T*)a.v_pool + (slot * a.num_kv_heads + hv) * D;
      store_nt(dst + e0, *(const uint4*)(src + e0));
      store_nt(dst + HALF + e0, *(const uint4*)(src + HALF + e0));
      continue;
    }
    const T* src;
    T* dst;
    if (h < a.num_q_heads) {
      src = (const T*)a.q + (n * a.num_q_heads + h) * D;
      dst = (T*)a.q_out + (n * a.num_q_heads + h) * D;
    } else {
      const int hk = h - a.num_q_heads;
      src = (const T*)a.k_new + (n * a.num_kv_heads + hk) * D;
      dst = (T*)a.k_pool + (slot * a.num_kv_heads + hk) * D;
    }
    // positions outside the table are clamped: a contract violation gives
    // wrong values, never an out-of-bounds read
    const int pos = min(max(a.positions[n], 0), a.max_position - 1);
    const float* ct = a.cos_table + (int64_t)pos * HALF + e0;
    const float* st = a.sin_table + (int64_t)pos * HALF + e0;
    float x0[EPV], x1[EPV], cs[EPV], sn[EPV], y0[EPV], y1[EPV];
    unpack<BF16>(*(const uint4*)(src + e0), x0);
    unpack<BF16>(*(const uint4*)(src + HALF + e0), x1);
#pragma unroll
    for (int k = 0; k < EPV; k += 4) {
      const float4 cv = *(const float4*)(ct + k);
      const float4 sv = *(const float4*)(st + k);
      cs[k] = cv.x; cs[k + 1] = cv.y; cs[k + 2] = cv.z; cs[k + 3] = cv.w;
      sn[k] = sv.x; sn[k + 1] = sv.y; sn[k + 2] = sv.z; sn[k + 3] = sv.w;
    }
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      y0[k] = fmaf(x0[k], cs[k], -(x1[k] * sn[k]));
      y1[k] = fmaf(x1[k], cs[k], x0[k] * sn[k]);
    }
    store_nt(dst + e0, pack<BF16>(y0));
    store_nt(dst + HALF + e0, pack<BF16>(y1));
  }
}

template <bool BF16>
hipError_t launch_rope_t(const RopeArgs& a, hipStream_t stream) {
  constexpr int EPV = RopeCfg<BF16>::EPV;
  const int vph = a.head_dim / 2 / EPV;
  const int64_t total = a.num_rows * (a.num_q_heads + 2 * a.num_kv_heads) * vph;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 16384) blocks = 16384;
  if (a.head_dim == 128)
    hipLaunchKernelGGL((rope_store_kernel<BF16, 128>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((rope_store_kernel<BF16, 64>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_store(const RopeArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_rope_t<true>(a, stream) : launch_rope_t<false>(a, stream);
}

}  // namespace pa

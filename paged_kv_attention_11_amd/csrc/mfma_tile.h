// Building blocks shared by the matrix-core attention kernels (extend,
// cascade prefix pass, verify): bf16 MFMA wrappers, the 64-key K/V tile
// staged in LDS by direct-to-LDS loads, its swizzles, and the transposing
// LDS read that feeds V^T to the matrix core.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace pa {
namespace tile {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKT = 64;            // keys per tile
constexpr int kTileThreads = 256;  // work-group size of the tile kernels (4 waves)

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
  static constexpr int PPR = D / 8;          // 16-byte pieces per K/V row
  static constexpr int KSTEPS = D / 16;      // MFMA k-steps over head_dim
  static constexpr int DT = D / 32;          // 32-row tiles of O^T
  static constexpr int RPB = 64 / PPR;       // rows per 1 KB LDS block (one DMA instruction)
  static constexpr int NDMA = kKT * PPR / kTileThreads;  // DMA instructions per thread per tile, per tensor
  static_assert(NDMA >= 1 && kKT * PPR % kTileThreads == 0, "bad tile");
};

constexpr int kPageCap = 1024;  // page ids staged in LDS at a time

// K rows: 16-byte piece p of key k is stored at piece p ^ (k mod PPR), so the
// 32 keys read by one MFMA operand fetch hit distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int key) { return key & (ExtCfg<D>::PPR - 1); }
// V rows: piece p of key k at p ^ v_swz(k), an XOR-linear function of the
// key's low three bits.  For D = 128 (four 64-byte blocks per row) bit 0
// moves the 64-byte block by one, bit 1 by two and the 16-byte chunk by two,
// bit 2 the chunk by two; for D = 64, pieces 2, 4 and 2.  Both transposing
// read patterns that use the layout (extend: lanes over 4 keys x 64 bytes,
// twice; verify: lanes over 8 keys x 32 bytes) then fall on distinct LDS
// banks, with 32 banks and with 64 (checked exhaustively on the CPU).
template <int D>
__device__ __forceinline__ int v_swz(int key) {
  const int b2 = 2 * ((key >> 2) & 1);
  if constexpr (ExtCfg<D>::PPR == 16)
    return (4 * (key & 3) + 2 * ((key >> 1) & 1)) ^ b2;
  else
    return (2 * (key & 3)) ^ b2;
}

__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's 16 bytes land at LDS address `lds` + 16 i.  Issued as inline asm
// without a memory clobber, so that the compiler's wait-count pass does not
// serialise it against unrelated LDS reads and may move ordinary LDS reads
// across it: for rings whose slots being filled are never read before the
// next barrier.  Completion is awaited explicitly with vm_wait below;
// ordering against the waits and barriers is kept (both are volatile).
__device__ __forceinline__ void dma16_unordered(uint32_t lds, const void* gptr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gptr) : "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j supplies the address of 4 consecutive 16-bit values; lane i receives
// value (i mod 4) of the chunks of lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ uint2 lds_read_tr16(const void* ptr) {
#if defined(__HIP_DEVICE_COMPILE__)
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)ptr);
  return __builtin_bit_cast(uint2, v);
#else
  (void)ptr;
  return make_uint2(0, 0);
#endif
}

// Work-group ids go to the chip's 8 XCDs in turn (id i to XCD i mod 8).
// Renumbered by this bijection, XCD x runs one contiguous range of logical
// ids, in order, so work-groups that read the same keys share its L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int nblocks) {
  constexpr int kXcds = 8;
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  const int x = bid % kXcds, local = bid / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

}  // namespace tile
}  // namespace pa

// Store of new K/V rows into the paged pool, and the gather of requests'
// pages back to contiguous rows.
//
// Store: the KV-cache write of each step ("mini-sglang from Scratch", section
// "How this book works"); row i goes to flat slot slot_mapping[i], slots below
// zero are padding.  Gather: the per-token copy out of the cache that the
// legacy engine did every layer (nanoSGLang README, section Ablation); here it
// is only a test of the page-table addressing and a bandwidth calibration.
//
// Both are plain byte copies: one 16-byte vector per lane, consecutive lanes
// on consecutive 16-byte pieces of a row, so every wavefront load and store
// covers whole 128-byte cache lines.
#include "internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void kv_store_kernel(const uint4* __restrict__ k_new,
                                                            const uint4* __restrict__ v_new,
                                                            const int64_t* __restrict__ slots,
                                                            uint4* __restrict__ k_pool,
                                                            uint4* __restrict__ v_pool,
                                                            int64_t total, int32_t row_chunks) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / row_chunks;
    const int64_t c = i - row * row_chunks;
    const int64_t slot = slots[row];
    if (slot < 0) continue;
    const int64_t dst = slot * row_chunks + c;
    k_pool[dst] = k_new[i];
    v_pool[dst] = v_new[i];
  }
}

// grid: (x = token blocks of the longest request, y = request).  A thread
// owns one 16-byte piece of a row; `tpi` whole rows are copied per block
// iteration (one row-piece per thread, so no division inside the loop).
__global__ __launch_bounds__(kThreads) void gather_kernel(const uint4* __restrict__ k_pool,
                                                          const uint4* __restrict__ v_pool,
                                                          const int32_t* __restrict__ page_table,
                                                          const int32_t* __restrict__ seq_lens,
                                                          const int64_t* __restrict__ out_offsets,
                                                          uint4* __restrict__ k_out,
                                                          uint4* __restrict__ v_out, int64_t pt_stride,
                                                          int32_t log2_page, int32_t row_chunks) {
  const int b = blockIdx.y;
  const int L = seq_lens[b];
  const int32_t* pt = page_table + (int64_t)b * pt_stride;
  const int32_t pmask = (1 << log2_page) - 1;
  const int64_t base = out_offsets[b];
  const int rc = row_chunks;
  const bool small = rc <= kThreads;
  const int tpi = small ? kThreads / rc : 1;           // rows per block iteration
  const int t_off = small ? (int)threadIdx.x / rc : 0;  // this thread's row in the iteration
  const int c0 = small ? (int)threadIdx.x - t_off * rc : (int)threadIdx.x;
  const int cstep = small ? rc : kThreads;
  if (t_off >= tpi) return;
#pragma unroll 4
  for (int t = blockIdx.x * tpi + t_off; t < L; t += gridDim.x * tpi) {
    const int64_t slot = ((int64_t)pt[t >> log2_page] << log2_page) | (t & pmask);
    const int64_t src = slot * rc;
    const int64_t dst = (base + t) * rc;
    for (int c = c0; c < rc; c += cstep) {
      k_out[dst + c] = k_pool[src + c];
      v_out[dst + c] = v_pool[src + c];
    }
  }
}

// Read-only streaming calibration.  The buffer is cut into chunks of
// kReadChunk 16-byte pieces (32 KB) and every work-group reads its own run of
// consecutive chunks, one chunk per iteration: wave w of the work-group reads
// the 8 KB of the chunk from byte 8 KB w, lane l the 16 bytes at 1 KB u +
// 16 l of it for u < kReadUnroll, all loads issued before any is used.  The
// XOR of what it read is folded over the work-group and one lane ORs it into
// the sink, so no load is dead.  The loads are nontemporal (streamed past
// the caches), the fastest of the forms measured: on one MI355X, 7.1-7.2 TB/s
// against 6.3-6.4 TB/s with ordinary loads, with 4, 8 or 16 work-groups per
// compute unit and 4 to 16 loads in flight per lane.  Measures the HBM read
// rate the device reaches, the ceiling the streaming kernels are compared
// with.
constexpr int kReadUnroll = 8;
constexpr int64_t kReadChunk = (int64_t)kThreads * kReadUnroll;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_x[kThreads / 64];
  uint32_t x = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nfull = n16 / kReadChunk;  // whole chunks
  const int64_t per = (nfull + gridDim.x - 1) / gridDim.x;  // chunks per work-group
  const int64_t c0 = (int64_t)blockIdx.x * per;
  const int64_t c1 = c0 + per < nfull ? c0 + per : nfull;
  for (int64_t c = c0; c < c1; ++c) {
    const uint4* p = src + c * kReadChunk + wave * (kReadUnroll * 64) + lane;
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(p + u * 64)));
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the pieces after the last whole chunk
  for (int64_t i = nfull * kReadChunk + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 v = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(src + i)));
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  if (lane == 0) s_x[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t ^= s_x[w];
    atomicOr(sink, t | 1u);
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // eight 256-thread work-groups per compute unit: enough loads in flight
  int64_t blocks = (int64_t)cus * 8;
  const int64_t need = (n16 + kThreads - 1) / kThreads;
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, (const uint4*)src, n16,
                     sink);
  return hipGetLastError();
}

hipError_t launch_kv_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t total = a.num_rows * a.row_chunks;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     (const uint4*)a.k_new, (const uint4*)a.v_new, a.slot_mapping, (uint4*)a.k_pool,
                     (uint4*)a.v_pool, total, a.row_chunks);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_seq_len == 0) return hipSuccess;
  const int tpi = a.row_chunks <= kThreads ? kThreads / a.row_chunks : 1;
  int64_t blocks = ((int64_t)a.max_seq_len + tpi - 1) / tpi;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks, (unsigned)a.num_seqs), dim3(kThreads), 0,
                     stream, (const uint4*)a.k_pool, (const uint4*)a.v_pool, a.page_table, a.seq_lens,
                     a.out_offsets, (uint4*)a.k_out, (uint4*)a.v_out, a.pt_stride, a.log2_page,
                     a.row_chunks);
  return hipGetLastError();
}

}  // namespace pa

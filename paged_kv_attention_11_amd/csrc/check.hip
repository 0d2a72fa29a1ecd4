// Debug check of the device-resident parts of a batch, the values the other
// calls take on trust (page ids, lengths, chunk offsets, slots).  The pages
// record what unchecked state costs an engine: KV-block exhaustion that
// killed the engine loop (nanoSGLang README, section Notable Fixes) and pages
// freed twice on abort ("mini-sglang from Scratch", section "Where we
// differ").  This call reads only the tables it is given -- never a pool page
// -- so it is safe on exactly the inputs it exists to catch, and reports what
// it found as bits of one word in device memory.
#include "internal.h"
#include "pagedattn.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

__global__ void clear_flags(uint32_t* flags) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *flags = 0u;
}

// One thread per (request, page slot of the table row): lengths, chunk
// offsets and the page ids a request's keys use.
__global__ __launch_bounds__(kThreads) void check_requests(const CheckArgs a) {
  const int64_t total = (int64_t)a.num_seqs * a.pt_stride;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int b = (int)(i / a.pt_stride);
    const int j = (int)(i - (int64_t)b * a.pt_stride);
    const int L = a.seq_lens[b];
    if (j == 0) {
      if (L < 0 || L > a.max_seq_len) bad |= PA_CHECK_SEQ_LEN;
      if (a.q_indptr) {
        const int n = a.q_indptr[b + 1] - a.q_indptr[b];
        if (n < 0 || n > L || n > a.max_q_len) bad |= PA_CHECK_Q_INDPTR;
        if (b == 0 && a.q_indptr[0] != 0) bad |= PA_CHECK_Q_INDPTR;
      }
    }
    const int Lc = min(max(L, 0), a.max_seq_len);  // pages the calls would read
    if ((int64_t)j * a.page_size < Lc) {
      const int32_t page = a.page_table[i];
      if (page < 0 || page >= a.num_pages) bad |= PA_CHECK_PAGE_ID;
    }
  }
  if (bad) atomicOr(a.flags, bad);
}

// Slots: in range, and no live slot twice (pairwise, for a debug check).
__global__ __launch_bounds__(kThreads) void check_slots(const CheckArgs a) {
  const int64_t n = a.num_rows;
  const int64_t slots = a.num_pages * a.page_size;
  uint32_t bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t s = a.slot_mapping[i];
    if (s >= slots) bad |= PA_CHECK_SLOT_RANGE;
    if (s < 0) continue;
    for (int64_t k = i + 1; k < n; ++k)
      if (a.slot_mapping[k] == s) {
        bad |= PA_CHECK_SLOT_DUPLICATE;
        break;
      }
  }
  if (bad) atomicOr(a.flags, bad);
}

// One thread per request of a cascade decode: its group (found by binary
// search in group_starts, which one thread checks whole), its shared length,
// and that the pages holding its shared keys are its group's prefix pages.
__global__ __launch_bounds__(kThreads) void check_groups(const CascadeCheckArgs a) {
  uint32_t bad = 0;
  const int tid = blockIdx.x * kThreads + threadIdx.x;
  if (tid == 0) {
    if (a.group_starts[0] != 0 || a.group_starts[a.num_groups] != a.num_seqs) bad |= PA_CHECK_GROUP_STARTS;
    for (int j = 0; j < a.num_groups; ++j) {
      const int n = a.group_starts[j + 1] - a.group_starts[j];
      if (n < 0 || n > a.max_group_size) bad |= PA_CHECK_GROUP_STARTS;
    }
  }
  for (int b = tid; b < a.num_seqs; b += gridDim.x * kThreads) {
    // the last group whose start is <= b (any in-range group if the starts
    // are broken: that is reported above)
    int lo = 0, hi = a.num_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.group_starts[mid] <= b) lo = mid;
      else hi = mid - 1;
    }
    const int sh = a.shared_lens[b];
    const int L = a.seq_lens[b];
    if (sh < 0 || sh > a.max_shared_len || sh > L) bad |= PA_CHECK_SHARED_LEN;
    // pages of the shared keys the calls would read, within both table rows
    const int64_t keys = min(max(sh, 0), a.max_shared_len);
    int64_t np = (keys + a.page_size - 1) / a.page_size;
    np = min(np, (int64_t)min(a.pt_stride, a.prefix_pt_stride));
    const int32_t* own = a.page_table + (int64_t)b * a.pt_stride;
    const int32_t* pre = a.prefix_page_table + (int64_t)lo * a.prefix_pt_stride;
    for (int64_t t = 0; t < np; ++t) {
      const int32_t pg = pre[t];
      if (pg < 0 || pg >= a.num_pages || pg != own[t]) {
        bad |= PA_CHECK_PREFIX_PAGE;
        break;
      }
    }
  }
  if (bad) atomicOr(a.flags, bad);
}

}  // namespace

hipError_t launch_check_cascade(const CascadeCheckArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(clear_flags, dim3(1), dim3(64), 0, stream, a.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_seqs <= 0 || a.num_groups <= 0) return e;
  const int64_t want = (a.num_seqs + kThreads - 1) / kThreads;
  const int64_t blocks = want < 1024 ? want : 1024;
  hipLaunchKernelGGL(check_groups, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(clear_flags, dim3(1), dim3(64), 0, stream, a.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t reqs = (int64_t)a.num_seqs * a.pt_stride;
  if (reqs > 0) {
    const int64_t want = (reqs + kThreads - 1) / kThreads;
    const int64_t blocks = want < 4096 ? want : 4096;
    hipLaunchKernelGGL(check_requests, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.slot_mapping && a.num_rows > 0) {
    const int64_t want = (a.num_rows + kThreads - 1) / kThreads;
    const int64_t blocks = want < 4096 ? want : 4096;
    hipLaunchKernelGGL(check_slots, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pa

// Work order of the split-K decode partial kernel, built on the device by one
// work-group: the decode kernel's own plan kernel, or one extra work-group of
// the cascade's shared-prefix pass (which runs just before the partial kernel
// and leaves most of the chip idle).
//
// Entry i of the order is the piece that work-groups i * nb .. i * nb + nb - 1
// take (nb blocks of neighbouring KV heads, one work-group each): {request,
// piece | kPlanSingle when it is the request's only piece and finishes the
// output, first key, keys}; keys = 0 marks a request
// with no keys that gets a zero row; request -1 marks no work.  Order: every
// full piece (split_tokens keys) in request order, then the shorter last
// pieces by decreasing key count in classes of kPlanClassKeys keys (request
// order within a class), then the zero rows, then empty entries up to
// max_splits x num_seqs.  Longest first: the short pieces run at the end,
// where they fill the gaps the long ones leave, and the grid holds no
// work-groups for pieces past a request's end before the last real one.
// Read-only probes of this access pattern on the Qwen3-8B-shaped radix batch
// (log-uniform lengths) moved 5.44 TB/s with the pieces in grid order among
// the empty work-groups, 5.61 TB/s with only the existing pieces in the same
// order, and 5.88 TB/s with the full pieces first.
//
// With C = xcd_classes > 1 the batch is cut into C contiguous request ranges
// and their full pieces are interleaved (entry k C + c is the k-th full piece
// of range c while every range has one; a range that runs out drops out of
// the rotation).  Entry i of head block gb runs on XCD (i NB + gb) mod 8, so
// with C = 8 / gcd(NB, 8) every full piece of range c for head block gb runs
// on one XCD, and neighbouring requests -- those a radix cache hands out
// together, which share their prefix pages -- read those pages through one
// L2 instead of several.
#pragma once

#include "internal.h"

namespace pa {

constexpr int kPlanSingle = 1 << 30;
constexpr int kPlanClassKeys = 128;
constexpr int kPlanClasses = kMaxSplitTokens / kPlanClassKeys + 2;  // none, key-count classes, zero row
constexpr int kPlanZero = kPlanClasses - 1;

// Every thread of the work-group (kThreads of them) calls this once.
template <int kThreads>
__device__ __forceinline__ void build_decode_plan(const PlanArgs& p) {
  constexpr int kWaves = kThreads / 64;
  __shared__ int s_wfull[kWaves];
  __shared__ int s_wcnt[kWaves][kPlanClasses];
  __shared__ int s_base[kPlanClasses];  // next free entry of each class
  __shared__ int s_full;                // next free entry of the full pieces
  __shared__ int s_ct[8];               // full pieces of each request range
  __shared__ int s_cb[8];               // full pieces of the ranges before it
  __shared__ int s_total;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = p.split_tokens, S = p.max_splits, B = p.num_seqs;
  const int C = p.xcd_classes;
  auto range_of = [&](int b) { return (int)((int64_t)b * C / B); };
  const uint64_t below = (1ull << lane) - 1;

  auto incl_scan = [&](int x) {  // inclusive prefix sum over the wave
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int y = __shfl_up(x, m, 64);
      if (lane >= m) x += y;
    }
    return x;
  };

  // request b: full pieces, class of its last piece (0: none), first key
  struct Req {
    int nfull, cls, k0, nlast;
    bool single;
  };
  auto info = [&](int b) {
    Req r = {0, 0, 0, 0, false};
    if (b >= B) return r;
    if (p.q_indptr && p.q_indptr[b + 1] - p.q_indptr[b] != 1) return r;  // not a decode request
    const int L = p.seq_lens[b];
    r.k0 = p.key_begin ? max(p.key_begin[b], 0) : 0;
    const int own = max(L - r.k0, 0);
    const int ns = min(own / split + (own % split != 0 ? 1 : 0), S);
    r.nfull = min(own / split, ns);
    r.single = ns == 1 && !p.always_partial;
    if (ns > r.nfull) {
      r.nlast = own - r.nfull * split;
      r.cls = (r.nlast + kPlanClassKeys - 1) / kPlanClassKeys;
    } else if (L <= 0 && !p.key_begin && !p.always_partial) {
      r.cls = kPlanZero;
    }
    return r;
  };

  // pass 1: how many entries of each kind.  The first chunk of requests is
  // kept in registers for pass 2 (a batch of at most kThreads requests is
  // read once).
  if (tid < kPlanClasses) s_base[tid] = 0;
  if (tid < 8) s_ct[tid] = 0;
  if (tid == 0) s_full = 0;
  const Req first = info(tid);
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += kThreads) {
    const Req r = b0 == 0 ? first : info(b0 + tid);
    const int nf = incl_scan(r.nfull);
    if (lane == 63 && nf) atomicAdd(&s_full, nf);
    if (C > 1 && r.nfull > 0) atomicAdd(&s_ct[range_of(b0 + tid)], r.nfull);
    for (int c = 1; c < kPlanClasses; ++c) {
      const int n = __popcll(__ballot(r.cls == c));
      if (lane == 0 && n) atomicAdd(&s_base[c], n);
    }
  }
  __syncthreads();
  if (tid == 0) {  // classes in decreasing key count after the full pieces; zero rows last
    int next = s_full;
    for (int c = kPlanClasses - 2; c >= 1; --c) {
      const int n = s_base[c];
      s_base[c] = next;
      next += n;
    }
    const int nz = s_base[kPlanZero];
    s_base[kPlanZero] = next;
    s_total = next + nz;
    s_full = 0;
    int e = 0;
    for (int c = 0; c < C; ++c) {
      s_cb[c] = e;
      e += s_ct[c];
    }
  }
  __syncthreads();

  // pass 2: write the entries
  int4* plan = p.plan;
  for (int b0 = 0; b0 < B; b0 += kThreads) {
    const int b = b0 + tid;
    const Req r = b0 == 0 ? first : info(b);
    // full pieces: exclusive prefix over the work-group
    const int incl = incl_scan(r.nfull);
    if (lane == 63) s_wfull[wave] = incl;
    int rank = 0;
    for (int c = 1; c < kPlanClasses; ++c) {
      const uint64_t bal = __ballot(r.cls == c);
      if (r.cls == c) rank = __popcll(bal & below);
      if (lane == 0) s_wcnt[wave][c] = __popcll(bal);
    }
    __syncthreads();
    int fpos = s_full + incl - r.nfull;
    int cpos = r.cls ? s_base[r.cls] + rank : 0;
    for (int w = 0; w < wave; ++w) {
      fpos += s_wfull[w];
      if (r.cls) cpos += s_wcnt[w][r.cls];
    }
    const int flag = r.single ? kPlanSingle : 0;
    if (C > 1) {
      // fpos - s_cb[c]: the request's first full piece within its range
      const int c = r.nfull > 0 ? range_of(b) : 0;
      for (int s = 0; s < r.nfull; ++s) {
        const int k = fpos + s - s_cb[c];
        int pos = 0;
        for (int c2 = 0; c2 < C; ++c2) pos += min(s_ct[c2], k) + (c2 < c && s_ct[c2] > k ? 1 : 0);
        plan[pos] = make_int4(b, s | flag, r.k0 + s * split, split);
      }
    } else {
      for (int s = 0; s < r.nfull; ++s) plan[fpos + s] = make_int4(b, s | flag, r.k0 + s * split, split);
    }
    if (r.cls == kPlanZero) {
      plan[cpos] = make_int4(b, 0, 0, 0);
    } else if (r.cls) {
      plan[cpos] = make_int4(b, r.nfull | flag, r.k0 + r.nfull * split, r.nlast);
    }
    __syncthreads();
    if (tid == 0) {
      int n = 0;
      for (int w = 0; w < kWaves; ++w) n += s_wfull[w];
      s_full += n;
    }
    if (tid > 0 && tid < kPlanClasses) {
      int n = 0;
      for (int w = 0; w < kWaves; ++w) n += s_wcnt[w][tid];
      s_base[tid] += n;
    }
    __syncthreads();
  }
  // the rest: no work
  const int n = S * B;
  for (int i = s_total + tid; i < n; i += kThreads) plan[i] = make_int4(-1, 0, 0, 0);
}

}  // namespace pa

#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

One step = one decode layer-step of the Qwen3-8B-shaped batch with radix
prefix sharing (256 requests, log-uniform lengths 512..8192, 32 query / 8 KV
heads, head_dim 128, page 16, bf16; groups of 16 requests share a 1024-token
prefix): the store of the 256 new K/V rows, then the cascade decode (shared
prefix pass on the matrix cores, each request's own keys through the split-K
decode kernel, combine).  The work order and the own-keys pass follow the
store on the caller's stream; the shared-prefix pass runs on a second stream
beside them from the start of the step (it reads only shared pages, which the
store does not write).  The same calls one after the other on one stream give the
per-kernel times.  Inputs are resident in HBM before timing starts.
The plain decode (partial + combine over every request's whole page list) and
the chunked-prefill extend call (8 requests, prefix 0..4096 + 512-token
chunk, same head shape) are timed in the same run and reported in their own
objects.

Prints one JSON line.  `value` is decode KV throughput in GB/s counted on the
distinct KV bytes the step must read (each physical slot once); `roofline`
describes the dominant kernel (the split-K decode kernel over the requests'
own keys) with its average duration taken from HIP events on the launch
stream; `cpu_baseline` is the CPU oracle timed on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
PROFILE_COUNTERS = {
    "cascade": os.path.join(ROOT, "profiles", "decode_partial_own_keys_qwen3_8b_radix_counters.txt"),
    "plain": os.path.join(ROOT, "profiles", "decode_partial_qwen3_8b_radix_counters.txt"),
    "extend": os.path.join(ROOT, "profiles", "extend_qwen3_8b_extend_counters.txt"),
    "rope": os.path.join(ROOT, "profiles", "rope_store_qwen3_8b_extend_rows_counters.txt"),
    "verify": os.path.join(ROOT, "profiles", "verify_qwen3_8b_verify_counters.txt"),
}
_CSRC = os.path.join(ROOT, "paged_kv_attention_11_amd", "csrc")
DECODE_SOURCES = [os.path.join(_CSRC, f) for f in ("decode.hip", "plan.h", "device.h", "internal.h")]
EXTEND_SOURCES = [os.path.join(_CSRC, f) for f in ("extend.hip", "mfma_tile.h", "device.h", "internal.h")]
ROPE_SOURCES = [os.path.join(_CSRC, f) for f in ("rope.hip", "device.h", "internal.h")]
VERIFY_SOURCES = [os.path.join(_CSRC, f) for f in ("verify.hip", "mfma_tile.h", "device.h", "internal.h")]
KERNEL_SOURCES = {"cascade": DECODE_SOURCES, "plain": DECODE_SOURCES, "extend": EXTEND_SOURCES,
                  "rope": ROPE_SOURCES, "verify": VERIFY_SOURCES}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="qwen3_8b_radix")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extend", action="store_true")
    ap.add_argument("--no-plain", action="store_true", help="skip the plain-decode comparison")
    ap.add_argument("--path", choices=["cascade", "plain"], default="cascade",
                    help="decode path of the timed step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU leg")
    ap.add_argument("--only", choices=["extend", "verify", "rope"],
                    help="time only this call (for profiler runs) and print its object")
    ap.add_argument("--copy-only", action="store_true",
                    help="only the plain-copy calibration (for hardware-counter scaling runs)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sources_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_profile(kind):
    """The fields of a committed counter summary, if it was taken on the
    current kernel source (its source_digest matches), else None."""
    fname = PROFILE_COUNTERS[kind]
    if not os.path.exists(fname):
        return None
    kv = {}
    for line in open(fname):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != sources_digest(KERNEL_SOURCES[kind]):
        return None
    return kv


def read_traffic(kind):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source."""
    kv = read_profile(kind)
    try:
        return float(kv["hbm_bytes_per_dispatch"]) if kv else None
    except (KeyError, ValueError):
        return None


def read_mfma_counters():
    """Matrix-core use of the extend kernel from its committed counter
    summary (SQ_VALU_MFMA_BUSY_CYCLES over the SIMD-cycles of the launch,
    the clock under load from GRBM_GUI_ACTIVE), if taken on the current
    source."""
    kv = read_profile("extend")
    keys = ("mfma_busy_frac", "clock_ghz_under_load", "peak_tflops_at_that_clock", "mfma_flops_executed",
            "valu_coexec_frac_of_mfma_busy", "lds_bank_conflict_cycles", "valu_insts_per_mfma")
    if not kv or any(k not in kv for k in keys):
        return None
    return {k: float(kv[k]) for k in keys}


COPY_PAGES = 16384  # per pool: 16384 pages x 16 tokens x 8 heads x 128 x bf16 = 512 MiB


def read_ceiling(iters=10, nbytes=2 << 30):
    """Read-only HBM rate through the library's calibration call
    (pa_stream_read over a 2 GiB buffer, far larger than the last-level
    cache): the ceiling the streaming kernels are compared with."""
    import torch

    import paged_kv_attention_11_amd as pa

    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ms = _time(torch, stream, lambda: pa.stream_read(buf, sink), iters)
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def copy_calibration(iters=10):
    """A plain copy of known size with the library's gather kernel: K and V
    pools of 512 MiB each, laid out as one request with an identity page
    table, so a launch reads 1 GiB and writes 1 GiB in long sequential runs.
    Returns (read+write GB/s, bytes read per launch, average launch ms)."""
    import torch

    import paged_kv_attention_11_amd as pa

    P, H, D = 16, 8, 128
    k = torch.randn(COPY_PAGES, P, H, D, device="cuda").to(torch.bfloat16)
    v = torch.randn(COPY_PAGES, P, H, D, device="cuda").to(torch.bfloat16)
    n = COPY_PAGES * P
    pt = torch.arange(COPY_PAGES, dtype=torch.int32, device="cuda")[None, :].contiguous()
    sl = torch.tensor([n], dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, n], dtype=torch.int64, device="cuda")
    ko = torch.empty(n, H, D, dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    f = lambda: pa.gather(k, v, pt, sl, offs, n, ko, vo)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        f()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / iters
    nread = 2 * k.numel() * k.element_size()
    del k, v, ko, vo
    torch.cuda.empty_cache()
    return 2 * nread / (ms * 1e-3) / 1e9, nread, ms


def bench_decode_configs(pa, W, torch, np, stream, iters):
    """pa_decode (partial + combine) on the smaller decode configurations:
    at these sizes a call is bound by launch and memory latency, not by HBM
    bandwidth, so the time is the figure of interest."""
    out = {}
    for name in ("tiny", "qwen25_05b", "qwen3_06b_p1"):
        wl = W.make(name)
        d = W.to_device(wl)
        pa.kv_store(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slot_mapping)
        o = torch.empty_like(d.q)
        ws = pa.decode_workspace(d.q, d.k_pool, wl.max_seq_len)
        def f():
            pa.decode(d.q, d.k_pool, d.v_pool, d.page_table, d.seq_lens, wl.max_seq_len, wl.scale, o, ws)

        ms = _time(torch, stream, f, iters)
        # The same calls captured back to back into one HIP graph: at these
        # sizes a call from Python costs more host time than the GPU spends,
        # so the replay shows the GPU-side time per call.
        per_graph = 20
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                f()
        torch.cuda.synchronize()
        gms = _time(torch, stream, graph.replay, max(3, iters // per_graph)) / per_graph
        del graph
        out[name] = {"us": round(ms * 1e3, 2), "graph_us": round(gms * 1e3, 2),
                     "GBps_unique": round(wl.kv_bytes_unique() / (ms * 1e-3) / 1e9, 1),
                     "GBps_unique_graph": round(wl.kv_bytes_unique() / (gms * 1e-3) / 1e9, 1),
                     "tokens_per_s": round(wl.num_seqs / (ms * 1e-3), 1), "dtype": wl.dtype,
                     "description": W.DESCRIPTIONS[name]}
        if name == "qwen3_06b_p1":
            # Cold: the calls rotate over three copies of the pools (3 x 302 MB
            # of keys and values touched, more than twice the 256 MB last-level
            # cache), so a call finds none of its bytes left there by the
            # previous one.
            reps = [d] + [W.to_device(wl) for _ in range(2)]
            for r in reps[1:]:
                pa.kv_store(r.k_pool, r.v_pool, r.k_new, r.v_new, r.slot_mapping)
            turn = [0]

            def g():
                r = reps[turn[0] % len(reps)]
                turn[0] += 1
                pa.decode(r.q, r.k_pool, r.v_pool, r.page_table, r.seq_lens, wl.max_seq_len, wl.scale, o, ws)

            cms = _time(torch, stream, g, 3 * max(1, iters // 3))
            out[name]["cold_us"] = round(cms * 1e3, 2)
            out[name]["GBps_unique_cold"] = round(wl.kv_bytes_unique() / (cms * 1e-3) / 1e9, 1)
            del reps
        elif name == "qwen25_05b":
            # Cold: about 6 MB, too small to rotate out of the last-level
            # cache; a 1 GiB scratch write between calls, outside the timed
            # events, evicts it instead.
            scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(iters)]
            f()
            for s_ev, e_ev in evs:
                scratch.fill_(1)
                s_ev.record(stream)
                f()
                e_ev.record(stream)
            torch.cuda.synchronize()
            cms = float(np.mean([s_ev.elapsed_time(e_ev) for s_ev, e_ev in evs]))
            out[name]["cold_us"] = round(cms * 1e3, 2)
            out[name]["GBps_unique_cold"] = round(wl.kv_bytes_unique() / (cms * 1e-3) / 1e9, 1)
            del scratch
        del d, ws
    return out


def bench_rope(pa, W, torch, np, stream, iters):
    """pa_rope_kv_store on the chunked-prefill workload's 4096 new rows:
    rotate q (32 heads) and k (8 heads), store k and v.  HBM-bound."""
    ew = W.make("qwen3_8b_extend")
    edw = W.to_device(ew)
    pos = ew.positions()
    cos_t, sin_t = W.rope_tables(int(ew.max_seq_len), ew.head_dim)
    pos_d = torch.from_numpy(pos).cuda()
    cos_d, sin_d = torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda()
    q_out = torch.empty_like(edw.q)

    def f():
        pa.rope_kv_store(edw.k_pool, edw.v_pool, edw.q, edw.k_new, edw.v_new, pos_d, edw.slot_mapping, cos_d, sin_d,
                         q_out=q_out)

    for _ in range(3):
        f()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(iters):
        f()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / iters
    N, Hq, Hkv, D, es = len(pos), ew.num_q_heads, ew.num_kv_heads, ew.head_dim, ew.elem_bytes
    # q read + written, k and v read + written, distinct table rows, positions and slots
    alg = 2 * N * Hq * D * es + 4 * N * Hkv * D * es + len(np.unique(pos)) * D * 4 + N * (4 + 8)
    gbps = alg / (ms * 1e-3) / 1e9
    return {"workload": "qwen3_8b_extend (4096 new rows)", "kernel_us": round(ms * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": read_traffic("rope"),
                         "algorithmic_bytes_per_launch": int(alg)}}


def _time(torch, stream, f, iters):
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(iters):
        f()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def bench_verify(pa, W, torch, np, stream, iters):
    """pa_verify on the Qwen3-8B-shaped verify workload (64 requests, 6 new
    rows each after contexts of 512..8192 keys), against pa_extend on the same
    batch.  HBM-bound: each request's K/V is read once for its 6 x 4 query
    rows per KV head."""
    vw = W.make("qwen3_8b_verify")
    d = W.to_device(vw)
    pa.kv_store(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slot_mapping)
    out = torch.empty_like(d.q)
    nb = pa.verify_workspace_bytes(vw.num_seqs, vw.max_q_len, vw.num_q_heads, vw.num_kv_heads, vw.head_dim,
                                   vw.max_seq_len)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")

    def ver():
        pa.verify(d.q, d.q_indptr, d.k_pool, d.v_pool, d.page_table, d.seq_lens, vw.max_q_len, vw.max_seq_len,
                  vw.scale, out=out, workspace=ws)

    def ext():
        pa.extend(d.q, d.q_indptr, d.k_pool, d.v_pool, d.page_table, d.seq_lens, vw.max_q_len, vw.max_seq_len,
                  vw.scale, out=out)

    ms = _time(torch, stream, ver, iters)
    ems = _time(torch, stream, ext, iters)
    kv = vw.kv_bytes_unique()
    P = vw.page_size
    alg = kv + 2 * int(vw.q_indptr[-1]) * vw.num_q_heads * vw.head_dim * 2 + \
        4 * int(sum((int(L) + P - 1) // P for L in vw.seq_lens))
    gbps = alg / (ms * 1e-3) / 1e9
    return {"workload": "qwen3_8b_verify", "description": W.DESCRIPTIONS["qwen3_8b_verify"],
            "kernel_us": round(ms * 1e3, 2), "extend_us": round(ems * 1e3, 2),
            "rows_per_s": round(int(vw.q_indptr[-1]) / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": read_traffic("verify"),
                         "algorithmic_bytes_per_launch": int(alg),
                         "note": "verify kernel + its combine; K/V counted once per request"}}


def bench_mixed(pa, W, torch, np, stream, iters):
    """One continuous-batching step of the Qwen3-8B-shaped mixed workload
    (8 prefill chunks of 512 rows + 248 decode requests): rope + store, then
    the mixed attention call; launched eagerly and as one replayed HIP graph.
    Also the attention alone routed (decode kernels for one-row requests)
    against every request through the extend kernel."""
    mw = W.make("qwen3_8b_mixed")
    d = W.to_device(mw)
    pos = torch.from_numpy(mw.positions()).cuda()
    cos_t, sin_t = W.rope_tables(int(mw.max_seq_len), mw.head_dim)
    cos_d, sin_d = torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda()
    q_rot, out = torch.empty_like(d.q), torch.empty_like(d.q)
    nb = pa.decode_workspace_bytes(mw.num_seqs, mw.num_q_heads, mw.num_kv_heads, mw.head_dim, mw.max_seq_len)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def attend():
        pa.attend_mixed(q_rot, d.q_indptr, d.k_pool, d.v_pool, d.page_table, d.seq_lens, mw.max_q_len, mw.max_seq_len,
                        mw.scale, out=out, workspace=ws)

    def step():
        pa.rope_kv_store(d.k_pool, d.v_pool, d.q, d.k_new, d.v_new, pos, d.slot_mapping, cos_d, sin_d, q_out=q_rot)
        attend()

    def all_extend():
        pa.extend(q_rot, d.q_indptr, d.k_pool, d.v_pool, d.page_table, d.seq_lens, mw.max_q_len, mw.max_seq_len,
                  mw.scale, out=out)

    eager = _time(torch, stream, step, iters)
    routed = _time(torch, stream, attend, iters)
    ext = _time(torch, stream, all_extend, iters)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    replay = _time(torch, stream, graph.replay, iters)
    del graph
    return {"workload": "qwen3_8b_mixed", "description": W.DESCRIPTIONS["qwen3_8b_mixed"],
            "step": "rope_kv_store + attend_mixed", "eager_us": round(eager * 1e3, 1),
            "graph_replay_us": round(replay * 1e3, 1), "attention_routed_us": round(routed * 1e3, 1),
            "attention_all_extend_us": round(ext * 1e3, 1),
            "tokens_per_s": round(int(mw.q_indptr[-1]) / (replay * 1e-3), 1)}


def bench_extend(pa, W, torch, np, stream, iters, warmup=3):
    """The extend call on the Qwen3-8B-shaped chunked-prefill workload, with
    its matrix-core roofline (algorithmic FLOPs: causal-visible pairs only)."""
    ew = W.make("qwen3_8b_extend")
    edw = W.to_device(ew)
    eout = torch.empty_like(edw.q)
    pa.kv_store(edw.k_pool, edw.v_pool, edw.k_new, edw.v_new, edw.slot_mapping)

    def ext():
        pa.extend(edw.q, edw.q_indptr, edw.k_pool, edw.v_pool, edw.page_table, edw.seq_lens, ew.max_q_len,
                  ew.max_seq_len, ew.scale, out=eout)

    for _ in range(warmup):
        ext()
    ems = _time(torch, stream, ext, iters)
    n = ew.n_new.astype(np.int64)
    p = (ew.seq_lens - ew.n_new).astype(np.int64)
    flops = 4 * ew.head_dim * ew.num_q_heads * int(np.sum(n * p + n * (n + 1) // 2))
    tf = flops / (ems * 1e-3) / 1e12
    return {
        "workload": "qwen3_8b_extend",
        "description": W.DESCRIPTIONS["qwen3_8b_extend"],
        "kernel_us": round(ems * 1e3, 2),
        "tokens_per_s": round(int(n.sum()) / (ems * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": read_traffic("extend"), "algorithmic_flops_per_launch": flops},
        # rocprofv3 counters of the same kernel on the same workload (committed summary)
        "mfma_counters": read_mfma_counters(),
    }


def cpu_baseline(wl, target_s):
    """The oracle, as it stands, in its float32 arithmetic mode (a plain CPU
    fp32 implementation: gather the pages, then naive softmax attention per
    request and head), on a bounded sample of the workload.  `cores` is the
    number of cores it kept busy on average (process CPU time / wall time);
    the BLAS pool size and the affinity set are reported beside it."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    order = np.random.default_rng(0).permutation(wl.num_seqs)
    done, t_used, cpu_used, nbytes = 0, 0.0, 0.0, 0
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    while done < wl.num_seqs and t_used < target_s:
        k = 4 if done == 0 else max(1, min(wl.num_seqs - done, int(done * (target_s - t_used) / max(t_used, 1e-3))))
        seqs = order[done:done + k]
        sub = wl.subset(seqs)
        t0, c0 = time.perf_counter(), time.process_time()
        oracle.decode(sub.q, kp, vp, sub.page_table, sub.seq_lens, wl.scale, wl.dtype, acc="f32")
        t_used += time.perf_counter() - t0
        cpu_used += time.process_time() - c0
        nbytes += int(sub.seq_lens.sum()) * per_tok
        done += k
    return {
        "value": round(nbytes / t_used / 1e9, 4),
        "unit": "GB/s",
        "cores": max(1, int(round(cpu_used / t_used))),
        "kind": "oracle",
        "sample": f"oracle.decode (numpy, float32 arithmetic) over {done} of {wl.num_seqs} requests of the same "
                  f"workload ({nbytes / 1e9:.3f} GB of K/V read, logical bytes), {t_used:.1f} s; store excluded",
        "cores_busy_avg": round(cpu_used / t_used, 2),
        "blas_threads": int(blas_threads),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "host_cpus": os.cpu_count(),
        "requests_per_s": round(done / t_used, 2),
    }


class StreamSync:
    """Orders one stream after another's enqueued work with HIP events that
    carry no system-scope fence (hipEventDisableSystemFence): both streams
    are on this device, so the device-scope ordering of the event suffices,
    and each cross-stream hop costs less.  Plumbing around torch's streams,
    through the HIP runtime (the library itself does not touch events)."""

    def __init__(self, slots=2):
        import ctypes

        self._c = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        flags = 0x2 | 0x20000000  # hipEventDisableTiming | hipEventDisableSystemFence
        self._ev = []
        for _ in range(slots):
            e = ctypes.c_void_p()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(e), flags) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self._ev.append(e)

    def order(self, stream, after, slot):
        """Work enqueued on `stream` from now on starts after the work already
        enqueued on `after`."""
        e = self._ev[slot]
        if self._hip.hipEventRecord(e, self._c.c_void_p(after.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
        if self._hip.hipStreamWaitEvent(self._c.c_void_p(stream.cuda_stream), e, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(attention shards over KV heads with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_attention_11_amd as pa
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    pa.load()
    dev_name = torch.cuda.get_device_name(0)

    if args.copy_only:
        gbps, nread, ms = copy_calibration()
        print(json.dumps({"copy_calibration": {"GBps_read_plus_write": round(gbps, 1),
                                               "bytes_read_per_launch": nread,
                                               "bytes_written_per_launch": nread,
                                               "launch_ms": round(ms, 4)}}), flush=True)
        return

    if args.only:
        stream = torch.cuda.current_stream()
        fn = {"extend": bench_extend, "verify": bench_verify, "rope": bench_rope}[args.only]
        print(json.dumps({args.only: fn(pa, W, torch, np, stream, args.steps)}), flush=True)
        return

    # ---------------- decode step
    t0 = time.perf_counter()
    wl = W.make(args.config)
    log(f"generated {args.config} in {time.perf_counter() - t0:.1f}s")
    dw = W.to_device(wl)
    B, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    P = wl.page_size
    split = args.split_tokens or pa.decode_split_tokens(B, Hkv, wl.max_seq_len)
    out = torch.empty_like(dw.q)
    stream = torch.cuda.current_stream()
    starts, ppt, shl = wl.cascade_inputs()
    gmax = int((starts[1:] - starts[:-1]).max()) if B else 0
    msh = int(shl.max()) if B else 0
    cascade = args.path == "cascade"
    if cascade:
        gs_d = torch.from_numpy(starts).cuda()
        ppt_d = torch.from_numpy(ppt).cuda()
        shl_d = torch.from_numpy(shl).cuda()
        piece_keys = pa.cascade_piece_keys(len(starts) - 1, gmax, Hq, Hkv, msh)
        nb = pa.decode_cascade_workspace_bytes(B, Hq, Hkv, D, wl.max_seq_len, len(starts) - 1, gmax, msh, split)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
        stages = ["order", "prefix", "suffix", "combine"]

        def call(stage):
            pa.decode_cascade(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, gs_d, gmax,
                              ppt_d, shl_d, msh, wl.scale, out=out, workspace=ws, split_tokens=split, stage=stage)
    else:
        ws = pa.decode_workspace(dw.q, dw.k_pool, wl.max_seq_len, split)
        stages = ["partial", "combine"]

        def call(stage):
            fn = pa.decode_partial if stage == "partial" else pa.decode_combine
            fn(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, wl.scale, out, ws, split)

    def step(ev=None):
        """The step's calls one after the other on one stream, with events
        between them (per-kernel times)."""
        pa.kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, dw.slot_mapping)
        for i, stage in enumerate(stages):
            if ev is not None:
                ev[i].record(stream)
            call(stage)
        if ev is not None:
            ev[len(stages)].record(stream)

    side = torch.cuda.Stream()  # default priority, like every stream here
    if cascade:
        # the new rows must not land on a page the prefix pass reads
        shared_pages = set()
        for j in range(len(starts) - 1):
            need = int(shl[starts[j]:starts[j + 1]].max(initial=0))
            shared_pages.update(ppt[j, :(need + P - 1) // P].tolist())
        new_pages = set((wl.slot_mapping[wl.slot_mapping >= 0] // P).tolist())
        assert not (shared_pages & new_pages), "a new row lands on a shared prefix page"

    sync = StreamSync()

    def step_overlapped():
        """The timed step.  Cascade: the shared-prefix pass (one latency-bound
        work-group per compute unit) on a second stream from the start of the
        step, beside the store, the work order and the HBM-bound own-keys
        pass; the merge after both.  The prefix pass reads only keys below
        each request's shared length, on the groups' prefix pages, which this
        step's store does not write (checked above), so it does not wait for
        the store, and its work-groups take their compute units before the
        own-keys pass fills the rest.  The two streams are ordered by events
        without a system-scope fence (both sides are on this device)."""
        if not cascade:
            return step()
        cur = torch.cuda.current_stream()
        sync.order(side, after=cur, slot=0)
        with torch.cuda.stream(side):
            call("prefix")
        pa.kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, dw.slot_mapping)
        call("order")
        call("suffix")
        sync.order(cur, after=side, slot=1)
        call("combine")

    for _ in range(args.warmup):
        step()
        step_overlapped()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    end.record(stream)
    torch.cuda.synchronize()
    ms_sequential = start.elapsed_time(end) / args.steps
    stage_ms = {st: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, st in enumerate(stages)}
    stage_stats = {}
    for i, st in enumerate(stages):
        v = np.array([e[i].elapsed_time(e[i + 1]) for e in evs]) * 1e3
        stage_stats[st] = {"median": round(float(np.median(v)), 2), "min": round(float(v.min()), 2),
                           "p90": round(float(np.percentile(v, 90)), 2)}
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step_overlapped()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    log(f"decode ({args.path}): {ms_step * 1e3:.1f} us/step ({ms_sequential * 1e3:.1f} us one call after the "
        f"other: " + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in stage_ms.items()) + f") (wall {wall:.3f}s)")

    # The timed (two-stream) step must give the same bits as the calls one
    # after the other on one stream.
    overlapped_out = out.clone()
    out.zero_()
    step()
    torch.cuda.synchronize()
    overlapped_same = bool(torch.equal(out.view(torch.int16), overlapped_out.view(torch.int16)))
    if not overlapped_same:
        log("WARNING: the timed two-stream step differs from the sequential step")

    # The same step captured once into a HIP graph and replayed (how a serving
    # loop would launch it): the launch gaps between its kernels shrink.  The
    # replayed output must equal the eager one bit for bit.
    eager_out = out.clone()
    warm = torch.cuda.Stream()
    warm.wait_stream(stream)
    with torch.cuda.stream(warm):
        step_overlapped()
    stream.wait_stream(warm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_overlapped()
    torch.cuda.synchronize()
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    graph_same = bool(torch.equal(out.view(torch.int16), eager_out.view(torch.int16)))
    ms_graph = _time(torch, stream, graph.replay, args.steps)
    del graph

    kv_unique = wl.kv_bytes_unique()
    kv_logical = wl.kv_bytes_logical()
    slot_bytes = 2 * Hkv * D * wl.elem_bytes
    q_bytes = B * Hq * D * wl.elem_bytes
    if cascade:
        # the split-K kernel reads each request's own keys [shared_len, seq_len): distinct slots
        own = set()
        pages_read = 0
        for b in range(B):
            L, s0 = int(wl.seq_lens[b]), int(shl[b])
            if L > s0:
                pl = wl.page_table[b]
                t = np.arange(s0, L)
                own.update((pl[t // P].astype(np.int64) * P + t % P).tolist())
                pages_read += (L - 1) // P - s0 // P + 1
        dom_kernel, dom_ms = "decode_partial_kernel<bf16, D=128, G=4> (own keys)", stage_ms["suffix"]
        dom_bytes = len(own) * slot_bytes + q_bytes + 4 * pages_read + 8 * B
    else:
        pages_read = int(sum((int(L) + P - 1) // P for L in wl.seq_lens))
        # the partial stage is the work-order kernel (one work-group) and the partial kernel
        dom_kernel, dom_ms = "decode_plan_kernel + decode_partial_kernel<bf16, D=128, G=4>", stage_ms["partial"]
        dom_bytes = kv_unique + q_bytes + 4 * pages_read + 4 * B
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = read_traffic(args.path)
    value = kv_unique / (ms_step * 1e-3) / 1e9

    result = {
        "metric": "paged-attn decode KV HBM GB/s (% of peak) + decode tokens/s, Qwen3-8B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.config,
            "description": W.DESCRIPTIONS.get(args.config, args.config),
            "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "page_size": P,
            "sum_seq_len": int(wl.seq_lens.sum()), "max_seq_len": wl.max_seq_len, "split_tokens": split,
            "step": ("kv_store of the 256 new rows, then the decode_cascade stages: the work order and the own-keys "
                     "pass after the store, the prefix pass on a second stream beside them, then combine" if cascade
                     else "kv_store + decode_partial + decode_combine"),
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "kv_bytes_unique": kv_unique,
        "kv_bytes_logical": kv_logical,
        "kernel_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "kernel_us_stats": stage_stats,
        "sequential_ms_per_step": round(ms_sequential, 5),
        "graph_replay": {"ms_per_step": round(ms_graph, 5),
                         "GBps_unique": round(kv_unique / (ms_graph * 1e-3) / 1e9, 2),
                         "pct_of_hbm_peak": round(100 * kv_unique / (ms_graph * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                         "same_bits_as_eager": graph_same},
        "timed_step_same_bits_as_sequential": overlapped_same,
        "roofline": {
            "kernel": dom_kernel,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
        },
        "device": dev_name,
    }
    if cascade:
        result["config"]["prefix_piece_keys"] = piece_keys
        result["config"]["groups"] = len(starts) - 1

    # ---------------- plain decode of the same step, for comparison
    if cascade and not args.no_plain:
        del ws
        pws = pa.decode_workspace(dw.q, dw.k_pool, wl.max_seq_len, split)
        pout = torch.empty_like(dw.q)

        def plain():
            pa.kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, dw.slot_mapping)
            pa.decode(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, wl.scale, pout, pws,
                      split)

        for _ in range(max(3, args.warmup // 2)):
            plain()
        torch.cuda.synchronize()
        ps, pe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ksteps = max(5, args.steps // 2)
        ps.record(stream)
        for _ in range(ksteps):
            plain()
        pe.record(stream)
        torch.cuda.synchronize()
        pms = ps.elapsed_time(pe) / ksteps
        result["plain_decode"] = {
            "step": "kv_store + decode (partial + combine over whole page lists)",
            "ms_per_step": round(pms, 5),
            "GBps_unique": round(kv_unique / (pms * 1e-3) / 1e9, 2),
            "decode_tokens_per_s": round(B / (pms * 1e-3), 1),
        }
        log(f"plain decode: {pms * 1e3:.1f} us/step")
        del pws

    # ---------------- extend (chunked prefill on the same head shape)
    if not args.no_extend:
        result["extend"] = bench_extend(pa, W, torch, np, stream, max(5, args.steps // 2), max(3, args.warmup // 2))
        log(f"extend: {result['extend']['kernel_us']} us, {result['extend']['roofline']['achieved']} TFLOP/s")

    # ---------------- the other decode configurations (plain decode, one call)
    if not args.no_extend:
        result["decode_configs"] = bench_decode_configs(pa, W, torch, np, stream, max(10, args.steps))
        log("decode configs: " + ", ".join(
            f"{k} {v['us']} us, {v['graph_us']} us in a graph ({v['GBps_unique']} GB/s)"
            + (f", {v['cold_us']} us cold ({v['GBps_unique_cold']} GB/s)" if "cold_us" in v else "")
            for k, v in result["decode_configs"].items()))

    # ---------------- fused rotary embedding + store (the step before attention)
    if not args.no_extend:
        result["rope_kv_store"] = bench_rope(pa, W, torch, np, stream, max(5, args.steps // 2))
        log(f"rope+store: {result['rope_kv_store']['kernel_us']} us, "
            f"{result['rope_kv_store']['roofline']['achieved']} GB/s")

    # ---------------- short-chunk verify (speculative decoding)
    if not args.no_extend:
        result["verify"] = bench_verify(pa, W, torch, np, stream, max(5, args.steps // 2))
        v = result["verify"]
        log(f"verify: {v['kernel_us']} us ({v['roofline']['achieved']} GB/s) vs extend {v['extend_us']} us")

    # ---------------- a mixed continuous-batching step, eager and as a replayed graph
    if not args.no_extend:
        result["mixed_step"] = bench_mixed(pa, W, torch, np, stream, max(5, args.steps // 2))
        m = result["mixed_step"]
        log(f"mixed step: eager {m['eager_us']} us, graph {m['graph_replay_us']} us, "
            f"all-extend attention {m['attention_all_extend_us']} us vs routed {m['attention_routed_us']} us")

    # ---------------- plain-copy reference and read-only ceiling on the same device
    cgb, _, _ = copy_calibration()
    result["copy_reference_GBps"] = round(cgb, 1)
    rgb = read_ceiling()
    result["hbm_read_ceiling_GBps"] = round(rgb, 1)
    result["roofline"]["frac_of_read_ceiling"] = round(result["roofline"]["achieved"] / rgb, 4)
    result["value_frac_of_read_ceiling"] = round(result["value"] / rgb, 4)
    log(f"plain copy: {cgb:.0f} GB/s read+write; read-only ceiling {rgb:.0f} GB/s "
        f"(dominant kernel at {100 * result['roofline']['achieved'] / rgb:.1f}% of it)")

    # ---------------- CPU oracle on a bounded sample (rank 0, N=1 only)
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        cb = cpu_baseline(wl, args.cpu_seconds)
        # the same basis on both sides: logical K/V bytes read per second
        gpu_logical = wl.kv_bytes_logical() / (result["ms_per_step"] * 1e-3) / 1e9
        cb["gpu_over_oracle"] = round(gpu_logical / cb["value"], 1)
        result["cpu_baseline"] = cb
        log(f"cpu baseline: {cb['value']} GB/s in {time.perf_counter() - t0:.1f}s "
            f"(GPU / oracle {cb['gpu_over_oracle']}x)")
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Shared helpers of the GPU tests: device copies of workloads, the library
calls in the order a serving step makes them, and the tolerance check."""
import functools

import numpy as np

import oracle
import workloads as W

ATOL, RTOL = 1e-2, 2e-2  # |gpu - ref| <= ATOL + RTOL * |ref|, element-wise


def pa():
    import paged_kv_attention_11_amd as lib

    return lib


def torch():
    import torch as t

    return t


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside |d| <= {atol} + {rtol}|ref|; "
            f"max abs {err.max():.3g}; worst at {i}: got {got[i]!r} ref {ref[i]!r}")
    return float(err.max()) if err.size else 0.0


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def stored_oracle_pools(wl):
    return oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)


@functools.lru_cache(maxsize=5)
def named(name, poison="nan"):
    """(workload, device copy with the new rows already stored by the GPU)."""
    wl = W.make(name, poison=poison)
    dw = W.to_device(wl)
    pa().kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, dw.slot_mapping)
    torch().cuda.synchronize()
    return wl, dw


def gpu_decode(wl, dw, split=0, out=None):
    o = pa().decode(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, wl.scale,
                    out=out, split_tokens=split)
    torch().cuda.synchronize()
    return o


def gpu_extend(wl, dw):
    o = pa().extend(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                    wl.max_seq_len, wl.scale)
    torch().cuda.synchronize()
    return o


def fresh(wl):
    """Device copy of a workload with the new rows stored by the GPU."""
    dw = W.to_device(wl)
    pa().kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, dw.slot_mapping)
    torch().cuda.synchronize()
    return dw

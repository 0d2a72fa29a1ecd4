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


def bits(t):
    """Raw bytes of a device tensor, for bit-for-bit comparisons."""
    if t.dtype == torch().bfloat16:
        return t.detach().cpu().view(torch().int16).numpy().tobytes()
    return t.detach().cpu().numpy().tobytes()


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


@functools.lru_cache(maxsize=4)
def oracle_whole(name):
    """The oracle's output for every request of a named workload (decode
    workloads: oracle.decode; workloads with chunks: oracle.extend), computed
    once per test session."""
    wl = W.make(name, poison="nan")
    kp, vp = stored_oracle_pools(wl)
    if wl.kind == "decode":
        return oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    return oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)


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


def cascade_device(wl, starts=None, ppt=None, shl=None):
    """Device copies of the group structure (the workload's own unless given)
    and its host-side bounds: (group_starts, prefix_page_table, shared_lens,
    max_group_size, max_shared_len)."""
    if starts is None:
        starts, ppt, shl = wl.cascade_inputs()
    T = torch()
    gmax = int((starts[1:] - starts[:-1]).max()) if len(starts) > 1 else 0
    msh = int(shl.max()) if len(shl) else 0
    return (T.from_numpy(np.ascontiguousarray(starts, np.int32)).cuda(),
            T.from_numpy(np.ascontiguousarray(ppt, np.int32)).cuda(),
            T.from_numpy(np.ascontiguousarray(shl, np.int32)).cuda(), gmax, msh)


def gpu_cascade(wl, dw, split=0, piece_keys=0, groups=None, out=None):
    gs, ppt, shl, gmax, msh = cascade_device(wl, *(groups or ()))
    o = pa().decode_cascade(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, gs, gmax,
                            ppt, shl, msh, wl.scale, out=out, split_tokens=split, prefix_piece_keys=piece_keys)
    torch().cuda.synchronize()
    return o

"""Python binding of libpagedattn.so (gfx950 paged KV-cache attention).

Argument marshalling only: every function passes torch tensors' device
pointers and the current HIP stream to the C ABI declared in
include/pagedattn.h, and raises PagedAttnError on a non-zero status.  All
computation happens in the library's HIP kernels; there is no fallback.  If
the shared library has not been built, the first call raises.

Tensors:
  k_pool, v_pool  [num_pages, page_size, num_kv_heads, head_dim], bf16 or fp32,
                  contiguous, on the GPU
  page_table      int32 [num_seqs, stride];  seq_lens int32 [num_seqs]
  slot_mapping    int64 [num_rows];  q_indptr int32 [num_seqs + 1]
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path
from typing import Optional

__all__ = [
    "PagedAttnError", "library_path", "load", "version", "kv_store", "decode", "decode_noalloc", "decode_partial",
    "decode_combine", "decode_split_tokens", "decode_heads_per_block", "decode_workspace_bytes", "extend",
    "extend_workspace_bytes", "gather",
]

_PKG = Path(__file__).resolve().parent
_LIB_NAME = "libpagedattn.so"

PA_F32, PA_BF16 = 0, 1
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_DTYPE",
                4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_HIP", 7: "PA_ERR_SCRATCH"}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().pa_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


class KVPool(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_LIB: Optional[ctypes.CDLL] = None

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_POOLP = ctypes.POINTER(KVPool)
_DECODE_ARGS = [_POOLP, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _vp, _vp, _sz, _vp]

_CASCADE_ARGS = [_POOLP, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32,
                 _i32, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]

SIGNATURES = {
    # name: (restype, argtypes) -- mirrors include/pagedattn.h
    "pa_version": (ctypes.c_char_p, []),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_kv_store": (_i32, [_POOLP, _vp, _vp, _vp, _i64, _vp]),
    "pa_rope_kv_store": (_i32, [_POOLP, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _vp, _vp]),
    "pa_decode_split_tokens": (_i32, [_i32, _i32, _i32]),
    "pa_decode_heads_per_block": (_i32, [_i32, _i32, _i32, _i32]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (_i32, _DECODE_ARGS),
    "pa_decode_noalloc": (_i32, [_POOLP, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _vp, _vp]),
    "pa_decode_partial": (_i32, _DECODE_ARGS),
    "pa_decode_combine": (_i32, _DECODE_ARGS),
    "pa_extend_workspace_bytes": (_sz, [_i32] * 7),
    "pa_extend": (_i32, [_POOLP, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _sz, _vp]),
    "pa_cascade_piece_keys": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_cascade_workspace_bytes": (_sz, [_i32] * 10),
    "pa_decode_cascade": (_i32, _CASCADE_ARGS),
    "pa_decode_cascade_prefix": (_i32, _CASCADE_ARGS),
    "pa_decode_cascade_suffix": (_i32, _CASCADE_ARGS),
    "pa_decode_cascade_combine": (_i32, _CASCADE_ARGS),
    "pa_decode_cascade_order": (_i32, _CASCADE_ARGS),
    "pa_attend_mixed": (_i32, [_POOLP, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _sz,
                               _vp]),
    "pa_verify_workspace_bytes": (_sz, [_i32] * 7),
    "pa_verify": (_i32, [_POOLP, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _sz, _vp]),
    "pa_check_batch": (_i32, [_POOLP, _vp, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _i64, _vp, _vp]),
    "pa_check_cascade": (_i32, [_POOLP, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp]),
    "pa_gather": (_i32, [_POOLP, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp]),
    "pa_stream_read": (_i32, [_vp, _i64, _vp, _vp]),
}


def library_path() -> Path:
    return Path(os.environ.get("PAGEDATTN_LIB", _PKG / _LIB_NAME))


def load() -> ctypes.CDLL:
    """Load the shared library (once) and declare its signatures."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not path.exists():
            raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_attention_11_amd.build`")
        lib = ctypes.CDLL(str(path))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


_lib = load


def version() -> str:
    return load().pa_version().decode()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _check(status: int, where: str) -> None:
    if status != 0:
        raise PagedAttnError(status, where)


def _torch():
    import torch

    return torch


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_pool(k_pool, v_pool) -> KVPool:
    torch = _torch()
    if k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype:
        raise ValueError("k_pool and v_pool must have the same shape and dtype")
    if k_pool.dim() != 4:
        raise ValueError("pools are [num_pages, page_size, num_kv_heads, head_dim]")
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    dt = {torch.bfloat16: PA_BF16, torch.float32: PA_F32}.get(k_pool.dtype)
    if dt is None:
        raise ValueError(f"unsupported pool dtype {k_pool.dtype}")
    n, P, H, D = k_pool.shape
    return KVPool(k_pool.data_ptr(), v_pool.data_ptr(), n, P, H, D, dt)


# --------------------------------------------------------------------------
# the calls
# --------------------------------------------------------------------------
def kv_store(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None) -> None:
    """Write row i of k_new/v_new [N, H_kv, D] to flat slot slot_mapping[i]
    (int64; negative = skip) of the pools, in place."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(k_new, "k_new", k_pool.dtype)
    _dev(v_new, "v_new", k_pool.dtype)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    st = load().pa_kv_store(ctypes.byref(pool), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                            slot_mapping.numel(), _stream(stream))
    _check(st, "pa_kv_store")


def rope_kv_store(k_pool, v_pool, q, k_new, v_new, positions, slot_mapping, cos_table, sin_table, q_out=None,
                  stream=None):
    """Rotate q [N, H_q, D] and k_new [N, H_kv, D] by the rotary tables
    (fp32 [max_position, D/2]) at `positions` (int32 [N]); write the rotated
    keys and v_new to slot_mapping's slots of the pools; return q_out."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, n, k_pool.dtype)
    if q is not None:
        _dev(q, "q", k_pool.dtype)
    _dev(positions, "positions", torch.int32)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(cos_table, "cos_table", torch.float32)
    _dev(sin_table, "sin_table", torch.float32)
    N = slot_mapping.numel()
    if positions.numel() != N or k_new.shape[0] != N or v_new.shape[0] != N or (q is not None and q.shape[0] != N):
        raise ValueError("q, k_new, v_new, positions and slot_mapping must have the same number of rows")
    if cos_table.dim() != 2 or cos_table.shape[1] * 2 != k_pool.shape[3] or sin_table.shape != cos_table.shape:
        raise ValueError("cos_table and sin_table must be [max_position, head_dim / 2]")
    Hq = 0 if q is None else q.shape[1]
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if q_out is not None:
        _dev(q_out, "q_out", k_pool.dtype)
    st = load().pa_rope_kv_store(ctypes.byref(pool), _ptr(q), Hq, _ptr(k_new), _ptr(v_new), _ptr(positions),
                                 _ptr(slot_mapping), N, _ptr(cos_table), _ptr(sin_table), cos_table.shape[0],
                                 _ptr(q_out), _stream(stream))
    _check(st, "pa_rope_kv_store")
    return q_out


def decode_split_tokens(num_seqs: int, num_kv_heads: int, max_seq_len: int) -> int:
    return load().pa_decode_split_tokens(num_seqs, num_kv_heads, max_seq_len)


def decode_heads_per_block(num_seqs: int, num_kv_heads: int, max_seq_len: int, split_tokens: int = 0) -> int:
    return load().pa_decode_heads_per_block(num_seqs, num_kv_heads, max_seq_len, split_tokens)


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, split_tokens=0) -> int:
    return load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                            split_tokens)


def decode_workspace(q, k_pool, max_seq_len, split_tokens=0):
    """A workspace tensor of the right size for decode(...)."""
    torch = _torch()
    nbytes = decode_workspace_bytes(q.shape[0], q.shape[1], k_pool.shape[2], k_pool.shape[3], max_seq_len,
                                    split_tokens)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)


def _decode_call(fn_name, q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale, out, workspace,
                 split_tokens, stream):
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(q, "q", k_pool.dtype)
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != k_pool.shape[3]:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    if page_table.dim() != 2 or page_table.shape[0] != q.shape[0] or seq_lens.numel() != q.shape[0]:
        raise ValueError("page_table [num_seqs, stride] and seq_lens [num_seqs] must match q")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if workspace is None:
        workspace = decode_workspace(q, k_pool, max_seq_len, split_tokens)
    _dev(workspace, "workspace")
    st = getattr(load(), fn_name)(
        ctypes.byref(pool), _ptr(q), q.shape[1], _ptr(page_table), page_table.shape[1], _ptr(seq_lens),
        q.shape[0], int(max_seq_len), float(scale), int(split_tokens), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, fn_name)
    return out


def decode(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale, out=None, workspace=None,
           split_tokens=0, stream=None):
    """Paged decode attention: q [B, H_q, D] -> out [B, H_q, D] (pool dtype)."""
    return _decode_call("pa_decode", q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale, out,
                        workspace, split_tokens, stream)


def decode_noalloc(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale, out, split_tokens=0, stream=None):
    """decode(...) without a workspace: the library's static scratch buffer
    holds the split partials, and nothing is allocated (so `out` must be
    given).  Calls that can overlap on one GPU race on that buffer."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(q, "q", k_pool.dtype)
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if out is None:
        raise ValueError("decode_noalloc allocates nothing: pass `out`")
    _dev(out, "out", q.dtype)
    if q.dim() != 3 or q.shape[2] != k_pool.shape[3] or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs, num_q_heads, head_dim]")
    if page_table.dim() != 2 or page_table.shape[0] != q.shape[0] or seq_lens.numel() != q.shape[0]:
        raise ValueError("page_table [num_seqs, stride] and seq_lens [num_seqs] must match q")
    st = load().pa_decode_noalloc(ctypes.byref(pool), _ptr(q), q.shape[1], _ptr(page_table), page_table.shape[1],
                                  _ptr(seq_lens), q.shape[0], int(max_seq_len), float(scale), int(split_tokens),
                                  _ptr(out), _stream(stream))
    _check(st, "pa_decode_noalloc")
    return out


def decode_partial(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale, out, workspace,
                   split_tokens=0, stream=None):
    """First kernel of decode (per-piece partials; single-piece rows to out)."""
    return _decode_call("pa_decode_partial", q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale,
                        out, workspace, split_tokens, stream)


def decode_combine(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale, out, workspace,
                   split_tokens=0, stream=None):
    """Second kernel of decode (merge pieces into out)."""
    return _decode_call("pa_decode_combine", q, k_pool, v_pool, page_table, seq_lens, max_seq_len, scale,
                        out, workspace, split_tokens, stream)


def extend_workspace_bytes(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                           split_tokens=0) -> int:
    """Workspace of extend(...) for these sizes: 0 when the keys are not split."""
    return load().pa_extend_workspace_bytes(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                            split_tokens)


def extend(q, q_indptr, k_pool, v_pool, page_table, seq_lens, max_q_len, max_seq_len, scale, out=None,
           stream=None, split_tokens=0, workspace=None):
    """Paged extend attention: q [T_q, H_q, D] bf16 -> out [T_q, H_q, D] bf16.
    split_tokens: keys per piece (0 = automatic; >= max_seq_len: no split)."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16)
    _dev(q_indptr, "q_indptr", torch.int32)
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != k_pool.shape[3]:
        raise ValueError("q must be [T_q, num_q_heads, head_dim]")
    B = seq_lens.numel()
    if q_indptr.numel() != B + 1 or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("q_indptr [B+1], page_table [B, stride], seq_lens [B] must agree")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if workspace is None:
        nbytes = extend_workspace_bytes(B, int(max_q_len), q.shape[1], k_pool.shape[2], k_pool.shape[3],
                                        int(max_seq_len), int(split_tokens))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().pa_extend(ctypes.byref(pool), _ptr(q), q.shape[1], _ptr(q_indptr), _ptr(page_table),
                          page_table.shape[1], _ptr(seq_lens), B, int(max_q_len), int(max_seq_len),
                          float(scale), int(split_tokens), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "pa_extend")
    return out


def cascade_piece_keys(num_groups, max_group_size, num_q_heads, num_kv_heads, max_shared_len) -> int:
    return load().pa_cascade_piece_keys(num_groups, max_group_size, num_q_heads, num_kv_heads, max_shared_len)


def decode_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, num_groups,
                                   max_group_size, max_shared_len, split_tokens=0, prefix_piece_keys=0) -> int:
    return load().pa_decode_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                    split_tokens, num_groups, max_group_size, max_shared_len,
                                                    prefix_piece_keys)


def decode_cascade(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, group_starts, max_group_size,
                   prefix_page_table, shared_lens, max_shared_len, scale, out=None, workspace=None,
                   split_tokens=0, prefix_piece_keys=0, stream=None, stage=None, k_new=None, v_new=None,
                   slot_mapping=None):
    """Decode of requests that share prefix pages: group j is requests
    group_starts[j]..group_starts[j+1]-1, whose first shared_lens[b] keys sit
    on prefix_page_table[j].  Same result as decode(...).  `stage` ("order",
    "prefix", "suffix" or "combine") enqueues only that kernel ("order" before
    "suffix"; "prefix" may run on another stream beside those two; "combine"
    after all three).  k_new, v_new [N, H_kv, D] and slot_mapping int64 [N]
    (optional): the step's new rows, stored by the work-order launch (the
    single call, or stage "order") as kv_store(...) would."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16)
    n_new = 0
    if slot_mapping is not None:
        _dev(k_new, "k_new", k_pool.dtype)
        _dev(v_new, "v_new", k_pool.dtype)
        _dev(slot_mapping, "slot_mapping", torch.int64)
        n_new = slot_mapping.numel()
        if k_new.shape[0] != n_new or v_new.shape[0] != n_new:
            raise ValueError("k_new, v_new and slot_mapping must have the same number of rows")
    for t, n in ((page_table, "page_table"), (seq_lens, "seq_lens"), (group_starts, "group_starts"),
                 (prefix_page_table, "prefix_page_table"), (shared_lens, "shared_lens")):
        _dev(t, n, torch.int32)
    if q.dim() != 3 or q.shape[2] != k_pool.shape[3]:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    B = q.shape[0]
    if page_table.dim() != 2 or page_table.shape[0] != B or seq_lens.numel() != B or shared_lens.numel() != B:
        raise ValueError("page_table [B, stride], seq_lens [B] and shared_lens [B] must match q")
    ng = group_starts.numel() - 1
    if ng < 0 or prefix_page_table.dim() != 2 or prefix_page_table.shape[0] != ng:
        raise ValueError("group_starts [num_groups+1] and prefix_page_table [num_groups, stride] must agree")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if workspace is None:
        nbytes = decode_cascade_workspace_bytes(B, q.shape[1], k_pool.shape[2], k_pool.shape[3], max_seq_len, ng,
                                                max_group_size, max_shared_len, split_tokens, prefix_piece_keys)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    fn = "pa_decode_cascade" + ("" if stage is None else "_" + stage)
    if fn not in SIGNATURES:
        raise ValueError(f"unknown cascade stage {stage!r}")
    st = getattr(load(), fn)(
        ctypes.byref(pool), _ptr(q), q.shape[1], _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B,
        int(max_seq_len), _ptr(group_starts), ng, int(max_group_size), _ptr(prefix_page_table),
        prefix_page_table.shape[1], _ptr(shared_lens), int(max_shared_len), float(scale), int(split_tokens),
        int(prefix_piece_keys), _ptr(k_new if n_new else None), _ptr(v_new if n_new else None),
        _ptr(slot_mapping if n_new else None), n_new, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, fn)
    return out


def attend_mixed(q, q_indptr, k_pool, v_pool, page_table, seq_lens, max_q_len, max_seq_len, scale, out=None,
                 workspace=None, split_tokens=0, stream=None):
    """Mixed prefill + decode batch: q [T_q, H_q, D] bf16 -> out [T_q, H_q, D];
    one-row requests take the split-K decode kernels, the others the extend
    kernel.  Same result as extend(...)."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16)
    _dev(q_indptr, "q_indptr", torch.int32)
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != k_pool.shape[3]:
        raise ValueError("q must be [T_q, num_q_heads, head_dim]")
    B = seq_lens.numel()
    if q_indptr.numel() != B + 1 or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("q_indptr [B+1], page_table [B, stride], seq_lens [B] must agree")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if workspace is None:
        nbytes = decode_workspace_bytes(B, q.shape[1], k_pool.shape[2], k_pool.shape[3], max_seq_len, split_tokens)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    st = load().pa_attend_mixed(ctypes.byref(pool), _ptr(q), q.shape[1], _ptr(q_indptr), _ptr(page_table),
                                page_table.shape[1], _ptr(seq_lens), B, int(max_q_len), int(max_seq_len),
                                float(scale), int(split_tokens), _ptr(out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "pa_attend_mixed")
    return out


def verify_workspace_bytes(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                           split_tokens=0) -> int:
    return load().pa_verify_workspace_bytes(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                            split_tokens)


def verify(q, q_indptr, k_pool, v_pool, page_table, seq_lens, max_q_len, max_seq_len, scale, out=None,
           workspace=None, split_tokens=0, stream=None):
    """Short-chunk extend (verification of drafted tokens): q [T_q, H_q, D]
    bf16 -> out [T_q, H_q, D]; same result as extend(...)."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16)
    _dev(q_indptr, "q_indptr", torch.int32)
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != k_pool.shape[3]:
        raise ValueError("q must be [T_q, num_q_heads, head_dim]")
    B = seq_lens.numel()
    if q_indptr.numel() != B + 1 or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("q_indptr [B+1], page_table [B, stride], seq_lens [B] must agree")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if workspace is None:
        nbytes = verify_workspace_bytes(B, max_q_len, q.shape[1], k_pool.shape[2], k_pool.shape[3], max_seq_len,
                                        split_tokens)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    st = load().pa_verify(ctypes.byref(pool), _ptr(q), q.shape[1], _ptr(q_indptr), _ptr(page_table),
                          page_table.shape[1], _ptr(seq_lens), B, int(max_q_len), int(max_seq_len), float(scale),
                          int(split_tokens), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                          _stream(stream))
    _check(st, "pa_verify")
    return out


CHECK_BITS = {1: "seq_len", 2: "q_indptr", 4: "page_id", 8: "slot_range", 16: "slot_duplicate",
              32: "group_starts", 64: "shared_len", 128: "prefix_page"}


def check_batch(k_pool, v_pool, page_table, seq_lens, max_seq_len, q_indptr=None, max_q_len=0, slot_mapping=None,
                stream=None):
    """Debug check of the device-resident batch description; synchronises and
    returns the names of the violations found (empty: none)."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(q_indptr, "q_indptr", torch.int32)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    flags = torch.empty(1, dtype=torch.int32, device=k_pool.device)
    n_rows = 0 if slot_mapping is None else slot_mapping.numel()
    st = load().pa_check_batch(ctypes.byref(pool), _ptr(page_table), page_table.shape[1], _ptr(seq_lens),
                               seq_lens.numel(), int(max_seq_len), _ptr(q_indptr), int(max_q_len),
                               _ptr(slot_mapping), n_rows, _ptr(flags), _stream(stream))
    _check(st, "pa_check_batch")
    return _read_flags(flags, stream)


def _read_flags(flags, stream):
    """Names of the bits set in a check's flag word, read after the check's
    own stream has finished (it need not be the current stream)."""
    torch = _torch()
    (stream if stream is not None else torch.cuda.current_stream()).synchronize()
    word = int(flags.item()) & 0xFFFFFFFF
    return sorted(name for bit, name in CHECK_BITS.items() if word & bit)


def check_cascade(k_pool, v_pool, page_table, seq_lens, group_starts, max_group_size, prefix_page_table,
                  shared_lens, max_shared_len, stream=None):
    """Debug check of a cascade decode's group description (group starts,
    shared lengths, prefix pages against each request's own pages);
    synchronises and returns the names of the violations found."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    for t, n in ((page_table, "page_table"), (seq_lens, "seq_lens"), (group_starts, "group_starts"),
                 (prefix_page_table, "prefix_page_table"), (shared_lens, "shared_lens")):
        _dev(t, n, torch.int32)
    flags = torch.empty(1, dtype=torch.int32, device=k_pool.device)
    st = load().pa_check_cascade(ctypes.byref(pool), _ptr(page_table), page_table.shape[1], _ptr(seq_lens),
                                 seq_lens.numel(), _ptr(group_starts), group_starts.numel() - 1, int(max_group_size),
                                 _ptr(prefix_page_table), prefix_page_table.shape[1], _ptr(shared_lens),
                                 int(max_shared_len), _ptr(flags), _stream(stream))
    _check(st, "pa_check_cascade")
    return _read_flags(flags, stream)


def gather(k_pool, v_pool, page_table, seq_lens, out_offsets, max_seq_len, k_out, v_out, stream=None):
    """Copy each request's first seq_lens[b] tokens to rows out_offsets[b].. of
    k_out / v_out [total, H_kv, D]."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool)
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(out_offsets, "out_offsets", torch.int64)
    _dev(k_out, "k_out", k_pool.dtype)
    _dev(v_out, "v_out", k_pool.dtype)
    st = load().pa_gather(ctypes.byref(pool), _ptr(page_table), page_table.shape[1], _ptr(seq_lens),
                          _ptr(out_offsets), seq_lens.numel(), int(max_seq_len), _ptr(k_out), _ptr(v_out),
                          _stream(stream))
    _check(st, "pa_gather")


def stream_read(src, sink, stream=None):
    """Read every byte of the GPU tensor `src` (calibration of the read-only
    HBM rate); ORs a nonzero digest into `sink` (int32 [1] on the GPU)."""
    _dev(src, "src")
    _dev(sink, "sink")
    st = load().pa_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream))
    _check(st, "pa_stream_read")

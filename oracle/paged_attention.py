"""Plain CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg import this module; the product path (the HIP
library and its binding) never does, and this module imports nothing from it.

It computes, slowly, what the pages define, in float64 by default or, with
acc="f32", in float32 throughout (the inputs are bf16 or fp32, which float32
holds exactly; only the arithmetic is rounded):

* Pool layout -- K and V live in fixed-size pages, each page holding
  page_size token rows of [num_kv_heads, head_dim] ("NHD"): nanoSGLang README,
  section Architecture (block-based KV cache in FlashInfer's NHD layout) and
  section Features (paged KV cache, zero-copy NHD paged attention).
* Page-table indirection -- a request's token t lives in physical page
  page_table[t // page_size] at offset t % page_size: nanoSGLang README,
  section Ablation (page-table indirection replaces the per-token copy);
  mini-sglang from Scratch, section "What you will be able to do" (paged KV
  pool, page table, token pool); mini-sglang README, section TODO (page size
  one and page size above one).
* The store -- each new K/V row is written to the flat slot given for it:
  mini-sglang from Scratch, section "How this book works" (the KV-cache
  writes).
* Attention -- Mini-SGLang README (yangyonggit fork), section Reference
  Attention Backends, the torch backend: gather the request's pages, map
  query heads to KV heads the way repeat_interleave expands them (query head
  h reads KV head h // G with G = H_q / H_kv), and attend causally with the
  prefix-cache offset (a chunk of n new tokens after a cached prefix of p
  tokens: new token i sits at absolute position p + i and sees keys 0..p+i).
* Split softmax and its combine -- the same attention computed over
  contiguous pieces of the key range and merged by log-sum-exp weights; the
  triton backend of the same section computes the softmax online, which is
  this merge applied one block at a time.

Readings where the pages are silent (each is listed in the design notes):
the context length counts the new token; the scale is 1/sqrt(head_dim) passed
as a float32 value; no soft-cap, window or bias; an empty sequence gives a
zero row; slots below zero in a slot mapping are padding and skipped;
duplicate slots are rejected.

bf16 arrays are carried as uint16 bit patterns and widened exactly.
Results are returned as float64 arrays in both precisions.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# element formats
# --------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a pool/query array in its storage format."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


ACC_TYPES = {"f64": np.float64, "f32": np.float32}


def _acc_type(acc: str):
    """numpy type of the arithmetic: "f64" or "f32"."""
    if acc not in ACC_TYPES:
        raise ValueError(f"unknown accumulation precision {acc!r}")
    return ACC_TYPES[acc]


# --------------------------------------------------------------------------
# the store and the page-table addressing
# --------------------------------------------------------------------------
def kv_store(k_pool, v_pool, k_new, v_new, slot_mapping) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with new row i written to flat slot
    slot_mapping[i] (page * page_size + offset); rows whose slot is negative
    are padding and skipped.  A byte copy: no conversion."""
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    live = slot_mapping[slot_mapping >= 0]
    if len(np.unique(live)) != len(live):
        raise ValueError("duplicate slots in slot_mapping")
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    if live.size and live.max() >= num_pages * P:
        raise ValueError("slot out of range")
    k_out, v_out = k_pool.copy(), v_pool.copy()
    k_flat = k_out.reshape(num_pages * P, *k_pool.shape[2:])
    v_flat = v_out.reshape(num_pages * P, *v_pool.shape[2:])
    for i, s in enumerate(slot_mapping):
        if s < 0:
            continue
        k_flat[s] = k_new[i]
        v_flat[s] = v_new[i]
    return k_out, v_out


def token_slots(page_table_row: Sequence[int], length: int, page_size: int) -> List[int]:
    """Flat slot of each of a request's first `length` tokens."""
    return [int(page_table_row[t // page_size]) * page_size + t % page_size for t in range(length)]


def gather(pool: np.ndarray, page_table_row, length: int) -> np.ndarray:
    """A request's rows [length, num_kv_heads, head_dim] in logical order,
    copied out of the paged pool (storage format unchanged)."""
    num_pages, P = pool.shape[0], pool.shape[1]
    flat = pool.reshape(num_pages * P, *pool.shape[2:])
    idx = np.asarray(token_slots(page_table_row, length, P), dtype=np.int64)
    return flat[idx]


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: repeat_interleave of the KV heads by
    G = H_q / H_kv puts KV head g at query heads g*G .. g*G+G-1."""
    return h // (num_q_heads // num_kv_heads)


def visible(i, j, prefix):
    """Causal rule with the prefix-cache offset: new token i (absolute
    position prefix + i) sees key j iff j <= prefix + i."""
    return j <= prefix + i


def _softmax_rows_attend(s: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(s) @ V along the last axis of s; rows of s with no finite
    entry (no visible key) give zero."""
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    den = e.sum(axis=-1, keepdims=True)
    num = e @ V
    return np.divide(num, den, out=np.zeros_like(num), where=den > 0)


def decode(q, k_pool, v_pool, page_table, seq_lens, scale: float, dtype: str, acc: str = "f64") -> np.ndarray:
    """One new token per request attends every key of its request.

    q [B, H_q, D]; returns float64 [B, H_q, D].  For request b with L_b keys
    and query head h (KV head g = h // G):  out = softmax(scale * K_g q) V_g.
    acc: precision of the arithmetic ("f64" or "f32").
    """
    at = _acc_type(acc)
    scale = at(scale)
    q = widen(q, dtype).astype(at)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K = widen(gather(k_pool, page_table[b], L), dtype).astype(at)  # [L, Hkv, D]
        V = widen(gather(v_pool, page_table[b], L), dtype).astype(at)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s = scale * (K[:, g, :] @ q[b, h])
            out[b, h] = _softmax_rows_attend(s[None, :], V[:, g, :])[0]
    return out


def extend(q, q_indptr, k_pool, v_pool, page_table, seq_lens, scale: float, dtype: str,
           acc: str = "f64") -> np.ndarray:
    """A chunk of n_b new tokens per request after a cached prefix.

    q [T_q, H_q, D] with request b's rows at q_indptr[b] .. q_indptr[b+1];
    n_b = q_indptr[b+1] - q_indptr[b], prefix p_b = seq_lens[b] - n_b.  New
    token i (absolute position p_b + i) sees keys j <= p_b + i.  Returns
    float64 [T_q, H_q, D].  acc: precision of the arithmetic.
    """
    at = _acc_type(acc)
    scale = at(scale)
    q = widen(q, dtype).astype(at)
    T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    out = np.zeros((T, Hq, D), np.float64)
    B = len(seq_lens)
    for b in range(B):
        r0, r1 = int(q_indptr[b]), int(q_indptr[b + 1])
        n, L = r1 - r0, int(seq_lens[b])
        if n == 0:
            continue
        p = L - n
        if p < 0:
            raise ValueError("chunk longer than the sequence")
        K = widen(gather(k_pool, page_table[b], L), dtype).astype(at)
        V = widen(gather(v_pool, page_table[b], L), dtype).astype(at)
        i = np.arange(n)[:, None]
        j = np.arange(L)[None, :]
        mask = visible(i, j, p)  # [n, L]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s = scale * (q[r0:r1, h, :] @ K[:, g, :].T)
            s = np.where(mask, s, -np.inf)
            out[r0:r1, h] = _softmax_rows_attend(s, V[:, g, :])
    return out


# --------------------------------------------------------------------------
# split softmax and combine
# --------------------------------------------------------------------------
def decode_partials(q, k_pool, v_pool, page_table, seq_lens, scale: float, dtype: str,
                    split_tokens: int):
    """Attention of each request's new token over consecutive key ranges
    [s*split_tokens, (s+1)*split_tokens): per range, the normalised output
    o_s and the natural log-sum-exp lse_s of the scaled scores.

    Returns (o [B, H_q, S, D], lse [B, H_q, S], n_splits [B]) in float64, with
    S = max number of ranges; ranges past a request's length are unused
    (o = 0, lse = -inf).
    """
    q = widen(q, dtype)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    n_splits = np.array([(int(L) + split_tokens - 1) // split_tokens for L in seq_lens], np.int64)
    S = int(n_splits.max()) if B else 0
    o = np.zeros((B, Hq, S, D), np.float64)
    lse = np.full((B, Hq, S), -np.inf, np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K = widen(gather(k_pool, page_table[b], L), dtype)
        V = widen(gather(v_pool, page_table[b], L), dtype)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s_all = scale * (K[:, g, :] @ q[b, h])
            for s in range(int(n_splits[b])):
                lo, hi = s * split_tokens, min(L, (s + 1) * split_tokens)
                sc = s_all[lo:hi]
                m = sc.max()
                e = np.exp(sc - m)
                o[b, h, s] = (e @ V[lo:hi, g, :]) / e.sum()
                lse[b, h, s] = m + math.log(e.sum())
    return o, lse, n_splits


def combine(o, lse, n_splits) -> np.ndarray:
    """Merge per-range outputs: out = sum_s w_s o_s / sum_s w_s with
    w_s = exp(lse_s - max_s lse_s).  A request with no ranges gives zero."""
    B, Hq, S, D = o.shape
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        n = int(n_splits[b])
        if n == 0:
            continue
        l = lse[b, :, :n]
        w = np.exp(l - l.max(axis=1, keepdims=True))  # [Hq, n]
        out[b] = np.einsum("hs,hsd->hd", w, o[b, :, :n, :]) / w.sum(axis=1)[:, None]
    return out

"""Plain CPU oracle for the rotary position embedding applied on the way into
the paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg import this module; the product path never does.

What is computed:

* Rotary embedding with half-split pairing -- channel i of a head is paired
  with channel i + D/2 (the rotate_half convention of the HF Llama/Qwen
  checkpoints), not with its neighbour: nanoSGLang README, section Notable
  Fixes (the RoPE convention bug).  For a row at position p the pair
  (a, b) = (x[i], x[i + D/2]) becomes
      (a * cos(p, i) - b * sin(p, i),  b * cos(p, i) + a * sin(p, i)),
  a rotation of the point (a, b) by the angle whose cosine and sine the
  caller's table holds for (p, i).
* The store that follows -- the rotated key row and the value row go to the
  flat slot the slot mapping gives: mini-sglang from Scratch, section "How
  this book works" (RoPE and the KV-cache writes each have a plain reference
  version); a negative slot marks a padding row, for which nothing is read
  or written.

The cosine and sine tables [max_position, D/2] are inputs, as an engine keeps
them precomputed; this module never builds them.  Results are float64; the
pools keep their storage format, and the slots written with rotated keys are
reported separately so a caller can compare them at the precision it wants.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .paged_attention import widen


def rope(x, positions, cos_table, sin_table, dtype: str) -> np.ndarray:
    """x [N, H, D] in its storage format, positions [N]; returns the rotated
    rows in float64 [N, H, D].  Pair (i, i + D/2) turns by the table's angle
    for (positions[n], i)."""
    xf = widen(x, dtype)
    N, H, D = xf.shape
    if D % 2:
        raise ValueError("head_dim must be even")
    half = D // 2
    cos_t = np.asarray(cos_table, np.float64)
    sin_t = np.asarray(sin_table, np.float64)
    if cos_t.shape[1] != half or sin_t.shape != cos_t.shape:
        raise ValueError("tables must be [max_position, head_dim / 2]")
    out = np.empty_like(xf)
    for n in range(N):
        p = int(positions[n])
        if not 0 <= p < cos_t.shape[0]:
            raise ValueError("position outside the table")
        c, s = cos_t[p], sin_t[p]  # [half]
        a, b = xf[n, :, :half], xf[n, :, half:]
        out[n, :, :half] = a * c - b * s
        out[n, :, half:] = b * c + a * s
    return out


def rope_kv_store(k_pool, v_pool, q, k_new, v_new, positions, slot_mapping, cos_table, sin_table,
                  dtype: str) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """The fused step: rotate q and k of every live row, store the rotated k
    and the unchanged v at the row's slot.

    Returns (q_rot, k_rot, live, k_pool_out, v_pool_out):
      q_rot [N, H_q, D], k_rot [N, H_kv, D] float64 (rows of padding are NaN);
      live  [N] bool, the rows with a slot >= 0;
      v_pool_out: the v pool with v_new[i] copied byte for byte to slot i;
      k_pool_out: the k pool with the written slots left as they were (their
      expected content is k_rot, at whatever precision the caller compares).
    Duplicate live slots are rejected."""
    slots = np.asarray(slot_mapping, np.int64)
    live = slots >= 0
    ls = slots[live]
    if len(np.unique(ls)) != len(ls):
        raise ValueError("duplicate slots in slot_mapping")
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    if ls.size and ls.max() >= num_pages * P:
        raise ValueError("slot out of range")
    pos = np.asarray(positions, np.int64)
    q_rot = np.full(widen(q, dtype).shape, np.nan)
    k_rot = np.full(widen(k_new, dtype).shape, np.nan)
    if live.any():
        q_rot[live] = rope(np.asarray(q)[live], pos[live], cos_table, sin_table, dtype)
        k_rot[live] = rope(np.asarray(k_new)[live], pos[live], cos_table, sin_table, dtype)
    v_out = v_pool.copy()
    v_flat = v_out.reshape(num_pages * P, *v_pool.shape[2:])
    for i, s in enumerate(slots):
        if s >= 0:
            v_flat[s] = v_new[i]
    return q_rot, k_rot, live, k_pool.copy(), v_out

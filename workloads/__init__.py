"""Seeded synthetic inputs for attention over a paged KV cache.

This module only draws inputs: sequence lengths, a page assignment (what a
serving engine's page allocator would hand out), pool contents, queries, and
the new K/V rows together with the slots they are stored to.  It holds none of
the attention arithmetic.  The CPU oracle's tests, the GPU parity tests and the
benchmark all take their inputs from here, so both sides see the same bytes.

Layout conventions (the pages' NHD paged pool):
  k_pool, v_pool   [num_pages, page_size, num_kv_heads, head_dim]
  page_table       int32 [B, stride]; entry j is the physical page that holds
                   the request's tokens j*page_size .. (j+1)*page_size-1
  seq_lens         int32 [B]; keys per request *including* the new tokens
  slot_mapping     int64 [N]; flat slot (page*page_size + offset) of new row i
bf16 tensors are carried as their raw uint16 bit patterns.

The five named configurations mirror the workloads the pages describe
(nanoSGLang's Qwen2.5-0.5B benchmark, mini-sglang's Qwen3-0.6B with page size
one, a Qwen3-8B decode batch with radix prefix sharing, and a chunked-prefill
extend on the same shape); values are N(0, 1) draws rounded to bf16.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 22  # values per independently seeded block (thread-count independent)


# --------------------------------------------------------------------------
# value drawing
# --------------------------------------------------------------------------
def _normal_f32(seed: int, stream: int, n: int) -> np.ndarray:
    """n standard-normal float32 values; block i of _CHUNK values comes from
    its own PCG64 stream keyed by (seed, stream, i), so the result does not
    depend on how many threads fill it."""
    out = np.empty(n, dtype=np.float32)
    nblk = (n + _CHUNK - 1) // _CHUNK

    def fill(i: int) -> None:
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(stream, i))
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        np.random.default_rng(ss).standard_normal(dtype=np.float32, out=out[lo:hi])

    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        workers = max(1, min(16, os.cpu_count() or 1, nblk))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    uint16 bit patterns.  Inputs here are finite normal draws."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:
        import torch

        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    except ImportError:  # pragma: no cover - torch is always present here
        u = x.view(np.uint32)
        return ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _values(seed: int, stream: int, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    v = _normal_f32(seed, stream, n)
    if dtype == "bf16":
        return f32_to_bf16_bits(v).reshape(shape)
    return v.reshape(shape)


# --------------------------------------------------------------------------
# the workload record
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    kind: str  # "decode" or "extend"
    dtype: str  # "f32" or "bf16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    seq_lens: np.ndarray  # int32 [B], keys incl. the new tokens
    n_new: np.ndarray  # int32 [B], new tokens (1 for decode, chunk for extend)
    q_indptr: np.ndarray  # int32 [B+1], row offsets of each request's new tokens
    page_table: np.ndarray  # int32 [B, stride]
    page_lists: List[np.ndarray]  # pages of each request in logical order
    k_pool: np.ndarray  # [num_pages, P, Hkv, D] storage dtype, before the store
    v_pool: np.ndarray
    q: np.ndarray  # [B, Hq, D] (decode) or [T_q, Hq, D] (extend)
    k_new: np.ndarray  # [N, Hkv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray  # int64 [N]
    scale: float
    seed: int
    poison: Optional[str]
    shared_pages: Dict[int, np.ndarray] = field(default_factory=dict)  # group -> pages
    group_size: int = 0  # requests per prefix-sharing group (0: no sharing)
    shared_counts: Optional[np.ndarray] = None  # [B] leading pages each request reads from its group

    def cascade_inputs(self):
        """What an engine's prefix cache knows about the sharing: requests in
        consecutive groups, each group's shared pages, and how many leading
        keys of each request sit on them.  Returns (group_starts int32 [G+1],
        prefix_page_table int32 [G, stride], shared_lens int32 [B])."""
        B, P = self.num_seqs, self.page_size
        if not self.group_size or self.shared_counts is None:
            starts = np.arange(B + 1, dtype=np.int32)
            return starts, np.zeros((B, 1), np.int32), np.zeros(B, np.int32)
        ng = (B + self.group_size - 1) // self.group_size
        starts = np.minimum(np.arange(ng + 1) * self.group_size, B).astype(np.int32)
        stride = max(1, max(len(self.shared_pages[j]) for j in range(ng)))
        ppt = np.zeros((ng, stride), np.int32)
        for j in range(ng):
            ppt[j, :len(self.shared_pages[j])] = self.shared_pages[j]
        return starts, ppt, (self.shared_counts.astype(np.int64) * P).astype(np.int32)

    def positions(self) -> np.ndarray:
        """int32 [N]: the position of each new row (new token i of request b
        sits at seq_len_b - n_b + i), the index rotary tables are read at."""
        out = np.empty(int(self.q_indptr[-1]) if self.num_seqs else 0, np.int32)
        for b in range(self.num_seqs):
            n, L = int(self.n_new[b]), int(self.seq_lens[b])
            out[self.q_indptr[b]:self.q_indptr[b + 1]] = np.arange(L - n, L)
        return out

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        return int(self.n_new.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def used_slot_set(self) -> np.ndarray:
        """Distinct flat slots that hold one of the requests' keys."""
        P = self.page_size
        parts = []
        for b in range(self.num_seqs):
            L = int(self.seq_lens[b])
            if L == 0:
                continue
            pages = self.page_lists[b]
            t = np.arange(L, dtype=np.int64)
            parts.append(pages[t // P].astype(np.int64) * P + t % P)
        if not parts:
            return np.zeros(0, np.int64)
        return np.unique(np.concatenate(parts))

    def kv_bytes_logical(self) -> int:
        return 2 * int(self.seq_lens.sum()) * self.num_kv_heads * self.head_dim * self.elem_bytes

    def kv_bytes_unique(self) -> int:
        return 2 * int(self.used_slot_set().size) * self.num_kv_heads * self.head_dim * self.elem_bytes

    def subset(self, seqs: Sequence[int]) -> "Workload":
        """The same pool with only the given requests (for sampled checks)."""
        seqs = np.asarray(list(seqs), dtype=np.int64)
        n_new = self.n_new[seqs]
        q_indptr = np.zeros(len(seqs) + 1, np.int32)
        q_indptr[1:] = np.cumsum(n_new)
        rows = np.concatenate(
            [np.arange(self.q_indptr[b], self.q_indptr[b + 1]) for b in seqs]
        ).astype(np.int64) if len(seqs) else np.zeros(0, np.int64)
        return Workload(
            name=self.name + "[subset]", kind=self.kind, dtype=self.dtype,
            num_seqs=len(seqs), num_q_heads=self.num_q_heads,
            num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
            page_size=self.page_size, num_pages=self.num_pages,
            seq_lens=self.seq_lens[seqs].copy(), n_new=n_new.copy(), q_indptr=q_indptr,
            page_table=self.page_table[seqs].copy(),
            page_lists=[self.page_lists[b] for b in seqs],
            k_pool=self.k_pool, v_pool=self.v_pool,
            q=self.q[rows] if self.kind == "extend" else self.q[seqs],
            k_new=self.k_new[rows], v_new=self.v_new[rows],
            slot_mapping=self.slot_mapping[rows], scale=self.scale, seed=self.seed,
            poison=self.poison, shared_pages=self.shared_pages,
            group_size=0, shared_counts=None,
        )


# --------------------------------------------------------------------------
# page assignment (what an allocator would produce)
# --------------------------------------------------------------------------
def _pages_needed(L: int, P: int) -> int:
    return (L + P - 1) // P


def _assign_private(rng, seq_lens, P, num_pages):
    perm = rng.permutation(num_pages).astype(np.int32)
    lists, pos = [], 0
    for L in seq_lens:
        k = _pages_needed(int(L), P)
        if pos + k > num_pages:
            raise ValueError("pool too small for the drawn lengths")
        lists.append(perm[pos:pos + k].copy())
        pos += k
    return lists, {}, None


def _assign_radix(rng, seq_lens, P, num_pages, group_size, prefix_pages):
    """Requests in consecutive groups of `group_size` share `prefix_pages`
    full pages of prefix; request b uses the first
    min(prefix_pages, (L_b - 1) // P) of them, so the page with its newest
    token is always private.  Shared and private ids come from one
    permutation of the pool."""
    B = len(seq_lens)
    ngroups = (B + group_size - 1) // group_size
    perm = rng.permutation(num_pages).astype(np.int32)
    shared = {g: perm[g * prefix_pages:(g + 1) * prefix_pages].copy() for g in range(ngroups)}
    pos = ngroups * prefix_pages
    lists, counts = [], []
    for b, L in enumerate(seq_lens):
        L = int(L)
        s = min(prefix_pages, max(0, (L - 1) // P)) if L > 0 else 0
        k = _pages_needed(L, P) - s
        if pos + k > num_pages:
            raise ValueError("pool too small for the drawn lengths")
        lists.append(np.concatenate([shared[b // group_size][:s], perm[pos:pos + k]]).astype(np.int32))
        counts.append(s)
        pos += k
    return lists, shared, np.array(counts, np.int32)


# --------------------------------------------------------------------------
# building a workload
# --------------------------------------------------------------------------
def build(
    name: str,
    kind: str,
    dtype: str,
    seq_lens: Sequence[int],
    n_new: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    page_size: int,
    num_pages: int,
    seed: int,
    rng: Optional[np.random.Generator] = None,
    poison: Optional[str] = None,
    radix: Optional[tuple] = None,
    stride: Optional[int] = None,
    with_values: bool = True,
) -> Workload:
    """Assemble a workload from explicit lengths.

    poison: None  -> every slot of a used page holds an N(0,1) draw, unused
                     pages are zero;
            "nan" -> every slot that is not a cached key (unused pages, page
                     tails, the slots the new rows go to) holds NaN;
            "zero"-> the same slots hold 0.
    radix:  (group_size, prefix_pages) for shared-prefix page assignment.
    """
    if kind not in ("decode", "extend"):
        raise ValueError(kind)
    rng = rng if rng is not None else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    n_new = np.asarray(n_new, dtype=np.int32)
    B = len(seq_lens)
    P = page_size
    if np.any(n_new > seq_lens):
        raise ValueError("more new tokens than keys")
    # -- page assignment
    if radix is not None:
        lists, shared, counts = _assign_radix(rng, seq_lens, P, num_pages, *radix)
    else:
        lists, shared, counts = _assign_private(rng, seq_lens, P, num_pages)
    max_pages = max([len(x) for x in lists] + [1])
    stride = max(stride or 0, max_pages)
    page_table = np.zeros((B, stride), np.int32)
    for b, pl in enumerate(lists):
        page_table[b, :len(pl)] = pl
    # -- cached / new slots
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    Hkv, D = num_kv_heads, head_dim
    q_indptr = np.zeros(B + 1, np.int32)
    q_indptr[1:] = np.cumsum(n_new)
    N = int(q_indptr[-1])
    slot_mapping = np.full(N, -1, np.int64)
    cached_parts = []
    for b in range(B):
        L, n = int(seq_lens[b]), int(n_new[b])
        t = np.arange(L, dtype=np.int64)
        flat = lists[b][t // P].astype(np.int64) * P + t % P
        cached_parts.append(flat[: L - n])
        slot_mapping[q_indptr[b]:q_indptr[b + 1]] = flat[L - n:]
    used_pages = np.unique(np.concatenate([x for x in lists if len(x)] + [np.zeros(0, np.int32)]))
    if not with_values:
        empty = np.zeros((0, P, Hkv, D), store_dt)
        return Workload(name, kind, dtype, B, num_q_heads, Hkv, D, P, num_pages, seq_lens, n_new,
                        q_indptr, page_table, lists, empty, empty,
                        np.zeros((0, num_q_heads, D), store_dt), np.zeros((0, Hkv, D), store_dt),
                        np.zeros((0, Hkv, D), store_dt), slot_mapping,
                        float(np.float32(1.0 / math.sqrt(D))), seed, poison, shared,
                        radix[0] if radix else 0, counts)
    # -- pool contents: draws for every slot of every used page, in page-id order
    k_pool = np.zeros((num_pages, P, Hkv, D), store_dt)
    v_pool = np.zeros((num_pages, P, Hkv, D), store_dt)
    shape = (len(used_pages), P, Hkv, D)
    k_pool[used_pages] = _values(seed, 1, shape, dtype)
    v_pool[used_pages] = _values(seed, 2, shape, dtype)
    # -- queries and new rows
    q_rows = B if kind == "decode" else N
    q = _values(seed, 3, (q_rows, num_q_heads, D), dtype)
    k_new = _values(seed, 4, (N, Hkv, D), dtype)
    v_new = _values(seed, 5, (N, Hkv, D), dtype)
    if poison is not None:
        fill = {"nan": (BF16_NAN if dtype == "bf16" else np.float32(np.nan)),
                "zero": store_dt(0)}[poison]
        keep = np.zeros(num_pages * P, bool)
        if cached_parts:
            keep[np.concatenate(cached_parts)] = True
        for pool in (k_pool, v_pool):
            flat = pool.reshape(num_pages * P, Hkv, D)
            flat[~keep] = fill
    return Workload(name, kind, dtype, B, num_q_heads, Hkv, D, P, num_pages, seq_lens, n_new,
                    q_indptr, page_table, lists, k_pool, v_pool, q, k_new, v_new, slot_mapping,
                    float(np.float32(1.0 / math.sqrt(D))), seed, poison, shared,
                    radix[0] if radix else 0, counts)


# --------------------------------------------------------------------------
# the five named configurations
# --------------------------------------------------------------------------
def _cfg_tiny(rng):
    return dict(kind="decode", dtype="f32", seq_lens=[1, 17, 33, 64], n_new=[1] * 4,
                num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, num_pages=32)


def _cfg_qwen25_05b(rng):
    L = rng.integers(100, 641, size=32)
    return dict(kind="decode", dtype="bf16", seq_lens=L, n_new=[1] * 32,
                num_q_heads=14, num_kv_heads=2, head_dim=64, page_size=16, num_pages=8000)


def _cfg_qwen3_06b_p1(rng):
    L = rng.integers(256, 2049, size=64)
    return dict(kind="decode", dtype="bf16", seq_lens=L, n_new=[1] * 64,
                num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=1, num_pages=200_000,
                stride=2048)


def _cfg_qwen3_8b_radix(rng):
    u = rng.uniform(math.log(512), math.log(8193), size=256)
    L = np.floor(np.exp(u)).astype(np.int64)
    return dict(kind="decode", dtype="bf16", seq_lens=L, n_new=[1] * 256,
                num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, num_pages=65_536,
                radix=(16, 64), stride=512)


def _cfg_qwen3_8b_extend(rng):
    p = rng.integers(0, 4097, size=8)
    return dict(kind="extend", dtype="bf16", seq_lens=p + 512, n_new=[512] * 8,
                num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, num_pages=4096,
                stride=288)


def _cfg_qwen3_8b_mixed(rng):
    # a continuous-batching step: 8 chunked-prefill requests (the extend
    # workload's shape) next to 248 decode requests (the decode workload's
    # lengths, private pages)
    p = rng.integers(0, 4097, size=8)
    u = rng.uniform(math.log(512), math.log(8193), size=248)
    L = np.concatenate([p + 512, np.floor(np.exp(u)).astype(np.int64)])
    return dict(kind="extend", dtype="bf16", seq_lens=L, n_new=[512] * 8 + [1] * 248,
                num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, num_pages=65_536, stride=512)


def _cfg_qwen3_8b_verify(rng):
    # speculative verification: k = 5 drafted tokens + 1 checked in one pass
    # per request, after a context of the decode workload's lengths
    u = rng.uniform(math.log(512), math.log(8193 - 6), size=64)
    L = np.floor(np.exp(u)).astype(np.int64) + 6
    return dict(kind="extend", dtype="bf16", seq_lens=L, n_new=[6] * 64,
                num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, num_pages=16_384, stride=512)


CONFIGS: Dict[str, tuple] = {
    # name: (default seed, spec)
    "tiny": (1, _cfg_tiny),
    "qwen25_05b": (2, _cfg_qwen25_05b),
    "qwen3_06b_p1": (3, _cfg_qwen3_06b_p1),
    "qwen3_8b_radix": (4, _cfg_qwen3_8b_radix),
    "qwen3_8b_extend": (5, _cfg_qwen3_8b_extend),
    "qwen3_8b_mixed": (6, _cfg_qwen3_8b_mixed),
    "qwen3_8b_verify": (7, _cfg_qwen3_8b_verify),
}

DESCRIPTIONS = {
    "tiny": "tiny decode: 4 seqs, lengths {1,17,33,64}, 2/1 heads, D=64, page 16, fp32",
    "qwen25_05b": "Qwen2.5-0.5B-shaped decode: 32 seqs, L~U[100,640], 14/2 heads, D=64, page 16, bf16",
    "qwen3_06b_p1": "Qwen3-0.6B-shaped decode: 64 seqs, L~U[256,2048], 16/8 heads, D=128, page 1, bf16",
    "qwen3_8b_radix": "Qwen3-8B-shaped decode: 256 seqs, L log-U[512,8192], 32/8 heads, D=128, page 16, "
                      "groups of 16 share a 1024-token prefix, bf16",
    "qwen3_8b_extend": "Qwen3-8B-shaped chunked-prefill extend: 8 reqs, prefix U[0,4096] + 512-token chunk, "
                       "32/8 heads, D=128, page 16, bf16",
    "qwen3_8b_mixed": "Qwen3-8B-shaped mixed step: 8 prefill chunks (prefix U[0,4096] + 512) and 248 decode reqs "
                      "(L log-U[512,8192]), 32/8 heads, D=128, page 16, bf16",
    "qwen3_8b_verify": "Qwen3-8B-shaped speculative verify: 64 reqs, 6 new rows (k=5 drafts + 1) after a context "
                       "log-U[512,8187], 32/8 heads, D=128, page 16, bf16",
}


def make(name: str, seed: Optional[int] = None, poison: Optional[str] = None,
         with_values: bool = True) -> Workload:
    """One of the five named configurations.  Draw order: lengths, page
    permutation, K pool, V pool, queries, new K/V rows."""
    default_seed, spec = CONFIGS[name]
    seed = default_seed if seed is None else seed
    rng = np.random.default_rng(seed)
    kw = spec(rng)
    return build(name=name, seed=seed, rng=rng, poison=poison, with_values=with_values, **kw)


def make_custom(seq_lens, num_q_heads, num_kv_heads, head_dim, page_size, dtype="bf16",
                kind="decode", n_new=None, num_pages=None, seed=0, poison="nan", radix=None,
                stride=None, name="custom") -> Workload:
    """A workload with explicit lengths, for parity sweeps and edge cases."""
    seq_lens = list(seq_lens)
    if n_new is None:
        n_new = [1 if L > 0 else 0 for L in seq_lens] if kind == "decode" else seq_lens
    if isinstance(n_new, int):
        n_new = [min(n_new, L) for L in seq_lens]
    if num_pages is None:
        need = sum(_pages_needed(int(L), page_size) for L in seq_lens)
        if radix is not None:
            need += ((len(seq_lens) + radix[0] - 1) // radix[0]) * radix[1]
        num_pages = max(4, need + need // 4 + 3)
    return build(name=name, kind=kind, dtype=dtype, seq_lens=seq_lens, n_new=n_new,
                 num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                 page_size=page_size, num_pages=num_pages, seed=seed, poison=poison,
                 radix=radix, stride=stride)


def rope_tables(max_position: int, head_dim: int, theta: float = 1.0e6):
    """The rotary cache an engine precomputes, as the inputs of the fused
    rope + store call: cos and sin of p * theta^(-2j / head_dim) for
    p < max_position, j < head_dim / 2, rounded to float32 (theta 1e6 is the
    Qwen3 value).  Input data only: neither side of the parity tests derives
    it."""
    half = head_dim // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact); used by tests to read back
    GPU outputs."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# device copies (plumbing for the GPU tests and the benchmark)
# --------------------------------------------------------------------------
@dataclass
class DeviceWorkload:
    k_pool: "object"
    v_pool: "object"
    q: "object"
    k_new: "object"
    v_new: "object"
    slot_mapping: "object"
    page_table: "object"
    seq_lens: "object"
    q_indptr: "object"


def to_device(wl: Workload, device="cuda") -> DeviceWorkload:
    """torch copies of a workload's arrays (pools before the store)."""
    import torch

    def t(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)

    def i(x, dt):
        return torch.from_numpy(np.ascontiguousarray(x).astype(dt)).to(device)

    return DeviceWorkload(
        k_pool=t(wl.k_pool), v_pool=t(wl.v_pool), q=t(wl.q), k_new=t(wl.k_new), v_new=t(wl.v_new),
        slot_mapping=i(wl.slot_mapping, np.int64), page_table=i(wl.page_table, np.int32),
        seq_lens=i(wl.seq_lens, np.int32), q_indptr=i(wl.q_indptr, np.int32))


def to_numpy_storage(t, dtype: str) -> np.ndarray:
    """A device tensor back to the storage format used here (uint16 bits for
    bf16)."""
    import torch

    x = t.detach().cpu()
    if dtype == "bf16":
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()

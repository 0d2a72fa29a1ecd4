"""Large decode batches, where the split-K partial kernel takes its pieces
from a work order built on the device (every piece that exists, the full
pieces first, then the shorter last pieces by decreasing length, then the
zero rows of empty requests).  Checked against the oracle (Mini-SGLang README,
yangyonggit fork, section Reference Attention Backends: paged gather and
naive softmax) with empty requests, more than 1024 requests, mixed batches
and the cascade's own keys; and bit for bit against the same requests in a
batch small enough to run in plain grid order: which work-group takes a piece
must not change any bit of the result."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, bits, f64, fresh, gpu_cascade, gpu_decode, pa, stored_oracle_pools, torch

pytestmark = pytest.mark.gpu

SPLIT = 64  # keys per piece; every batch below has at least 8192 work-groups (work order from 6144 on)


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def lengths(n, hi, seed, zeros=0.05):
    """A ragged mix: empty requests, one key, piece boundaries and their
    neighbours, and uniform lengths up to hi."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, 2, 63, 64, 65, 127, 128, 129, hi]
    L = rng.integers(1, hi + 1, n)
    pick = rng.random(n) < 0.3
    L[pick] = rng.choice([e for e in edges if e <= hi], int(pick.sum()))
    L[rng.random(n) < zeros] = 0
    return [int(x) for x in L]


@pytest.mark.parametrize("B,hi", [(1500, 128), (700, 300)])
def test_large_decode_batch_matches_oracle(B, hi):
    lens = lengths(B, hi, seed=B)
    banner(f"decode B={B} lengths<= {hi} split {SPLIT}")
    wl = W.make_custom(lens, 16, 8, 64, 16, dtype="bf16", seed=1000 + B)
    S = (wl.max_seq_len + SPLIT - 1) // SPLIT
    assert B * 8 * S >= 8192
    dw = fresh(wl)
    out = gpu_decode(wl, dw, split=SPLIT)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, f"decode B={B}")
    zero = [b for b, L in enumerate(lens) if L == 0]
    assert zero and np.all(f64(out)[zero] == 0)
    print(f"[result] max abs err {err:.3g}", flush=True)

    # the same requests in a small batch run in grid order: identical bits
    seqs = sorted(set(range(0, B, 13)) | set(zero[:5]))
    sub = wl.subset(seqs)
    assert len(seqs) * 8 * ((sub.max_seq_len + SPLIT - 1) // SPLIT) < 6144
    out_sub = gpu_decode(sub, fresh(sub), split=SPLIT)
    assert bits(out_sub) == bits(out[seqs])


@pytest.mark.parametrize("B,hkv,hq,hi,split", [
    (997, 4, 16, 300, 64),      # one block of four KV heads: eight request ranges, 997 = 8 * 124 + 5
    (403, 8, 32, 2200, 1024),   # two heads per block, four blocks: two ranges of 201 and 202 requests
    (5, 4, 8, 20000, 64),       # fewer requests than ranges: some ranges hold none
])
def test_decode_request_ranges_match_oracle(B, hkv, hq, hi, split):
    """The work order cuts the batch into 8 / gcd(head blocks, 8) contiguous
    request ranges and interleaves their full pieces (so that each range's
    pieces of a head block run on one XCD); uneven and empty ranges included.
    Checked against the oracle and bit for bit against the same requests in
    plain grid order."""
    lens = lengths(B, hi, seed=B + hkv)
    lens[0] = hi  # sets the grid
    D = 64 if hkv == 4 else 128
    banner(f"decode B={B} kv heads {hkv} q heads {hq} lengths<= {hi} split {split}")
    wl = W.make_custom(lens, hq, hkv, D, 16, dtype="bf16", seed=2000 + B)
    S = (wl.max_seq_len + split - 1) // split
    assert B * hkv * S >= 6144  # the work order is used
    dw = fresh(wl)
    out = gpu_decode(wl, dw, split=split)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, f"decode ranges B={B}")
    print(f"[result] max abs err {err:.3g}", flush=True)

    seqs = [0, 3] if B < 13 else list(range(0, B, 13))
    sub = wl.subset(seqs)
    assert len(seqs) * hkv * ((sub.max_seq_len + split - 1) // split) < 6144
    out_sub = gpu_decode(sub, fresh(sub), split=split)
    assert bits(out_sub) == bits(out[seqs])


def test_large_mixed_batch_matches_oracle():
    """Decode requests next to short chunks: the work order lists only the
    one-row requests."""
    B = 1100
    rng = np.random.default_rng(77)
    lens = [max(1, L) for L in lengths(B, 200, seed=78, zeros=0.0)]  # every request has its new row
    n_new = [1] * B
    for b in rng.choice(B, 40, replace=False):
        n_new[b] = int(min(lens[b], rng.integers(2, 40)))
    banner(f"mixed B={B}: {sum(n > 1 for n in n_new)} chunks, split {SPLIT}")
    wl = W.make_custom(lens, 16, 8, 64, 16, dtype="bf16", kind="extend", n_new=n_new, seed=79)
    dw = fresh(wl)
    out = pa().attend_mixed(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                            wl.max_seq_len, wl.scale, split_tokens=SPLIT)
    torch().cuda.synchronize()
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, "mixed large batch")
    print(f"[result] max abs err {err:.3g}", flush=True)


def test_large_cascade_batch_matches_oracle():
    """Groups of 8 requests sharing 64 keys; each request's own keys go
    through the work order (the pieces start at the shared length)."""
    B = 1200
    lens = [max(65, L) for L in lengths(B, 320, seed=81, zeros=0.0)]
    banner(f"cascade B={B} groups of 8 sharing 64 keys, split {SPLIT}")
    wl = W.make_custom(lens, 16, 8, 64, 16, dtype="bf16", radix=(8, 64), seed=82)
    dw = fresh(wl)
    out = gpu_cascade(wl, dw, split=SPLIT, piece_keys=64)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, "cascade large batch")
    print(f"[result] max abs err {err:.3g}", flush=True)
    again = gpu_cascade(wl, dw, split=SPLIT, piece_keys=64)
    assert bits(again) == bits(out)


def test_largest_pieces_in_work_order():
    """2048-key pieces (the largest split) on a batch large enough for the
    work order, lengths around the piece boundaries."""
    B = 260
    rng = np.random.default_rng(90)
    lens = rng.integers(1, 601, B)  # mostly short: the few long requests set the grid
    lens[:8] = [1, 2047, 2048, 2049, 4095, 4096, 4097, 6000]
    lens = [int(x) for x in lens]
    banner(f"decode B={B} lengths<= 6000 split 2048")
    wl = W.make_custom(lens, 32, 8, 128, 16, dtype="bf16", seed=91)
    assert B * 8 * ((wl.max_seq_len + 2047) // 2048) >= 6144
    dw = fresh(wl)
    out = gpu_decode(wl, dw, split=2048)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, "decode split 2048")
    print(f"[result] max abs err {err:.3g}", flush=True)


def test_large_cascade_without_groups():
    """No shared pages: the cascade's first stage only writes the work order
    of the own-keys pass (no prefix kernel runs)."""
    B = 900
    lens = lengths(B, 300, seed=85)
    banner(f"cascade B={B} without groups, split {SPLIT}")
    wl = W.make_custom(lens, 16, 8, 64, 16, dtype="bf16", seed=86)
    dw = fresh(wl)
    out = gpu_cascade(wl, dw, split=SPLIT)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, "cascade without groups")
    print(f"[result] max abs err {err:.3g}", flush=True)

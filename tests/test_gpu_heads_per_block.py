"""Decode work-groups that serve several neighbouring KV heads (two or four)
of the same keys, one or two waves per head.  Checked against the oracle
(Mini-SGLang README, yangyonggit fork, section Reference Attention Backends:
paged gather, GQA by repeat_interleave, naive softmax) for every group size,
head dim, page size and dtype the plain decode takes, through the plain, the
cascade and the mixed calls, with the automatic split of a large batch and
with explicit splits; and bit for bit across batches at an explicit split,
where the heads per work-group depend only on the split and the head count."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, bits, f64, fresh, gpu_cascade, gpu_decode, pa, stored_oracle_pools, torch

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def ragged(n, hi, seed, long=()):
    """Empty requests, one key, piece boundaries and uniform lengths up to
    hi, then the given long requests."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 513]
    L = rng.integers(1, hi + 1, n)
    pick = rng.random(n) < 0.4
    L[pick] = rng.choice([e for e in edges if e <= hi], int(pick.sum()))
    return [int(x) for x in L] + list(long)


def oracle_decode(wl):
    kp, vp = stored_oracle_pools(wl)
    return oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)


@pytest.mark.parametrize("Hq,Hkv,D,P,dtype,split,hb", [
    (32, 8, 128, 16, "bf16", 512, 4),   # Qwen3-8B heads: four KV heads per work-group
    (32, 8, 128, 16, "bf16", 64, 4),    # shortest pieces
    (32, 4, 128, 16, "bf16", 256, 4),   # group of 8
    (16, 8, 128, 1, "bf16", 320, 4),    # page size 1, group of 2
    (14, 2, 64, 16, "bf16", 1024, 2),   # Qwen2.5-0.5B heads: pairs, two waves per head
    (18, 6, 64, 16, "bf16", 512, 2),    # group of 3, six KV heads: pairs
    (8, 8, 128, 16, "bf16", 128, 4),    # group of 1
    (20, 4, 64, 16, "bf16", 128, 4),    # group of 5
    (8, 4, 128, 16, "f32", 64, 4),      # fp32 pools
    (16, 2, 64, 1, "f32", 1024, 2),     # fp32, page size 1, group of 8
])
def test_explicit_split_matches_oracle(Hq, Hkv, D, P, dtype, split, hb):
    banner(f"heads per block {hb}: {Hq}/{Hkv} D={D} P={P} {dtype} split {split}")
    lens = ragged(40, 700, seed=Hq * 100 + Hkv * 10 + D, long=[2 * split - 1, 2 * split, 2 * split + 1, 3000])
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype=dtype, seed=Hq + Hkv + D + P)
    assert pa().decode_heads_per_block(wl.num_seqs, Hkv, wl.max_seq_len, split) == hb
    out = gpu_decode(wl, fresh(wl), split=split)
    err = assert_close(f64(out), oracle_decode(wl), "decode")
    zero = [b for b, L in enumerate(lens) if L == 0]
    assert np.all(f64(out)[zero] == 0)
    print(f"[result] max abs err {err:.3g}", flush=True)


def big_batch(seed, radix=None):
    """160 requests, mostly short, a few up to 8192 keys: the automatic split
    takes two KV heads per work-group and 1024-key pieces, in the work order."""
    lens = ragged(152, 600, seed=seed, long=[1, 1024, 2047, 4096, 5000, 6001, 7777, 8192])
    return W.make_custom(lens, 32, 8, 128, 16, dtype="bf16", seed=seed, radix=radix)


def test_automatic_split_of_a_large_batch():
    wl = big_batch(501)
    banner(f"automatic split B={wl.num_seqs} max {wl.max_seq_len}")
    assert pa().decode_heads_per_block(wl.num_seqs, 8, wl.max_seq_len) == 2
    assert pa().decode_split_tokens(wl.num_seqs, 8, wl.max_seq_len) == 1024
    dw = fresh(wl)
    out = gpu_decode(wl, dw)
    err = assert_close(f64(out), oracle_decode(wl), "decode automatic split")
    assert bits(gpu_decode(wl, dw)) == bits(out)  # reruns identical
    print(f"[result] max abs err {err:.3g}", flush=True)


def test_cascade_own_keys_with_two_heads_per_work_group():
    wl = big_batch(502, radix=(16, 40))
    banner(f"cascade B={wl.num_seqs} groups of 16 sharing 40 pages")
    assert pa().decode_heads_per_block(wl.num_seqs, 8, wl.max_seq_len) == 2
    dw = fresh(wl)
    ref = oracle_decode(wl)
    out = gpu_cascade(wl, dw)
    err = assert_close(f64(out), ref, "cascade automatic split")
    print(f"[result] max abs err {err:.3g}", flush=True)
    # four heads per work-group at an explicit 512-key split
    assert pa().decode_heads_per_block(wl.num_seqs, 8, wl.max_seq_len, 512) == 4
    err = assert_close(f64(gpu_cascade(wl, dw, split=512)), ref, "cascade split 512")
    print(f"[result] split 512: max abs err {err:.3g}", flush=True)


def test_mixed_batch_with_two_heads_per_work_group():
    wl0 = big_batch(503)
    lens = [int(x) for x in wl0.seq_lens]
    n_new = [1 if L > 0 else 0 for L in lens]
    rng = np.random.default_rng(504)
    for b in rng.choice(len(lens), 12, replace=False):
        if lens[b] >= 2:
            n_new[b] = int(min(lens[b], rng.integers(2, 100)))
    wl = W.make_custom(lens, 32, 8, 128, 16, dtype="bf16", kind="extend", n_new=n_new, seed=505)
    banner(f"mixed B={wl.num_seqs}: {sum(n > 1 for n in n_new)} chunks")
    assert pa().decode_heads_per_block(wl.num_seqs, 8, wl.max_seq_len) == 2
    dw = fresh(wl)
    out = pa().attend_mixed(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                            wl.max_seq_len, wl.scale)
    torch().cuda.synchronize()
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, "mixed automatic split")
    print(f"[result] max abs err {err:.3g}", flush=True)


@pytest.mark.parametrize("split", [256, 1024])
def test_same_bits_in_any_batch_at_an_explicit_split(split):
    """At an explicit split the heads per work-group do not depend on the
    batch: the same requests in a large batch (work order) and in a small one
    (grid order) give identical bits."""
    wl = big_batch(506)
    banner(f"batch invariance at split {split}")
    hb = pa().decode_heads_per_block(wl.num_seqs, 8, wl.max_seq_len, split)
    assert hb == (4 if split == 256 else 2)
    out = gpu_decode(wl, fresh(wl), split=split)
    seqs = list(range(0, wl.num_seqs, 11)) + [wl.num_seqs - 1]
    sub = wl.subset(seqs)
    assert pa().decode_heads_per_block(sub.num_seqs, 8, sub.max_seq_len, split) == hb
    out_sub = gpu_decode(sub, fresh(sub), split=split)
    assert bits(out_sub) == bits(out[seqs])

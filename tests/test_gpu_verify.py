"""Short-chunk extend (parallel verification of drafted tokens) against the
oracle's extend, which pins it (a verify chunk is an extend chunk; the
oracle's extend row i equals its decode at length p + i + 1)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, bits, f64, fresh, gpu_extend, pa, stored_oracle_pools, torch

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_verify(wl, dw, split=0, max_q_len=None):
    o = pa().verify(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens,
                    max_q_len or wl.max_q_len, wl.max_seq_len, wl.scale, split_tokens=split)
    torch().cuda.synchronize()
    return o


VERIFY_SWEEP = [
    # (prefixes, rows per request, Hq, Hkv, D, P, split)
    ([500, 3000, 0, 63, 64, 1000], [6, 6, 6, 6, 6, 6], 32, 8, 128, 16, 0),
    ([500, 3000, 0, 63, 64, 1000], [6, 6, 6, 6, 6, 6], 32, 8, 128, 16, 64),   # many pieces, masks in the last
    ([2000, 10], [8, 8], 32, 8, 128, 16, 1024),                                 # 8 x 4 = 32 rows
    ([700, 0, 129], [1, 3, 6], 32, 8, 128, 16, 128),                            # uneven chunks, one decode row
    ([900, 33], [4, 4], 64, 8, 128, 16, 0),                                     # group 8
    ([900, 33], [16, 2], 16, 8, 128, 1, 256),                                   # group 2, page 1
    ([300, 4100], [32, 5], 4, 4, 128, 64, 192),                                 # group 1, 32 rows
    ([1500, 70], [6, 6], 8, 2, 64, 16, 0),                                      # D = 64
    ([0, 0], [1, 2], 8, 2, 128, 16, 0),                                         # tiny contexts
    ([500, 3000, 0, 63], [4, 4, 4, 1], 14, 2, 64, 16, 0),                       # group 7: 4 x 7 = 28 rows
    ([900, 1200], [6, 6], 40, 8, 128, 16, 128),                                 # group 5: 30 rows
    ([77, 2100, 640], [6, 3, 6], 24, 8, 128, 16, 0),                            # group 3
    ([1500, 70], [5, 5], 12, 2, 128, 1, 256),                                   # group 6, page size 1
    ([800, 50, 3100], [6, 6, 2], 12, 3, 128, 16, 0),                            # odd KV heads: one per work-group
    ([400, 2000], [3, 4], 8, 1, 64, 16, 256),                                   # one KV head, group 8, D = 64
    ([1018, 2042, 58, 4090], [6, 6, 6, 6], 32, 8, 128, 16, 1024),              # lengths 1024, 2048, 64, 4096: no short last piece
    ([1018, 2042, 58, 4090], [6, 6, 6, 6], 32, 8, 128, 16, 64),                # the same in 64-key pieces
    ([2043, 6139, 3066, 100], [6, 6, 6, 6], 32, 8, 128, 16, 0),                # automatic 1536-key pieces: 2049, 6145 and 3072 keys
    ([5000, 300], [4, 4], 16, 8, 64, 1, 0),                                     # page size 1: 1536 page ids per piece
    ([5000, 300], [4, 4], 16, 8, 64, 1, 2048),                                  # page size 1, 2048-key pieces: 2048 page ids
]


@pytest.mark.parametrize("case", range(len(VERIFY_SWEEP)))
def test_verify_sweep(case):
    prefixes, n, Hq, Hkv, D, P, split = VERIFY_SWEEP[case]
    banner(f"verify sweep {case}: prefixes={prefixes} n={n} Hq={Hq} Hkv={Hkv} D={D} P={P} split={split}")
    lens = [p + k for p, k in zip(prefixes, n)]
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype="bf16", kind="extend", n_new=n, seed=700 + case)
    dw = fresh(wl)
    out = f64(gpu_verify(wl, dw, split))
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    assert_close(out, ref, f"verify sweep {case}")
    assert_close(out, f64(gpu_extend(wl, dw)), f"verify sweep {case} vs extend")


def test_verify_more_than_64_requests():
    """Batches of more than 64 requests take the plain piece order (piece
    index slowest, every request), not the longest-first one."""
    rng = np.random.default_rng(731)
    B = 70
    n = [int(x) for x in rng.integers(1, 7, B)]
    lens = [int(p) + k for p, k in zip(rng.integers(0, 2500, B), n)]
    banner(f"verify B={B} lengths<= {max(lens)}")
    for Hq, Hkv in ((32, 8), (12, 3)):
        wl = W.make_custom(lens, Hq, Hkv, 128, 16, dtype="bf16", kind="extend", n_new=n, seed=732 + Hkv)
        dw = fresh(wl)
        out = f64(gpu_verify(wl, dw, 512))
        kp, vp = stored_oracle_pools(wl)
        ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
        err = assert_close(out, ref, f"verify B={B} Hkv={Hkv}")
        print(f"[result] Hkv={Hkv} max abs err {err:.3g}", flush=True)


def test_verify_padding_requests_and_bound_above_the_chunks():
    """Requests with no rows (and no keys) are skipped; max_q_len may exceed
    every chunk."""
    banner("verify padding")
    wl = W.make_custom([600, 0, 80, 0], 32, 8, 128, 16, dtype="bf16", kind="extend", n_new=[6, 0, 3, 0], seed=720)
    dw = fresh(wl)
    out = f64(gpu_verify(wl, dw, 64, max_q_len=8))
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    assert_close(out, ref, "verify padding")


def test_verify_qwen3_8b_workload_whole_and_deterministic():
    """All 64 requests x 6 rows against the oracle; a second call gives the
    same bits."""
    banner("verify qwen3_8b_verify")
    wl = W.make("qwen3_8b_verify")
    dw = fresh(wl)
    first = gpu_verify(wl, dw)
    assert bits(gpu_verify(wl, dw)) == bits(first)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(first), ref, "qwen3_8b_verify")
    print(f"[result] verify: all {wl.num_seqs} requests checked, max abs err {err:.3g}", flush=True)

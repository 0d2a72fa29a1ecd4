"""Extend over many items: batches whose (token block, request, KV head)
items outnumber four chip-fulls of work-groups run on a fixed grid of
work-groups that each take their share of the items, with the requests that
have work ranked ahead of those that have none.  Checked element by element
against the oracle (Mini-SGLang README, yangyonggit fork, section Reference
Attention Backends: causal attention with the prefix-cache offset), through
pa_extend and through the mixed call, across the three ways the kernel
orders requests: ranked by key count (at most 64 with work), partitioned
only (more than 64 with work), and the plain request order (more than 256
requests)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, f64, fresh, gpu_extend, pa, stored_oracle_pools, torch

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def batch(num, active, max_new, seed):
    """num requests: `active` of them with 2..max_new new rows, one with the
    largest chunk, the rest single-row or empty; short cached prefixes."""
    rng = np.random.default_rng(seed)
    lens, n_new = [], []
    for b in range(num):
        if b % (num // active) == 0 and len([x for x in n_new if x > 1]) < active:
            n = int(rng.integers(2, max_new + 1)) if b else max_new
            lens.append(n + int(rng.integers(0, 90)))
        elif b % 17 == 5:
            n = 0
            lens.append(0)  # padding request: no rows, no keys
        else:
            n = 1
            lens.append(1 + int(rng.integers(0, 120)))
        n_new.append(n)
    return lens, n_new


CASES = [
    # (requests, requests with several rows, largest chunk, Hq, Hkv, D, P)
    (300, 20, 70, 32, 8, 128, 16),   # > 256 requests: request order
    (200, 80, 40, 32, 8, 128, 16),   # > 64 with work: partition only
    (240, 12, 150, 16, 2, 64, 8),    # ranked by key count
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_extend_many_items(case):
    num, active, max_new, Hq, Hkv, D, P = CASES[case]
    lens, n_new = batch(num, active, max_new, 900 + case)
    G = Hq // Hkv
    items = -(-max(n_new) // (128 // G)) * Hkv * num
    banner(f"extend items {case}: {num} requests, {sum(n > 1 for n in n_new)} with several rows, "
           f"{items} items, Hq={Hq} Hkv={Hkv} D={D} P={P}")
    assert items > 4 * 512, "the case must exceed four chip-fulls of work-groups"
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype="bf16", kind="extend", n_new=n_new, seed=910 + case)
    dw = fresh(wl)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    got = f64(gpu_extend(wl, dw))
    torch().cuda.synchronize()
    err = assert_close(got, ref, f"extend items {case}")
    mixed = f64(pa().attend_mixed(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens,
                                  wl.max_q_len, wl.max_seq_len, wl.scale))
    torch().cuda.synchronize()
    assert_close(mixed, ref, f"mixed items {case}")
    print(f"[result] {wl.q.shape[0]} rows checked, max abs err {err:.3g}", flush=True)

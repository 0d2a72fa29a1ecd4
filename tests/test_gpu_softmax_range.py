"""Scores over a wide range: the online softmax must keep its running
reference and rescale its accumulators correctly when scores grow by far
more than the slack the kernels allow before moving the reference, peak in
the middle of a request, or fall.  Queries are a constant vector and each
key row a constant times the all-ones row, so the score of key t is a chosen
function of t; values stay random.  Checked against the oracle (exact
softmax in float64; Mini-SGLang README, yangyonggit fork, section Reference
Attention Backends) through decode, extend, verify and the mixed call."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_close, f64, fresh, gpu_cascade, gpu_decode, gpu_extend, pa, stored_oracle_pools,
                         torch)

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
Q_VALUE = 0.125  # exact in bf16


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def shape_scores(wl, pattern, span):
    """Rewrite q and the key rows of wl in place so that key t of request b
    scores span * pattern(t / (L_b - 1)) in log2 units (score * scale * log2 e)
    for every query row and head."""
    D, P = wl.head_dim, wl.page_size
    sl2 = wl.scale * LOG2E
    wl.q[...] = W.f32_to_bf16_bits(np.full(wl.q.shape, Q_VALUE, np.float32))
    for b in range(wl.num_seqs):
        L, n = int(wl.seq_lens[b]), int(wl.n_new[b])
        if L == 0:
            continue
        for t in range(L):
            x = t / max(L - 1, 1)
            c = span * pattern(x) / sl2 / (Q_VALUE * D)  # score = Q_VALUE * D * c
            row = W.f32_to_bf16_bits(np.full((wl.num_kv_heads, D), c, np.float32))
            if t < L - n:
                page = int(wl.page_table[b, t // P])
                wl.k_pool[page, t % P] = row
            else:
                wl.k_new[int(wl.q_indptr[b]) + t - (L - n)] = row


PATTERNS = {
    "growing": lambda x: x,                          # the maximum moves at every tile
    "spike": lambda x: 1.0 if abs(x - 0.5) < 1e-3 else 0.0,
    "falling": lambda x: 1.0 - x,                    # the first keys dominate
}
PATTERN_NAMES = sorted(PATTERNS)


def check(got, wl, what):
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(got), ref, what)
    print(f"[result] {what}: max abs err {err:.3g}", flush=True)


@pytest.mark.parametrize("pattern", PATTERN_NAMES)
def test_extend_wide_scores(pattern):
    lens, n_new = [700, 1500, 90], [64, 130, 90]
    banner(f"extend {pattern}: lens={lens} n={n_new}")
    wl = W.make_custom(lens, 32, 8, 128, 16, dtype="bf16", kind="extend", n_new=n_new, seed=970)
    shape_scores(wl, PATTERNS[pattern], 60.0)
    dw = fresh(wl)
    check(gpu_extend(wl, dw), wl, f"extend {pattern}")


@pytest.mark.parametrize("pattern", PATTERN_NAMES)
def test_decode_wide_scores(pattern):
    lens = [700, 2900, 65, 1]
    banner(f"decode {pattern}: lens={lens}")
    wl = W.make_custom(lens, 16, 8, 128, 16, dtype="bf16", kind="decode", seed=971)
    shape_scores(wl, PATTERNS[pattern], 60.0)
    dw = fresh(wl)
    for split in (0, 64):
        check(gpu_decode(wl, dw, split=split), wl, f"decode {pattern} split {split}")


@pytest.mark.parametrize("pattern", PATTERN_NAMES)
def test_verify_and_mixed_wide_scores(pattern):
    lens, n_new = [900, 2100, 40, 300], [6, 6, 1, 6]
    banner(f"verify + mixed {pattern}: lens={lens} n={n_new}")
    wl = W.make_custom(lens, 32, 8, 128, 16, dtype="bf16", kind="extend", n_new=n_new, seed=972)
    shape_scores(wl, PATTERNS[pattern], 60.0)
    dw = fresh(wl)
    ver = pa().verify(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                      wl.max_seq_len, wl.scale)
    torch().cuda.synchronize()
    check(ver, wl, f"verify {pattern}")
    mix = pa().attend_mixed(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                            wl.max_seq_len, wl.scale)
    torch().cuda.synchronize()
    check(mix, wl, f"mixed {pattern}")


@pytest.mark.parametrize("pattern", PATTERN_NAMES)
def test_cascade_wide_scores(pattern):
    """Groups share their leading pages (each shared row keeps the value its
    last writer gave it, so scores still span the range); the shared-prefix
    pass and the requests' own keys see different references, which the
    combine reconciles."""
    lens = [700, 1200, 1500, 900, 1800, 2100, 513, 1025]
    banner(f"cascade {pattern}: lens={lens}")
    wl = W.make_custom(lens, 32, 8, 128, 16, dtype="bf16", radix=(4, 64), seed=973)
    shape_scores(wl, PATTERNS[pattern], 60.0)
    dw = fresh(wl)
    for split, pk in ((0, 0), (128, 192)):
        check(gpu_cascade(wl, dw, split=split, piece_keys=pk), wl, f"cascade {pattern} split {split} pieces {pk}")

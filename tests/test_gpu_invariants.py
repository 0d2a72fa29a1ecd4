"""GPU invariants: properties of the HIP path that hold exactly (bit for bit)
or within the parity tolerance, whatever the workload size."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, bits, f64, fresh, gpu_decode, gpu_extend, named, pa, stored_oracle_pools, torch

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("name", ["qwen25_05b", "qwen3_06b_p1", "qwen3_8b_radix"])
def test_decode_reruns_are_bit_identical(name):
    banner(f"rerun determinism {name}")
    wl, dw = named(name)
    a = bits(gpu_decode(wl, dw))
    for _ in range(3):
        assert bits(gpu_decode(wl, dw)) == a


def test_extend_reruns_are_bit_identical():
    banner("rerun determinism extend")
    wl, dw = named("qwen3_8b_extend")
    a = bits(gpu_extend(wl, dw))
    assert bits(gpu_extend(wl, dw)) == a


def _permuted(wl, seed):
    """Same logical content, every page moved to a new physical id."""
    perm = np.random.default_rng(seed).permutation(wl.num_pages)
    k2, v2 = np.empty_like(wl.k_pool), np.empty_like(wl.v_pool)
    k2[perm], v2[perm] = wl.k_pool, wl.v_pool
    pt2 = perm[wl.page_table].astype(np.int32)
    lists = [perm[pl].astype(np.int32) for pl in wl.page_lists]
    P = wl.page_size
    sm = wl.slot_mapping.copy()
    live = sm >= 0
    sm[live] = perm[sm[live] // P] * P + sm[live] % P
    return W.Workload(**{**wl.__dict__, "k_pool": k2, "v_pool": v2, "page_table": pt2, "page_lists": lists,
                         "slot_mapping": sm})


@pytest.mark.parametrize("kind", ["decode", "extend"])
def test_physical_page_permutation_is_bit_identical(kind):
    banner(f"page permutation {kind}")
    if kind == "decode":
        wl = W.make_custom([1, 17, 300, 1000, 2047], 32, 8, 128, 16, dtype="bf16", seed=31)
        run = gpu_decode
    else:
        wl = W.make_custom([70, 600, 129], 32, 8, 128, 16, dtype="bf16", kind="extend", n_new=[30, 256, 129],
                           seed=32)
        run = gpu_extend
    a = bits(run(wl, fresh(wl)))
    wl2 = _permuted(wl, 5)
    assert bits(run(wl2, fresh(wl2))) == a


def test_shared_prefix_equals_private_copies_bit_for_bit():
    banner("shared prefix vs private copies")
    wl = W.make_custom([700, 1200, 1500, 900, 1800, 2100, 513, 1025], 32, 8, 128, 16, dtype="bf16",
                       radix=(4, 64), seed=33)
    a = bits(gpu_decode(wl, fresh(wl)))
    # private copies: every request gets its own copy of each page it reads
    extra = sum(len(pl) for pl in wl.page_lists)
    k2 = np.concatenate([wl.k_pool, np.zeros((extra,) + wl.k_pool.shape[1:], wl.k_pool.dtype)])
    v2 = np.concatenate([wl.v_pool, np.zeros((extra,) + wl.v_pool.shape[1:], wl.v_pool.dtype)])
    pt2 = wl.page_table.copy()
    lists, nxt = [], wl.num_pages
    P = wl.page_size
    sm = wl.slot_mapping.copy()
    for b, pl in enumerate(wl.page_lists):
        new = []
        for j, page in enumerate(pl):
            k2[nxt], v2[nxt] = wl.k_pool[page], wl.v_pool[page]
            pt2[b, j] = nxt
            new.append(nxt)
            nxt += 1
        lists.append(np.array(new, np.int32))
        L = int(wl.seq_lens[b])
        sm[b] = new[(L - 1) // P] * P + (L - 1) % P
    wl2 = W.Workload(**{**wl.__dict__, "k_pool": k2, "v_pool": v2, "num_pages": nxt, "page_table": pt2,
                        "page_lists": lists, "slot_mapping": sm})
    assert bits(gpu_decode(wl2, fresh(wl2))) == a


@pytest.mark.parametrize("kind", ["decode", "extend"])
def test_garbage_in_unused_slots_changes_nothing(kind):
    banner(f"NaN vs zero garbage {kind}")
    outs = []
    for poison in ("nan", "zero"):
        if kind == "decode":
            wl = W.make_custom([1, 15, 17, 100, 333], 8, 2, 128, 16, dtype="bf16", poison=poison, seed=34)
            outs.append(bits(gpu_decode(wl, fresh(wl))))
        else:
            wl = W.make_custom([50, 200], 8, 2, 128, 16, dtype="bf16", kind="extend", n_new=[13, 77],
                               poison=poison, seed=35)
            outs.append(bits(gpu_extend(wl, fresh(wl))))
    assert outs[0] == outs[1]


@pytest.mark.parametrize("split", [64, 128, 320, 1024, 0])
def test_split_invariance(split):
    banner(f"split {split}")
    wl = W.make_custom([1, 63, 64, 65, 700, 2500, 5000], 32, 8, 128, 16, dtype="bf16", seed=36)
    dw = fresh(wl)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    got = f64(gpu_decode(wl, dw, split=split))
    assert_close(got, ref, f"split {split}")
    base = f64(gpu_decode(wl, dw, split=64))
    assert_close(got, base, f"split {split} vs split 64")


def test_extend_rows_equal_decode_at_their_length():
    banner("extend row i == decode at p+i+1")
    prefixes, chunks = [100, 0, 37], [40, 70, 129]
    lens = [p + n for p, n in zip(prefixes, chunks)]
    wl = W.make_custom(lens, 32, 8, 128, 16, dtype="bf16", kind="extend", n_new=chunks, seed=37)
    dw = fresh(wl)
    ext = f64(gpu_extend(wl, dw))
    T = torch()
    for b in range(wl.num_seqs):
        p = prefixes[b]
        rows = np.arange(wl.q_indptr[b], wl.q_indptr[b + 1])
        # every row of the chunk as its own decode request with length p+i+1
        q = dw.q[T.from_numpy(rows).cuda()].contiguous()
        pt = dw.page_table[b:b + 1].expand(len(rows), -1).contiguous()
        sl = T.tensor([p + i + 1 for i in range(len(rows))], dtype=T.int32, device="cuda")
        out = pa().decode(q, dw.k_pool, dw.v_pool, pt, sl, int(sl.max()), wl.scale)
        T.cuda.synchronize()
        assert_close(ext[rows], f64(out), f"extend vs decode request {b}")


def test_length_one_returns_the_v_row_exactly():
    banner("length one")
    for dtype in ("bf16", "f32"):
        wl = W.make_custom([1, 1, 1], 8, 2, 64, 16, dtype=dtype, seed=38)
        out = gpu_decode(wl, fresh(wl))
        expect = np.repeat(wl.v_new, 4, axis=1)  # [B, Hq, D] in storage format
        assert W.to_numpy_storage(out, dtype).tobytes() == np.ascontiguousarray(expect).tobytes()
    # extend: first token of a chunk with no prefix sees only itself
    wl = W.make_custom([9], 8, 2, 128, 16, dtype="bf16", kind="extend", n_new=[9], seed=39)
    out = W.to_numpy_storage(gpu_extend(wl, fresh(wl)), "bf16")
    assert out[0].tobytes() == np.ascontiguousarray(np.repeat(wl.v_new[0][None], 4, axis=1)[0]).tobytes()


def test_long_single_request_sampled():
    banner("one request of 65536 keys")
    wl = W.make_custom([65536], 32, 8, 128, 16, dtype="bf16", seed=40, poison=None)
    out = f64(gpu_decode(wl, fresh(wl)))
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    assert_close(out, ref, "65536-key decode")

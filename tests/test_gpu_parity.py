"""GPU parity: the HIP library against the CPU oracle on the same seeded
inputs.  Store and gather must be bit-exact; attention outputs must satisfy
|gpu - oracle| <= 1e-2 + 2e-2 |oracle| element by element (the oracle works in
float64 on the same bf16/fp32 inputs)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_close, f64, fresh, gpu_decode, gpu_extend, named, oracle_whole, pa,
                         stored_oracle_pools, torch)

pytestmark = pytest.mark.gpu

ALL = ["tiny", "qwen25_05b", "qwen3_06b_p1", "qwen3_8b_radix", "qwen3_8b_extend"]
DECODE = ["tiny", "qwen25_05b", "qwen3_06b_p1", "qwen3_8b_radix"]


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


# --------------------------------------------------------------------------
# store and gather: bit-exact over the whole pool
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ALL)
def test_store_is_bit_exact_over_whole_pool(name):
    banner(f"kv_store {name}")
    wl, dw = named(name)
    kp, vp = stored_oracle_pools(wl)
    gk = W.to_numpy_storage(dw.k_pool, wl.dtype)
    gv = W.to_numpy_storage(dw.v_pool, wl.dtype)
    assert gk.tobytes() == kp.tobytes()
    assert gv.tobytes() == vp.tobytes()


def test_store_skips_negative_slots_and_is_idempotent():
    banner("kv_store padding rows")
    wl = W.make_custom([5, 9, 16], 4, 2, 64, 4, dtype="bf16", seed=3)
    dw = W.to_device(wl)
    slots = dw.slot_mapping.clone()
    slots[1] = -1
    pa().kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, slots)
    pa().kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, slots)
    torch().cuda.synchronize()
    sm = wl.slot_mapping.copy()
    sm[1] = -1
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, sm)
    assert W.to_numpy_storage(dw.k_pool, wl.dtype).tobytes() == kp.tobytes()
    assert W.to_numpy_storage(dw.v_pool, wl.dtype).tobytes() == vp.tobytes()


@pytest.mark.parametrize("name", ALL)
def test_gather_is_bit_exact(name):
    banner(f"gather {name}")
    wl, dw = named(name)
    seqs = list(range(wl.num_seqs)) if wl.num_seqs <= 64 else list(range(0, wl.num_seqs, 8))
    kp, vp = stored_oracle_pools(wl)
    sub = wl.subset(seqs)
    T = torch()
    lens = sub.seq_lens.astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ko = T.empty((int(offs[-1]), wl.num_kv_heads, wl.head_dim), dtype=dw.k_pool.dtype, device="cuda")
    vo = T.empty_like(ko)
    pt = T.from_numpy(sub.page_table).cuda()
    sl = T.from_numpy(sub.seq_lens).cuda()
    pa().gather(dw.k_pool, dw.v_pool, pt, sl, T.from_numpy(offs).cuda(), sub.max_seq_len, ko, vo)
    T.cuda.synchronize()
    gk = W.to_numpy_storage(ko, wl.dtype)
    gv = W.to_numpy_storage(vo, wl.dtype)
    for i in range(sub.num_seqs):
        L = int(sub.seq_lens[i])
        assert gk[offs[i]:offs[i + 1]].tobytes() == oracle.gather(kp, sub.page_table[i], L).tobytes()
        assert gv[offs[i]:offs[i + 1]].tobytes() == oracle.gather(vp, sub.page_table[i], L).tobytes()


# --------------------------------------------------------------------------
# decode on the named configurations (the launch configuration of the bench)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", DECODE)
def test_decode_matches_oracle(name):
    """Every element of every request's output against the oracle."""
    banner(f"decode {name}")
    wl, dw = named(name)
    got = f64(gpu_decode(wl, dw))
    ref = oracle_whole(name)
    err = assert_close(got, ref, f"decode {name}")
    print(f"[result] decode {name}: all {wl.num_seqs} requests checked, max abs err {err:.3g}", flush=True)
    if wl.dtype == "f32":
        assert_close(got, ref, f"decode {name} (fp32 bound)", atol=1e-5, rtol=1e-5)


# --------------------------------------------------------------------------
# extend on the named configuration: every row against oracle.extend, and
# sampled rows against the oracle's decode at the row's own length (extend
# row i == decode at p+i+1 is pinned in the oracle tests)
# --------------------------------------------------------------------------
def test_extend_matches_oracle():
    name = "qwen3_8b_extend"
    banner(f"extend {name}")
    wl, dw = named(name)
    out = f64(gpu_extend(wl, dw))
    err = assert_close(out, oracle_whole(name), f"extend {name} (all rows)")
    kp, vp = stored_oracle_pools(wl)
    rng = np.random.default_rng(0)
    checked = 0
    for b in range(wl.num_seqs):
        n = int(wl.n_new[b])
        p = int(wl.seq_lens[b]) - n
        rows = sorted({0, 1, 31, 32, 63, 127, 128, n - 1} | set(rng.integers(0, n, 4).tolist()))
        for i in rows:
            r = int(wl.q_indptr[b]) + i
            ref = oracle.decode(wl.q[r][None], kp, vp, wl.page_table[b][None], np.array([p + i + 1]),
                                wl.scale, wl.dtype)[0]
            assert_close(out[r], ref, f"extend {name} req {b} row {i} (prefix {p})")
            checked += 1
    print(f"[result] extend {name}: all {out.shape[0]} rows (max abs err {err:.3g}) + {checked} rows vs decode",
          flush=True)


# --------------------------------------------------------------------------
# sweeps at sizes the oracle finishes quickly: several tiles and ragged tails
# --------------------------------------------------------------------------
DECODE_SWEEP = [
    # (lengths, Hq, Hkv, D, P, dtype, split)
    ([1, 15, 16, 17, 63, 64, 65, 200], 2, 1, 64, 16, "f32", 0),
    ([1, 100, 640, 333], 14, 2, 64, 16, "bf16", 0),
    ([1, 100, 640, 333], 14, 2, 64, 16, "bf16", 64),
    ([511, 512, 513, 1500, 2049], 16, 8, 128, 1, "bf16", 0),
    ([511, 512, 513, 1500, 2049], 16, 8, 128, 1, "bf16", 1024),
    ([3, 70, 130, 700], 4, 4, 128, 2, "bf16", 128),
    ([3, 70, 130, 700], 24, 8, 128, 32, "bf16", 0),     # group 3
    ([77, 300, 1025], 40, 8, 128, 16, "bf16", 192),     # group 5
    ([77, 300, 1025], 48, 8, 64, 8, "bf16", 0),         # group 6
    ([77, 300, 1025], 64, 8, 128, 256, "bf16", 0),      # group 8, largest page
    ([1, 33, 257], 8, 1, 64, 4, "f32", 64),             # fp32, group 8 x 64
    ([1, 33, 257], 4, 1, 128, 64, "f32", 0),            # fp32, group 4 x 128
    ([0, 5, 0, 40], 8, 2, 128, 16, "bf16", 0),          # empty requests
    ([4097], 32, 8, 128, 16, "bf16", 0),                # one long request
    ([1, 2047, 2048, 2049, 4097], 32, 8, 128, 16, "bf16", 2048),  # largest pieces
    ([300, 1500, 2100], 8, 8, 128, 16, "f32", 0),       # fp32, group 1 x 128 (octet reduction padded)
    ([65, 700, 1300], 6, 2, 64, 16, "f32", 128),        # fp32, group 3 x 64
    ([900, 1800, 40], 56, 8, 128, 16, "bf16", 0),       # group 7 x 128
]


@pytest.mark.parametrize("case", range(len(DECODE_SWEEP)))
def test_decode_sweep(case):
    lens, Hq, Hkv, D, P, dtype, split = DECODE_SWEEP[case]
    banner(f"decode sweep {case}: lens={lens} Hq={Hq} Hkv={Hkv} D={D} P={P} {dtype} split={split}")
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype=dtype, seed=100 + case)
    dw = fresh(wl)
    out = f64(gpu_decode(wl, dw, split=split))
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    assert_close(out, ref, f"decode sweep {case}")
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0)


EXTEND_SWEEP = [
    # (prefixes, chunks, Hq, Hkv, D, P)
    ([0, 1, 15, 100], [1, 5, 6, 31], 8, 2, 128, 16),
    ([0, 64, 17], [128, 129, 33], 32, 8, 128, 16),
    ([300, 0], [200, 64], 4, 4, 128, 1),
    ([64, 63], [100, 257], 16, 2, 128, 64),     # group 8
    ([10, 1000], [130, 40], 2, 1, 64, 16),      # group 2, D=64
    ([0, 5], [7, 300], 8, 8, 64, 32),           # group 1, D=64
    ([0], [1], 4, 1, 128, 16),                  # a single token
    # group sizes that do not divide the 128 rows of a work-group: the last
    # rows of every work-group are padding
    ([300, 0, 77], [200, 64, 19], 14, 2, 64, 16),    # group 7: the Qwen2.5-0.5B head shape
    ([1000, 17], [100, 300], 40, 8, 128, 16),        # group 5 (40/8)
    ([64, 500], [129, 37], 24, 8, 128, 16),          # group 3
    ([5, 2000], [250, 18], 12, 2, 128, 1),           # group 6, page size 1
    ([0], [1], 14, 2, 64, 16),                       # group 7, a single token
]


@pytest.mark.parametrize("case", range(len(EXTEND_SWEEP)))
def test_extend_sweep(case):
    prefixes, chunks, Hq, Hkv, D, P = EXTEND_SWEEP[case]
    banner(f"extend sweep {case}: prefixes={prefixes} chunks={chunks} Hq={Hq} Hkv={Hkv} D={D} P={P}")
    lens = [p + n for p, n in zip(prefixes, chunks)]
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype="bf16", kind="extend", n_new=chunks, seed=200 + case)
    dw = fresh(wl)
    out = f64(gpu_extend(wl, dw))
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    assert_close(out, ref, f"extend sweep {case}")


EXTEND_SPLIT = [
    # (prefixes, chunks, Hq, Hkv, D, P, split): keys cut into pieces merged by
    # the combine kernel; rows of the first pieces see every key of a piece,
    # the last piece of a block is causal
    ([0, 64, 1000], [128, 129, 33], 32, 8, 128, 16, 64),
    ([3000, 17], [100, 300], 32, 8, 128, 16, 192),
    ([300, 0, 77], [200, 64, 19], 14, 2, 64, 16, 128),        # group 7
    ([5000, 0, 900], [40, 0, 1], 8, 2, 128, 1, 1024),        # an empty request, a one-row chunk, page size 1
    ([20000], [300], 32, 8, 128, 16, 0),                      # automatic: one long-prefix request is split
    ([4000, 6000], [64, 512], 40, 8, 128, 16, 0),             # automatic, group 5
]


@pytest.mark.parametrize("case", range(len(EXTEND_SPLIT)))
def test_extend_split_keys(case):
    prefixes, chunks, Hq, Hkv, D, P, split = EXTEND_SPLIT[case]
    lens = [p + n for p, n in zip(prefixes, chunks)]
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype="bf16", kind="extend", n_new=chunks, seed=260 + case)
    nbytes = pa().extend_workspace_bytes(wl.num_seqs, wl.max_q_len, Hq, Hkv, D, wl.max_seq_len, split)
    banner(f"extend split {case}: prefixes={prefixes} chunks={chunks} Hq={Hq} Hkv={Hkv} D={D} P={P} "
           f"split={split} workspace={nbytes}")
    assert nbytes > 0, "this case is meant to split the keys"
    dw = fresh(wl)
    T = torch()
    o1 = pa().extend(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                     wl.max_seq_len, wl.scale, split_tokens=split)
    o2 = pa().extend(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                     wl.max_seq_len, wl.scale, split_tokens=split)
    T.cuda.synchronize()
    assert T.equal(o1.view(T.int16), o2.view(T.int16)), "split extend is not deterministic"
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(o1), ref, f"extend split {case}")
    # the unsplit kernel on the same inputs
    whole = pa().extend(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                        wl.max_seq_len, wl.scale, split_tokens=(wl.max_seq_len + 63) // 64 * 64)
    T.cuda.synchronize()
    assert_close(f64(o1), f64(whole), f"extend split {case} vs unsplit")
    print(f"[result] extend split {case}: max abs err {err:.3g}", flush=True)


def test_empty_batch_is_a_no_op():
    banner("empty batch")
    T = torch()
    k = T.zeros(4, 16, 1, 64, dtype=T.bfloat16, device="cuda")
    q = T.zeros(0, 2, 64, dtype=T.bfloat16, device="cuda")
    pt = T.zeros(0, 4, dtype=T.int32, device="cuda")
    sl = T.zeros(0, dtype=T.int32, device="cuda")
    out = pa().decode(q, k, k, pt, sl, 64, 0.125)
    pa().kv_store(k, k, q[:, :1], q[:, :1], T.zeros(0, dtype=T.int64, device="cuda"))
    qi = T.zeros(1, dtype=T.int32, device="cuda")
    out2 = pa().extend(q, qi, k, k, pt, sl, 0, 64, 0.125)
    T.cuda.synchronize()
    assert out.numel() == 0 and out2.numel() == 0

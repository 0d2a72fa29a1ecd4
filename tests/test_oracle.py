"""Pins for the CPU oracle.

Every check here gets its expected value from somewhere other than the oracle:
hand-worked examples (tests/golden), brute force in plain Python loops with
the KV heads expanded the way repeat_interleave does, torch's
scaled_dot_product_attention in float64 (the library routine the nanoSGLang
README, section Notable Fixes, falls back to), closed forms, and invariants of
the paging.  The mutation tests at the end plant plausible mistakes in the
oracle and check that at least one pin catches each.
"""
import json
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_attention as O
import workloads as W

GOLDEN = Path(__file__).parent / "golden"


# --------------------------------------------------------------------------
# helpers (independent of the oracle's own code)
# --------------------------------------------------------------------------
def _num(s):
    if isinstance(s, (int, float)):
        return float(s)
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    return float(Fraction(s))


def _arr(nested, dtype=np.float32):
    if isinstance(nested, list):
        return np.array([_arr(x, dtype) for x in nested], dtype=dtype)
    return dtype(_num(nested))


def _lib_widen(x, dtype):
    """Storage format -> float64 through torch's own bf16 type."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return np.asarray(x, np.float32).astype(np.float64)


def _to_storage(x32, dtype):
    return W.f32_to_bf16_bits(x32) if dtype == "bf16" else np.asarray(x32, np.float32)


def paginate(Ks, Vs, P, rng, dtype, extra_pages=3):
    """Lay out contiguous per-request rows [L_b, Hkv, D] as a paged pool:
    each request's rows are padded to whole pages (with NaN), cut into pages
    by a reshape, and placed at randomly permuted physical pages."""
    Hkv, D = Ks[0].shape[1], Ks[0].shape[2]
    npg = [max(1, -(-len(k) // P)) for k in Ks]
    num_pages = sum(npg) + extra_pages
    perm = rng.permutation(num_pages)
    nan = W.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    sd = np.uint16 if dtype == "bf16" else np.float32
    k_pool = np.full((num_pages, P, Hkv, D), nan, sd)
    v_pool = np.full((num_pages, P, Hkv, D), nan, sd)
    pt = np.zeros((len(Ks), max(npg)), np.int32)
    pos = 0
    for b, (k, v) in enumerate(zip(Ks, Vs)):
        pages = perm[pos:pos + npg[b]]
        pos += npg[b]
        for src, pool in ((k, k_pool), (v, v_pool)):
            pad = np.full((npg[b] * P, Hkv, D), nan, sd)
            pad[:len(src)] = src
            pool[pages] = pad.reshape(npg[b], P, Hkv, D)
        pt[b, :npg[b]] = pages
    return k_pool, v_pool, pt, np.array([len(k) for k in Ks], np.int32)


def brute_attend(qrow, K, V, scale, G):
    """Pure-Python float64 attention of one query row over rows K, V given as
    nested lists [L][Hkv][D]; the KV heads are expanded by repeating each one
    G times in place (repeat_interleave), then query head h uses expanded head
    h.  Returns [Hq][D]."""
    Hq = len(qrow)
    Kx = [[head for head in row for _ in range(G)] for row in K]
    Vx = [[head for head in row for _ in range(G)] for row in V]
    L = len(K)
    out = []
    for h in range(Hq):
        D = len(qrow[h])
        if L == 0:
            out.append([0.0] * D)
            continue
        sc = [scale * sum(qrow[h][d] * Kx[t][h][d] for d in range(D)) for t in range(L)]
        m = max(sc)
        e = [math.exp(s - m) for s in sc]
        z = sum(e)
        out.append([sum(e[t] * Vx[t][h][d] for t in range(L)) / z for d in range(D)])
    return out


def make_tiny_case(rng, B, Ls, Hq, Hkv, D, P, dtype):
    Ks = [_to_storage(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype) for L in Ls]
    Vs = [_to_storage(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype) for L in Ls]
    q = _to_storage(rng.standard_normal((B, Hq, D)).astype(np.float32), dtype)
    k_pool, v_pool, pt, sl = paginate(Ks, Vs, P, rng, dtype)
    return Ks, Vs, q, k_pool, v_pool, pt, sl


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------
BRUTE_CASES = [
    # (D, Hq, Hkv, P, dtype, lengths)
    (4, 1, 1, 1, "f32", [1, 5, 9]),
    (8, 2, 1, 2, "bf16", [3, 16, 17, 1]),
    (8, 4, 2, 16, "f32", [15, 16, 33, 64]),
    (4, 7, 1, 16, "bf16", [1, 17, 40]),
    (64, 4, 2, 2, "bf16", [7, 30]),
    (64, 2, 1, 16, "f32", [1, 17, 33, 64]),
]


# Agreement with the float64 brute force: float64 arithmetic to rounding;
# float32 arithmetic (a few dozen keys, dot products of at most 64 terms) to
# a few float32 ulps of the operands.
TOL = {"f64": dict(rtol=1e-10, atol=1e-12), "f32": dict(rtol=2e-5, atol=2e-6)}


@pytest.mark.parametrize("acc", ["f64", "f32"])
@pytest.mark.parametrize("D,Hq,Hkv,P,dtype,Ls", BRUTE_CASES)
def test_decode_brute_force(D, Hq, Hkv, P, dtype, Ls, acc):
    rng = np.random.default_rng(D * 1000 + Hq * 100 + P)
    Ks, Vs, q, k_pool, v_pool, pt, sl = make_tiny_case(rng, len(Ls), Ls, Hq, Hkv, D, P, dtype)
    scale = float(np.float32(1 / math.sqrt(D)))
    got = oracle.decode(q, k_pool, v_pool, pt, sl, scale, dtype, acc=acc)
    G = Hq // Hkv
    for b in range(len(Ls)):
        ref = brute_attend(_lib_widen(q[b], dtype).tolist(), _lib_widen(Ks[b], dtype).tolist(),
                           _lib_widen(Vs[b], dtype).tolist(), scale, G)
        np.testing.assert_allclose(got[b], np.array(ref), **TOL[acc])


@pytest.mark.parametrize("acc", ["f64", "f32"])
@pytest.mark.parametrize("D,Hq,Hkv,P,dtype", [(4, 2, 1, 2, "f32"), (8, 4, 2, 16, "bf16"), (8, 7, 1, 1, "f32")])
def test_extend_brute_force(D, Hq, Hkv, P, dtype, acc):
    rng = np.random.default_rng(7 + D + Hq)
    Ls = [5, 20, 3]
    ns = [2, 20, 3]  # prefixes 3, 0, 0
    Ks, Vs, _, k_pool, v_pool, pt, sl = make_tiny_case(rng, len(Ls), Ls, Hq, Hkv, D, P, dtype)
    T = sum(ns)
    q = _to_storage(rng.standard_normal((T, Hq, D)).astype(np.float32), dtype)
    qi = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    scale = float(np.float32(1 / math.sqrt(D)))
    got = oracle.extend(q, qi, k_pool, v_pool, pt, sl, scale, dtype, acc=acc)
    G = Hq // Hkv
    for b in range(len(Ls)):
        p = Ls[b] - ns[b]
        K, V = _lib_widen(Ks[b], dtype).tolist(), _lib_widen(Vs[b], dtype).tolist()
        for i in range(ns[b]):
            pos = p + i  # this token's own position; it sees keys up to and including it
            ref = brute_attend(_lib_widen(q[qi[b] + i], dtype).tolist(), K[:pos + 1], V[:pos + 1], scale, G)
            np.testing.assert_allclose(got[qi[b] + i], np.array(ref), **TOL[acc])


# --------------------------------------------------------------------------
# library routine: scaled_dot_product_attention in float64
# --------------------------------------------------------------------------
@pytest.mark.parametrize("acc", ["f64", "f32"])
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 2, 16), (14, 2, 64), (8, 8, 32)])
def test_decode_matches_sdpa(Hq, Hkv, D, acc):
    """One page per request (page_size = longest length) and an identity page
    table reduce paged decode to dense GQA attention."""
    rng = np.random.default_rng(11)
    Ls = [1, 9, 40, 23]
    Lmax = max(Ls)
    B = len(Ls)
    kp = rng.standard_normal((B, Lmax, Hkv, D)).astype(np.float32)
    vp = rng.standard_normal((B, Lmax, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    pt = np.arange(B, dtype=np.int32)[:, None]
    scale = 0.3
    got = oracle.decode(q, kp, vp, pt, np.array(Ls), scale, "f32", acc=acc)
    F = torch.nn.functional
    tol = dict(rtol=1e-12, atol=1e-13) if acc == "f64" else dict(rtol=2e-5, atol=2e-6)
    for b, L in enumerate(Ls):
        qt = torch.from_numpy(q[b]).double()[None, :, None, :]  # [1, Hq, 1, D]
        kt = torch.from_numpy(kp[b, :L]).double().permute(1, 0, 2)[None]  # [1, Hkv, L, D]
        vt = torch.from_numpy(vp[b, :L]).double().permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)[0, :, 0, :]
        np.testing.assert_allclose(got[b], ref.numpy(), **tol)


@pytest.mark.parametrize("prefix", [0, 1, 13, 32])
def test_extend_matches_sdpa(prefix):
    rng = np.random.default_rng(100 + prefix)
    Hq, Hkv, D, n = 4, 2, 16, 9
    L = prefix + n
    kp = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    vp = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((n, Hq, D)).astype(np.float32)
    got = oracle.extend(q, np.array([0, n]), kp, vp, np.zeros((1, 1), np.int32), np.array([L]), 0.25, "f32")
    F = torch.nn.functional
    qt = torch.from_numpy(q).double().permute(1, 0, 2)[None]  # [1, Hq, n, D]
    kt = torch.from_numpy(kp[0]).double().permute(1, 0, 2)[None]
    vt = torch.from_numpy(vp[0]).double().permute(1, 0, 2)[None]
    if prefix == 0:
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.25, is_causal=True, enable_gqa=True)
    else:  # bottom-right aligned causal mask
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=prefix)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.25, enable_gqa=True)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------
def _load(name):
    return json.loads((GOLDEN / name).read_text())


def test_golden_decode_gqa():
    g = _load("decode_gqa_hand.json")
    got = oracle.decode(_arr(g["q"]), _arr(g["k_pool"]), _arr(g["v_pool"]), np.array(g["page_table"]),
                        np.array(g["seq_lens"]), g["scale"], g["dtype"])
    np.testing.assert_allclose(got, _arr(g["expected"], np.float64), rtol=g["rtol"])


def test_golden_extend_causal_offset():
    g = _load("extend_causal_hand.json")
    got = oracle.extend(_arr(g["q"]), np.array(g["q_indptr"]), _arr(g["k_pool"]), _arr(g["v_pool"]),
                        np.array(g["page_table"]), np.array(g["seq_lens"]), g["scale"], g["dtype"])
    np.testing.assert_allclose(got, _arr(g["expected"], np.float64), rtol=g["rtol"])


def test_golden_store_and_addressing():
    g = _load("store_addressing_hand.json")
    P, npg = g["page_size"], g["num_pages"]
    pool = _arr(g["pool_before_flat"]).reshape(npg, P, 1, 1)
    rows = _arr(g["rows"]).reshape(-1, 1, 1)
    k2, v2 = oracle.kv_store(pool, pool.copy(), rows, rows, np.array(g["slot_mapping"]))
    assert oracle.token_slots(g["page_table"][0], g["seq_len"], P) == g["expected_slots"]
    np.testing.assert_array_equal(k2.reshape(-1), _arr(g["expected_pool_flat"]))
    np.testing.assert_array_equal(v2.reshape(-1), _arr(g["expected_pool_flat"]))
    got = oracle.gather(k2, g["page_table"][0], g["seq_len"]).reshape(-1)
    np.testing.assert_array_equal(got, _arr(g["expected_gather"]))


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("acc", ["f64", "f32"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_length_one_returns_v_row_exactly(dtype, acc):
    rng = np.random.default_rng(3)
    Ks, Vs, q, k_pool, v_pool, pt, sl = make_tiny_case(rng, 3, [1, 1, 1], 4, 2, 8, 4, dtype)
    got = oracle.decode(q, k_pool, v_pool, pt, sl, 0.35, dtype, acc=acc)
    for b in range(3):
        expect = np.repeat(_lib_widen(Vs[b][0], dtype), 2, axis=0)  # [Hq, D]
        np.testing.assert_array_equal(got[b], expect)


def test_zero_query_gives_mean_of_v():
    rng = np.random.default_rng(4)
    Ks, Vs, q, k_pool, v_pool, pt, sl = make_tiny_case(rng, 2, [7, 50], 2, 1, 8, 16, "f32")
    q[:] = 0
    got = oracle.decode(q, k_pool, v_pool, pt, sl, 1.0, "f32")
    for b in range(2):
        mean = Vs[b].astype(np.float64).mean(axis=0)  # [Hkv, D]
        np.testing.assert_allclose(got[b], np.repeat(mean, 2, axis=0), rtol=1e-13, atol=1e-14)


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(5)
    Ks, Vs, q, k_pool, v_pool, pt, sl = make_tiny_case(rng, 1, [33], 4, 4, 8, 2, "f32")
    same = Ks[0][:1].repeat(33, axis=0)
    k_pool2, v_pool2, pt2, sl2 = paginate([same], Vs, 2, np.random.default_rng(0), "f32")
    got = oracle.decode(q, k_pool2, v_pool2, pt2, sl2, 0.7, "f32")
    np.testing.assert_allclose(got[0], Vs[0].astype(np.float64).mean(axis=0), rtol=1e-13, atol=1e-14)


def test_float32_arithmetic_agrees_with_float64_on_named_workloads():
    """The two precisions of the oracle on real workload shapes (hundreds of
    keys, D = 64 and 128): float32 accumulation stays within 1e-5 of float64,
    a thousand times inside the GPU tolerance."""
    for name in ("qwen25_05b", "qwen3_06b_p1"):
        wl = W.make(name, poison="nan")
        kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
        sub = list(range(0, wl.num_seqs, max(1, wl.num_seqs // 6)))
        args = (wl.q[sub], kp, vp, wl.page_table[sub], wl.seq_lens[sub], wl.scale, wl.dtype)
        np.testing.assert_allclose(oracle.decode(*args, acc="f32"), oracle.decode(*args), rtol=1e-5, atol=1e-5)
    wl = W.make_custom([300, 70], 8, 2, 128, 16, dtype="bf16", kind="extend", n_new=[100, 70], seed=21)
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    args = (wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    np.testing.assert_allclose(oracle.extend(*args, acc="f32"), oracle.extend(*args), rtol=1e-5, atol=1e-5)
    with pytest.raises(ValueError):
        oracle.decode(*args[:1], kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype, acc="f16")


def test_empty_sequence_gives_zero_row():
    rng = np.random.default_rng(6)
    Ks, Vs, q, k_pool, v_pool, pt, sl = make_tiny_case(rng, 2, [0, 5], 2, 1, 4, 2, "f32")
    got = oracle.decode(q, k_pool, v_pool, pt, sl, 1.0, "f32")
    assert np.all(got[0] == 0) and np.all(np.isfinite(got[1]))


# --------------------------------------------------------------------------
# invariants of the paging
# --------------------------------------------------------------------------
def _permute_pages(wl, rng):
    """Move every page to a new physical id and rewrite the page table."""
    perm = rng.permutation(wl.num_pages)  # old id -> new id
    k2 = np.empty_like(wl.k_pool)
    v2 = np.empty_like(wl.v_pool)
    k2[perm] = wl.k_pool
    v2[perm] = wl.v_pool
    return k2, v2, perm[wl.page_table].astype(np.int32)


@pytest.mark.parametrize("name", ["tiny", "qwen25_05b"])
def test_physical_page_permutation_is_bit_identical(name):
    wl = W.make(name, poison="nan")
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    sub = list(range(min(6, wl.num_seqs)))
    ref = oracle.decode(wl.q[sub], kp, vp, wl.page_table[sub], wl.seq_lens[sub], wl.scale, wl.dtype)
    perm = np.random.default_rng(9).permutation(wl.num_pages)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    got = oracle.decode(wl.q[sub], kp2, vp2, perm[wl.page_table[sub]], wl.seq_lens[sub], wl.scale, wl.dtype)
    np.testing.assert_array_equal(got, ref)


def test_shared_prefix_equals_private_copies():
    wl = W.make_custom([40, 70, 33, 90], 4, 2, 16, 4, dtype="bf16", radix=(4, 8), seed=3)
    # requests 0..3 share up to 8 prefix pages
    assert len(set(map(tuple, [pl[:5] for pl in wl.page_lists]))) == 1
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    # give every request private copies of its shared pages
    extra = sum(len(pl) for pl in wl.page_lists)
    kp2 = np.concatenate([kp, np.zeros((extra,) + kp.shape[1:], kp.dtype)])
    vp2 = np.concatenate([vp, np.zeros((extra,) + vp.shape[1:], vp.dtype)])
    pt2 = wl.page_table.copy()
    nxt = wl.num_pages
    for b, pl in enumerate(wl.page_lists):
        for j, page in enumerate(pl):
            kp2[nxt], vp2[nxt] = kp[page], vp[page]
            pt2[b, j] = nxt
            nxt += 1
    got = oracle.decode(wl.q, kp2, vp2, pt2, wl.seq_lens, wl.scale, wl.dtype)
    np.testing.assert_array_equal(got, ref)


def test_garbage_in_unused_slots_does_not_matter():
    a = W.make("qwen25_05b", poison="nan")
    z = W.make("qwen25_05b", poison="zero")
    outs = []
    for wl in (a, z):
        kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
        outs.append(oracle.decode(wl.q[:4], kp, vp, wl.page_table[:4], wl.seq_lens[:4], wl.scale, wl.dtype))
    assert np.all(np.isfinite(outs[0]))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_extend_row_equals_decode_at_that_length():
    wl = W.make_custom([21, 40], 4, 2, 32, 16, dtype="bf16", kind="extend", n_new=[6, 40], seed=8)
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    ext = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    for b in range(2):
        p = int(wl.seq_lens[b] - wl.n_new[b])
        for i in range(int(wl.n_new[b])):
            row = wl.q_indptr[b] + i
            dec = oracle.decode(wl.q[row][None], kp, vp, wl.page_table[b][None], np.array([p + i + 1]),
                                wl.scale, wl.dtype)
            np.testing.assert_allclose(ext[row], dec[0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("split", [1, 7, 16, 64, 1000])
def test_split_and_combine_equals_decode(split):
    wl = W.make_custom([1, 17, 100, 64, 0], 6, 2, 16, 16, dtype="bf16", seed=12)
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    o, lse, ns = oracle.decode_partials(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype, split)
    np.testing.assert_array_equal(ns, [-(-int(L) // split) for L in wl.seq_lens])
    np.testing.assert_allclose(oracle.combine(o, lse, ns), ref, rtol=1e-12, atol=1e-14)


def test_store_then_gather_round_trip():
    wl = W.make("tiny", poison="nan")
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        gk = oracle.gather(kp, wl.page_table[b], L)
        gv = oracle.gather(vp, wl.page_table[b], L)
        assert gk[-1].tobytes() == wl.k_new[b].tobytes()
        assert gv[-1].tobytes() == wl.v_new[b].tobytes()
        assert np.all(np.isfinite(gk)) and np.all(np.isfinite(gv))
    # every slot other than the stored ones is byte-identical to before
    flat_b = wl.k_pool.reshape(-1, 1, 64)
    flat_a = kp.reshape(-1, 1, 64)
    other = np.setdiff1d(np.arange(flat_b.shape[0]), wl.slot_mapping)
    assert flat_a[other].tobytes() == flat_b[other].tobytes()


def test_store_rejects_duplicates_and_skips_padding():
    pool = np.zeros((2, 2, 1, 1), np.float32)
    rows = np.ones((2, 1, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.kv_store(pool, pool, rows, rows, np.array([1, 1]))
    k2, _ = oracle.kv_store(pool, pool, rows, rows, np.array([-1, 3]))
    assert k2.reshape(-1).tolist() == [0, 0, 0, 1]


# --------------------------------------------------------------------------
# planted mistakes: each must trip at least one pin
# --------------------------------------------------------------------------
def _run_pins():
    """Run a fixed set of pins; return the names of those that fail."""
    pins = {
        "brute_decode_gqa": lambda: test_decode_brute_force(8, 4, 2, 16, "f32", [15, 16, 33, 64], "f64"),
        "brute_decode_bf16": lambda: test_decode_brute_force(8, 2, 1, 2, "bf16", [3, 16, 17, 1], "f64"),
        "brute_decode_f32_acc": lambda: test_decode_brute_force(8, 4, 2, 16, "bf16", [15, 16, 33, 64], "f32"),
        "brute_extend": lambda: test_extend_brute_force(4, 2, 1, 2, "f32", "f64"),
        "brute_extend_f32_acc": lambda: test_extend_brute_force(8, 4, 2, 16, "bf16", "f32"),
        "sdpa_decode": lambda: test_decode_matches_sdpa(4, 2, 16, "f64"),
        "sdpa_extend": lambda: test_extend_matches_sdpa(13),
        "golden_decode": test_golden_decode_gqa,
        "golden_extend": test_golden_extend_causal_offset,
        "golden_store": test_golden_store_and_addressing,
        "length_one": lambda: test_length_one_returns_v_row_exactly("bf16", "f64"),
        "zero_query": test_zero_query_gives_mean_of_v,
    }
    failed = []
    for name, fn in pins.items():
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_all_pins():
    assert _run_pins() == []


_orig_widen = O.widen

MUTATIONS = {
    "gqa_interleaved": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "causal_off_by_one": ("visible", lambda i, j, p: j < p + i),
    "causal_ignores_prefix": ("visible", lambda i, j, p: j <= i),
    "reversed_offset_in_page": (
        "token_slots",
        lambda row, L, P: [int(row[t // P]) * P + (P - 1 - t % P) for t in range(L)]),
    "page_index_off_by_one": (
        "token_slots",
        lambda row, L, P: [int(row[min(t // P + (t % P == P - 1), len(row) - 1)]) * P + t % P
                           for t in range(L)]),
    "bf16_widen_wrong_shift": (
        "widen",
        lambda x, dt: (((np.asarray(x, np.uint16).astype(np.uint32) << 15).view(np.float32)).astype(np.float64)
                       if dt == "bf16" else _orig_widen(x, dt))),
    "normalise_by_count": (
        "_softmax_rows_attend",
        lambda s, V: (np.exp(s - np.max(s, -1, keepdims=True)) @ V) / s.shape[-1]),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(O, attr, fn)
    failed = _run_pins()
    assert failed, f"no pin caught the planted mistake {mutation!r}"

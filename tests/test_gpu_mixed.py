"""Mixed prefill + decode batches, and a whole step captured into a HIP graph
with fixed buffers and replayed with other contents (the fixed-buffer
contract of "mini-sglang from Scratch"; continuous batching with mixed
prefill and decode, nanoSGLang README, section Features)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, bits, f64, fresh, gpu_extend, pa, stored_oracle_pools, torch

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


MIXED = [
    # (lengths, new rows per request, Hq, Hkv, D, P)
    ([600, 1500, 40, 3000, 1, 77, 2049, 700], [1, 1, 40, 1, 1, 6, 1, 129], 32, 8, 128, 16),
    ([5000, 300, 300, 9], [1, 300, 6, 1], 16, 2, 128, 1),
    ([64, 65, 0, 130, 0], [1, 65, 0, 1, 0], 8, 8, 64, 32),  # padding requests (no rows, no keys)
    ([1, 2, 3], [1, 1, 1], 8, 1, 128, 16),                    # decode only
    ([100, 200], [100, 7], 4, 2, 64, 16),                     # extend only
    ([600, 140, 40, 3000, 1, 77], [1, 1, 40, 1, 1, 6], 14, 2, 64, 16),  # group 7 (Qwen2.5-0.5B heads)
    ([1000, 300, 2000, 9], [1, 300, 1, 9], 40, 8, 128, 16),             # group 5
]


@pytest.mark.parametrize("case", range(len(MIXED)))
def test_mixed_batch_matches_oracle(case):
    lens, n_new, Hq, Hkv, D, P = MIXED[case]
    banner(f"mixed {case}: lens={lens} n={n_new} Hq={Hq} Hkv={Hkv} D={D} P={P}")
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype="bf16", kind="extend", n_new=n_new, seed=500 + case)
    dw = fresh(wl)
    out = pa().attend_mixed(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_q_len,
                            wl.max_seq_len, wl.scale)
    torch().cuda.synchronize()
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    got = f64(out)
    assert_close(got, ref, f"mixed {case}")
    assert_close(got, f64(gpu_extend(wl, dw)), f"mixed {case} vs extend")


def test_mixed_qwen3_8b_batch_whole():
    """248 decode requests of the Qwen3-8B decode shape next to 8 prefill
    chunks of 512 rows: every row against the oracle."""
    banner("mixed qwen3_8b_mixed whole")
    wl = W.make("qwen3_8b_mixed")
    dw = fresh(wl)
    out = f64(pa().attend_mixed(dw.q, dw.q_indptr, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens,
                                wl.max_q_len, wl.max_seq_len, wl.scale))
    torch().cuda.synchronize()
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.extend(wl.q, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(out, ref, "qwen3_8b_mixed")
    print(f"[result] mixed: all {wl.num_seqs} requests ({out.shape[0]} rows) checked, max abs err {err:.3g}",
          flush=True)


# --------------------------------------------------------------------------
# a whole step (rope + store, then attention) captured once, replayed with
# three different batches copied into the same fixed buffers
# --------------------------------------------------------------------------
B_CAP, T_CAP, L_CAP, Q_CAP, NPAGES = 12, 160, 1024, 128, 400
Hq, Hkv, D, P = 16, 4, 128, 16
STRIDE = L_CAP // P

BATCHES = [
    ([300, 1000, 64, 5], [1, 128, 1, 5]),
    ([1, 2, 900, 901, 17, 400, 1024, 33], [1, 1, 1, 100, 1, 1, 1, 33]),
    ([128, 256], [128, 1]),
]


def _batch(case):
    lens, n_new = BATCHES[case]
    return W.make_custom(lens, Hq, Hkv, D, P, dtype="bf16", kind="extend", n_new=n_new, num_pages=NPAGES,
                         stride=STRIDE, seed=600 + case, poison="zero")


def _fill(static, wl, cos_t):
    """Copy one batch into the fixed buffers; the rest is padding: requests
    with no rows and no keys, rows with slot -1."""
    T = torch()
    B, N = wl.num_seqs, int(wl.q_indptr[-1])
    assert B <= B_CAP and N <= T_CAP and wl.max_seq_len <= L_CAP and wl.max_q_len <= Q_CAP
    dev = lambda x: T.from_numpy(np.ascontiguousarray(x)).cuda()
    bf = lambda x: T.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(T.bfloat16).cuda()
    static["k_pool"].copy_(bf(wl.k_pool))
    static["v_pool"].copy_(bf(wl.v_pool))
    q = np.zeros((T_CAP, Hq, D), np.uint16); q[:N] = wl.q
    kn = np.zeros((T_CAP, Hkv, D), np.uint16); kn[:N] = wl.k_new
    vn = np.zeros((T_CAP, Hkv, D), np.uint16); vn[:N] = wl.v_new
    slots = np.full(T_CAP, -1, np.int64); slots[:N] = wl.slot_mapping
    pos = np.zeros(T_CAP, np.int32); pos[:N] = wl.positions()
    qi = np.full(B_CAP + 1, N, np.int32); qi[:B + 1] = wl.q_indptr
    pt = np.zeros((B_CAP, STRIDE), np.int32); pt[:B] = wl.page_table
    sl = np.zeros(B_CAP, np.int32); sl[:B] = wl.seq_lens
    for k, v in (("q", bf(q)), ("k_new", bf(kn)), ("v_new", bf(vn)), ("slots", dev(slots)), ("pos", dev(pos)),
                 ("q_indptr", dev(qi)), ("page_table", dev(pt)), ("seq_lens", dev(sl))):
        static[k].copy_(v)
    static["out"].copy_(T.zeros_like(static["out"]))


def _step(s, cos_d, sin_d, scale):
    pa().rope_kv_store(s["k_pool"], s["v_pool"], s["q"], s["k_new"], s["v_new"], s["pos"], s["slots"], cos_d,
                       sin_d, q_out=s["q_rot"])
    pa().attend_mixed(s["q_rot"], s["q_indptr"], s["k_pool"], s["v_pool"], s["page_table"], s["seq_lens"], Q_CAP,
                      L_CAP, scale, out=s["out"], workspace=s["ws"])


def _oracle_step(wl, cos_t, sin_t):
    pos = wl.positions()
    q_rot, k_rot, live, _, _ = oracle.rope_kv_store(wl.k_pool, wl.v_pool, wl.q, wl.k_new, wl.v_new, pos,
                                                    wl.slot_mapping, cos_t, sin_t, "bf16")
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, W.f32_to_bf16_bits(k_rot.astype(np.float32)), wl.v_new,
                             wl.slot_mapping)
    q_o = W.f32_to_bf16_bits(q_rot.astype(np.float32))
    return oracle.extend(q_o, wl.q_indptr, kp, vp, wl.page_table, wl.seq_lens, wl.scale, "bf16")


def test_captured_step_replays_match_eager_and_oracle():
    banner("graph capture of rope+store+mixed attention, 3 batches x 2 replays")
    T = torch()
    scale = 1.0 / np.sqrt(D)
    cos_t, sin_t = W.rope_tables(L_CAP, D)
    cos_d, sin_d = T.from_numpy(cos_t).cuda(), T.from_numpy(sin_t).cuda()
    bf = dict(dtype=T.bfloat16, device="cuda")
    static = {
        "k_pool": T.zeros(NPAGES, P, Hkv, D, **bf), "v_pool": T.zeros(NPAGES, P, Hkv, D, **bf),
        "q": T.zeros(T_CAP, Hq, D, **bf), "q_rot": T.zeros(T_CAP, Hq, D, **bf), "out": T.zeros(T_CAP, Hq, D, **bf),
        "k_new": T.zeros(T_CAP, Hkv, D, **bf), "v_new": T.zeros(T_CAP, Hkv, D, **bf),
        "slots": T.full((T_CAP,), -1, dtype=T.int64, device="cuda"),
        "pos": T.zeros(T_CAP, dtype=T.int32, device="cuda"),
        "q_indptr": T.zeros(B_CAP + 1, dtype=T.int32, device="cuda"),
        "page_table": T.zeros(B_CAP, STRIDE, dtype=T.int32, device="cuda"),
        "seq_lens": T.zeros(B_CAP, dtype=T.int32, device="cuda"),
    }
    nb = pa().decode_workspace_bytes(B_CAP, Hq, Hkv, D, L_CAP)
    static["ws"] = T.empty(nb, dtype=T.uint8, device="cuda")

    # warm up on a side stream, then capture
    _fill(static, _batch(0), cos_t)
    side = T.cuda.Stream()
    side.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(side):
        _step(static, cos_d, sin_d, scale)
    T.cuda.current_stream().wait_stream(side)
    T.cuda.synchronize()
    graph = T.cuda.CUDAGraph()
    _fill(static, _batch(0), cos_t)
    with T.cuda.graph(graph):
        _step(static, cos_d, sin_d, scale)
    T.cuda.synchronize()

    for rep in range(2):
        for case in range(len(BATCHES)):
            wl = _batch(case)
            N = int(wl.q_indptr[-1])
            # eager reference on the same inputs
            _fill(static, wl, cos_t)
            T.cuda.synchronize()
            _step(static, cos_d, sin_d, scale)
            T.cuda.synchronize()
            eager = static["out"][:N].clone()
            eager_pool = static["k_pool"].clone()
            # the replay
            _fill(static, wl, cos_t)
            T.cuda.synchronize()
            graph.replay()
            T.cuda.synchronize()
            assert bits(static["out"][:N]) == bits(eager), f"replay {rep} batch {case} differs from eager"
            assert bits(static["k_pool"]) == bits(eager_pool)
            assert_close(f64(static["out"][:N]), _oracle_step(wl, cos_t, sin_t), f"replay {rep} batch {case}")
            print(f"[result] replay {rep} batch {case}: {N} rows match eager bit for bit and the oracle",
                  flush=True)

"""Cascade (prefix-aware) decode against the oracle's plain decode: reading a
group's shared prefix pages once for all its members must not change the
attention result (radix prefix sharing: nanoSGLang README, section
Architecture; "mini-sglang from Scratch", section "What you will be able to
do")."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_close, bits, f64, fresh, gpu_cascade, gpu_decode, named, oracle_whole, pa,
                         stored_oracle_pools, torch)

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def oracle_decode(wl, seqs=None):
    kp, vp = stored_oracle_pools(wl)
    sub = wl if seqs is None else wl.subset(seqs)
    return oracle.decode(sub.q, kp, vp, sub.page_table, sub.seq_lens, wl.scale, wl.dtype)


def test_cascade_matches_oracle_on_the_qwen3_8b_radix_workload():
    """Every element of all 256 requests against the oracle, and against the
    plain decode of the same inputs."""
    name = "qwen3_8b_radix"
    banner(f"cascade {name}")
    wl, dw = named(name)
    out = f64(gpu_cascade(wl, dw))
    err = assert_close(out, oracle_whole(name), f"cascade {name}")
    assert_close(out, f64(gpu_decode(wl, dw)), f"cascade vs decode {name}")
    print(f"[result] cascade {name}: all {wl.num_seqs} requests vs oracle, max abs err {err:.3g}", flush=True)


CASCADE_SWEEP = [
    # (lengths, Hq, Hkv, D, P, (group size, prefix pages), split, piece_keys)
    ([700, 1200, 1500, 900, 1800, 2100, 513, 1025], 32, 8, 128, 16, (4, 64), 0, 0),
    ([700, 1200, 1500, 900, 1800, 2100, 513, 1025], 32, 8, 128, 16, (4, 64), 128, 192),
    ([5, 40, 17, 3000, 64, 65], 8, 2, 128, 16, (3, 8), 64, 64),        # short members, partial use
    (list(range(1, 80)), 8, 2, 128, 16, (40, 4), 0, 0),                 # 40 members: two row blocks
    (list(range(1, 80)), 16, 2, 128, 16, (40, 4), 64, 64),              # group 8: three row blocks
    ([2000, 2100, 1, 4000], 4, 4, 128, 16, (2, 60), 0, 128),            # group 1
    ([300, 301, 302, 900], 4, 2, 64, 16, (4, 16), 0, 0),                # group 2, D=64
    ([3000, 2500, 2900, 1200], 8, 2, 128, 1, (4, 2048), 512, 2048),     # page size 1, page ids restaged
    ([3000, 2500, 2900, 1200], 8, 2, 128, 1, (4, 2048), 0, 0),
    ([1000, 1000, 1000], 64, 8, 128, 256, (3, 3), 0, 0),               # largest page
    ([0, 5, 0, 40, 33], 8, 2, 128, 16, (5, 2), 0, 0),                   # empty requests in a group
    ([300, 500, 640, 128, 200, 610, 333], 14, 2, 64, 16, (4, 8), 0, 0),  # group 7 (Qwen2.5-0.5B heads)
    (list(range(100, 140)), 14, 2, 64, 16, (20, 6), 64, 64),            # group 7: 20 members, two row blocks
    ([700, 1200, 1500, 900, 1800], 40, 8, 128, 16, (5, 32), 0, 0),      # group 5
    ([700, 1200, 1500, 900], 24, 8, 128, 16, (2, 32), 0, 0),            # group 3
    ([700, 1200, 1500, 900], 48, 8, 128, 16, (4, 32), 128, 0),          # group 6
]


@pytest.mark.parametrize("case", range(len(CASCADE_SWEEP)))
def test_cascade_sweep(case):
    lens, Hq, Hkv, D, P, radix, split, pk = CASCADE_SWEEP[case]
    banner(f"cascade sweep {case}: lens={lens[:8]} Hq={Hq} Hkv={Hkv} D={D} P={P} radix={radix} "
           f"split={split} pk={pk}")
    wl = W.make_custom(lens, Hq, Hkv, D, P, dtype="bf16", radix=radix, seed=300 + case)
    dw = fresh(wl)
    out = f64(gpu_cascade(wl, dw, split=split, piece_keys=pk))
    assert_close(out, oracle_decode(wl), f"cascade sweep {case}")
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0)


def test_cascade_at_any_cut_inside_the_shared_pages():
    """A member may declare any number of its shared keys as shared, also
    mid-page and zero; the rest are read as its own keys."""
    banner("cascade arbitrary cuts")
    wl = W.make_custom([900, 1000, 1100, 1200, 700, 800, 1500, 1600], 32, 8, 128, 16, dtype="bf16",
                       radix=(4, 40), seed=320)
    dw = fresh(wl)
    starts, ppt, shl = wl.cascade_inputs()
    rng = np.random.default_rng(7)
    cut = np.array([rng.integers(0, s + 1) for s in shl], np.int32)
    cut[0], cut[5] = 0, shl[5]
    out = f64(gpu_cascade(wl, dw, piece_keys=64, groups=(starts, ppt, cut)))
    assert_close(out, oracle_decode(wl), "cascade with arbitrary cuts")


def test_cascade_with_everything_shared():
    """Singleton groups whose prefix table is the request's own: every key
    goes through the matrix-core pass and the request's own pass is empty."""
    banner("cascade all keys shared")
    lens = [1, 63, 64, 65, 1000, 2047]
    wl = W.make_custom(lens, 16, 4, 128, 16, dtype="bf16", seed=321)
    dw = fresh(wl)
    starts = np.arange(len(lens) + 1, dtype=np.int32)
    out = f64(gpu_cascade(wl, dw, piece_keys=128, groups=(starts, wl.page_table, wl.seq_lens.astype(np.int32))))
    assert_close(out, oracle_decode(wl), "cascade all shared")


def test_cascade_without_sharing_is_the_plain_decode():
    banner("cascade no sharing")
    wl = W.make_custom([1, 17, 300, 1000, 2047], 32, 8, 128, 16, dtype="bf16", seed=322)
    dw = fresh(wl)
    out = gpu_cascade(wl, dw)
    assert_close(f64(out), oracle_decode(wl), "cascade without sharing")


def test_cascade_reruns_are_bit_identical():
    banner("cascade determinism")
    wl, dw = named("qwen3_8b_radix")
    a = bits(gpu_cascade(wl, dw))
    for _ in range(2):
        assert bits(gpu_cascade(wl, dw)) == a


def test_cascade_stages_called_one_at_a_time_match_the_single_call():
    banner("cascade staged calls")
    from gpu_helpers import cascade_device, pa

    wl, dw = named("qwen3_8b_radix")
    whole = bits(gpu_cascade(wl, dw))
    gs, ppt, shl, gmax, msh = cascade_device(wl)
    T = torch()
    out = T.empty_like(dw.q)
    nb = pa().decode_cascade_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                             wl.max_seq_len, gs.numel() - 1, gmax, msh)
    ws = T.empty(nb, dtype=T.uint8, device="cuda")
    for stage in ("order", "prefix", "suffix", "combine"):
        pa().decode_cascade(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, gs, gmax, ppt,
                            shl, msh, wl.scale, out=out, workspace=ws, stage=stage)
    T.cuda.synchronize()
    assert bits(out) == whole


def test_cascade_prefix_stage_on_a_second_stream():
    """The shared-prefix pass on another stream, concurrently with the work
    order and the own-keys pass: the same bits as the single call, on several
    steps in a row with a fresh output each time."""
    banner("cascade prefix stage on a second stream")
    from gpu_helpers import cascade_device, pa

    wl, dw = named("qwen3_8b_radix")
    whole = bits(gpu_cascade(wl, dw))
    gs, ppt, shl, gmax, msh = cascade_device(wl)
    T = torch()
    nb = pa().decode_cascade_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                             wl.max_seq_len, gs.numel() - 1, gmax, msh)
    ws = T.empty(nb, dtype=T.uint8, device="cuda")
    main = T.cuda.current_stream()
    side = T.cuda.Stream()

    def stage(name, out):
        pa().decode_cascade(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, gs, gmax, ppt,
                            shl, msh, wl.scale, out=out, workspace=ws, stage=name)

    for _ in range(3):
        out = T.full_like(dw.q, float("nan"))
        side.wait_stream(main)
        with T.cuda.stream(side):
            stage("prefix", out)
        stage("order", out)
        stage("suffix", out)
        main.wait_stream(side)
        stage("combine", out)
        T.cuda.synchronize()
        assert bits(out) == whole


def test_cascade_prefix_stage_beside_the_store():
    """The prefix pass started before the store of the step's new rows, on a
    second stream (the new rows lie on pages of their own requests, which the
    prefix pass never reads): the same bits as the single call after the
    store."""
    banner("cascade prefix stage beside the store")
    from gpu_helpers import cascade_device, pa

    wl, dw_stored = named("qwen3_8b_radix")
    whole = bits(gpu_cascade(wl, dw_stored))
    starts, ppt_h, shl_h = wl.cascade_inputs()
    P = wl.page_size
    shared = set()
    for j in range(len(starts) - 1):
        need = int(shl_h[starts[j]:starts[j + 1]].max(initial=0))
        shared.update(ppt_h[j, :(need + P - 1) // P].tolist())
    assert not shared & set((wl.slot_mapping[wl.slot_mapping >= 0] // P).tolist())
    gs, ppt, shl, gmax, msh = cascade_device(wl)
    T = torch()
    nb = pa().decode_cascade_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                             wl.max_seq_len, gs.numel() - 1, gmax, msh)
    ws = T.empty(nb, dtype=T.uint8, device="cuda")
    main = T.cuda.current_stream()
    side = T.cuda.Stream()
    for _ in range(2):
        dw = W.to_device(wl)  # new rows not stored yet
        T.cuda.synchronize()
        out = T.full_like(dw.q, float("nan"))

        def stage(name):
            pa().decode_cascade(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, gs, gmax,
                                ppt, shl, msh, wl.scale, out=out, workspace=ws, stage=name)

        side.wait_stream(main)
        with T.cuda.stream(side):
            stage("prefix")
        pa().kv_store(dw.k_pool, dw.v_pool, dw.k_new, dw.v_new, dw.slot_mapping)
        stage("order")
        stage("suffix")
        main.wait_stream(side)
        stage("combine")
        T.cuda.synchronize()
        assert bits(out) == whole


# --------------------------------------------------------------------------
# the step's new rows stored by the work-order launch
# --------------------------------------------------------------------------
def _cascade_with_rows(wl, dw, stage=None, out=None, ws=None, stream=None):
    gs, ppt, shl, gmax, msh = cascade_device_cached(wl)
    return pa().decode_cascade(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, gs, gmax,
                               ppt, shl, msh, wl.scale, out=out, workspace=ws, stage=stage, stream=stream,
                               k_new=dw.k_new, v_new=dw.v_new, slot_mapping=dw.slot_mapping)


_GROUPS = {}


def cascade_device_cached(wl):
    key = id(wl)
    if key not in _GROUPS:
        from gpu_helpers import cascade_device
        _GROUPS[key] = cascade_device(wl)
    return _GROUPS[key]


def _assert_pools_stored(wl, dw):
    kp, vp = stored_oracle_pools(wl)
    assert W.to_numpy_storage(dw.k_pool, wl.dtype).tobytes() == kp.tobytes(), "K pool differs from the store"
    assert W.to_numpy_storage(dw.v_pool, wl.dtype).tobytes() == vp.tobytes(), "V pool differs from the store"


def test_cascade_stores_the_new_rows_on_the_radix_workload():
    """One call stores the 256 new rows and attends them: pools bit-exact
    against the oracle's store, every output element against the oracle;
    the two-stream staged schedule gives the same bits."""
    name = "qwen3_8b_radix"
    banner(f"cascade with new rows {name}")
    T = torch()
    wl = W.make(name, poison="nan")
    dw = W.to_device(wl)  # new rows not stored yet
    out = _cascade_with_rows(wl, dw)
    T.cuda.synchronize()
    _assert_pools_stored(wl, dw)
    err = assert_close(f64(out), oracle_whole(name), f"cascade with rows {name}")
    # staged: prefix on a second stream from the start, the order-and-store
    # launch, own keys and combine on the main stream, on fresh pools
    dw2 = W.to_device(wl)
    gs, ppt, shl, gmax, msh = cascade_device_cached(wl)
    nb = pa().decode_cascade_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                             wl.max_seq_len, len(gs) - 1, gmax, msh)
    ws = T.empty(nb, dtype=T.uint8, device="cuda")
    out2 = T.empty_like(dw2.q)
    side = T.cuda.Stream()
    cur = T.cuda.current_stream()
    side.wait_stream(cur)
    with T.cuda.stream(side):
        _cascade_with_rows(wl, dw2, stage="prefix", out=out2, ws=ws, stream=side)
    for st in ("order", "suffix"):
        _cascade_with_rows(wl, dw2, stage=st, out=out2, ws=ws)
    cur.wait_stream(side)
    _cascade_with_rows(wl, dw2, stage="combine", out=out2, ws=ws)
    T.cuda.synchronize()
    _assert_pools_stored(wl, dw2)
    assert bits(out2) == bits(out), "staged schedule differs from the single call"
    print(f"[result] cascade with rows {name}: pools exact, max abs err {err:.3g}", flush=True)


@pytest.mark.parametrize("case", ["small", "large"])
def test_cascade_stores_rows_without_and_with_a_work_order(case):
    """A batch too small for a work order (the launch only stores), and a
    batch of more than 256 requests (1024-thread order work-group)."""
    if case == "small":
        lens, radix = [300, 200, 90, 400, 129, 40], (3, 8)
    else:
        rng = np.random.default_rng(77)
        lens, radix = rng.integers(200, 1500, 640).tolist(), (16, 8)
    banner(f"cascade with new rows, {case} batch: {len(lens)} requests")
    # the large batch: 640 requests x 8 KV heads, work order of 10240 units
    Hq, Hkv = (8, 2) if case == "small" else (32, 8)
    wl = W.make_custom(lens, Hq, Hkv, 128, 16, dtype="bf16", radix=radix, seed=330)
    dw = W.to_device(wl)
    out = _cascade_with_rows(wl, dw)
    torch().cuda.synchronize()
    _assert_pools_stored(wl, dw)
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    assert_close(f64(out), ref, f"cascade with rows, {case}")

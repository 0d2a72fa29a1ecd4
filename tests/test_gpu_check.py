"""The debug check of device-resident inputs: a valid batch reports nothing,
and each planted violation (made on the host, in the tables only: no kernel
that reads pool pages ever sees them) reports its own bit."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import fresh, pa, torch

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def check(wl, dw, page_table=None, seq_lens=None, q_indptr=None, slots=None, max_q_len=None):
    T = torch()
    dev = lambda x, dt: T.from_numpy(np.ascontiguousarray(x).astype(dt)).cuda()
    pt = dw.page_table if page_table is None else dev(page_table, np.int32)
    sl = dw.seq_lens if seq_lens is None else dev(seq_lens, np.int32)
    qi = dw.q_indptr if q_indptr is None else dev(q_indptr, np.int32)
    sm = dw.slot_mapping if slots is None else dev(slots, np.int64)
    return pa().check_batch(dw.k_pool, dw.v_pool, pt, sl, wl.max_seq_len, q_indptr=qi,
                            max_q_len=max_q_len or wl.max_q_len, slot_mapping=sm)


def test_valid_batches_report_nothing():
    banner("check: valid batches")
    for name in ("qwen25_05b", "qwen3_06b_p1", "qwen3_8b_extend"):
        wl = W.make(name)
        assert check(wl, fresh(wl)) == [], name


def test_each_violation_sets_its_bit():
    banner("check: planted violations")
    wl = W.make_custom([40, 300, 17, 1000], 8, 2, 128, 16, dtype="bf16", kind="extend", n_new=[5, 1, 17, 64],
                       seed=800)
    dw = fresh(wl)
    assert check(wl, dw) == []
    sl = wl.seq_lens.copy(); sl[2] = wl.max_seq_len + 1
    assert check(wl, dw, seq_lens=sl) == ["seq_len"]
    sl = wl.seq_lens.copy(); sl[0] = -3
    assert "seq_len" in check(wl, dw, seq_lens=sl)
    pt = wl.page_table.copy(); pt[1, 5] = wl.num_pages
    assert check(wl, dw, page_table=pt) == ["page_id"]
    pt = wl.page_table.copy(); pt[3, 0] = -1
    assert check(wl, dw, page_table=pt) == ["page_id"]
    pt = wl.page_table.copy(); pt[0, pt.shape[1] - 1] = -7  # beyond the request's pages: not read, not reported
    assert check(wl, dw, page_table=pt) == []
    qi = wl.q_indptr.copy(); qi[1] = qi[2] + 1  # a negative chunk
    assert "q_indptr" in check(wl, dw, q_indptr=qi)
    assert check(wl, dw, max_q_len=32) == ["q_indptr"]  # a chunk of 64 rows above the bound
    sm = wl.slot_mapping.copy(); sm[3] = wl.num_pages * wl.page_size
    assert check(wl, dw, slots=sm) == ["slot_range"]
    sm = wl.slot_mapping.copy(); sm[10] = sm[50]
    assert check(wl, dw, slots=sm) == ["slot_duplicate"]
    sm = wl.slot_mapping.copy(); sm[10] = -1; sm[50] = -1  # padding twice is fine
    assert check(wl, dw, slots=sm) == []


def test_cascade_description_checks():
    banner("check: cascade group description")
    T = torch()
    wl = W.make_custom([300, 200, 90, 400, 129, 40], 8, 2, 128, 16, dtype="bf16", radix=(3, 8), seed=801)
    dw = fresh(wl)
    starts, ppt, shl = wl.cascade_inputs()
    dev = lambda x: T.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()
    gmax = int(np.diff(starts).max())
    msh = int(shl.max())

    def run(starts=starts, ppt=ppt, shl=shl, gmax=gmax, msh=msh):
        return pa().check_cascade(dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, dev(starts), gmax, dev(ppt),
                                  dev(shl), msh)

    assert run() == []
    s2 = starts.copy(); s2[-1] -= 1
    assert run(starts=s2) == ["group_starts"]
    assert run(gmax=gmax - 1) == ["group_starts"]
    sh2 = shl.copy(); sh2[0] = msh + 16
    assert "shared_len" in run(shl=sh2)
    assert run(msh=msh - 1) == ["shared_len"]
    sh2 = shl.copy(); sh2[1] = -1
    assert run(shl=sh2) == ["shared_len"]
    p2 = ppt.copy(); p2[0, 0] = (p2[0, 0] + 1) % wl.num_pages  # not request 0's first page any more
    assert run(ppt=p2) == ["prefix_page"]
    p2 = ppt.copy(); p2[1, 0] = wl.num_pages
    assert run(ppt=p2) == ["prefix_page"]
    # a request that shares nothing may sit in a group of its own
    sh2 = shl.copy(); sh2[2] = 0
    assert run(shl=sh2) == []


def test_stream_read_calibration_reads_the_buffer():
    banner("stream_read calibration")
    T = torch()
    src = T.arange(0, 1 << 20, dtype=T.int32, device="cuda")  # 4 MiB
    sink = T.zeros(1, dtype=T.int32, device="cuda")
    pa().stream_read(src, sink)
    T.cuda.synchronize()
    assert int(sink.item()) != 0
    # a size that is not a whole number of grid strides
    sink.zero_()
    pa().stream_read(src[: (1 << 20) - 4 * 37], sink)
    T.cuda.synchronize()
    assert int(sink.item()) != 0

"""The allocation-free decode entry point (pa_decode_noalloc) against the
decode entry point with a caller workspace (pa_decode): the same kernels and
split plan, so the same bits, on two calls in a row through the static
scratch buffer, the second with a smaller batch; both also within the
tolerance of the CPU oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, bits, f64, fresh, pa, stored_oracle_pools, torch

pytestmark = pytest.mark.gpu


def _check(wl, split):
    print(f"\n[case] decode_noalloc {wl.name}: {wl.num_seqs} requests, Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
          f"D={wl.head_dim} P={wl.page_size} split={split}", flush=True)
    T = torch()
    dw = fresh(wl)
    ref_out = pa().decode(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, wl.scale,
                          split_tokens=split)
    out = T.full_like(dw.q, float("nan"))
    pa().decode_noalloc(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, wl.scale, out,
                        split_tokens=split)
    T.cuda.synchronize()
    assert bits(out) == bits(ref_out), "decode_noalloc differs from decode"
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    err = assert_close(f64(out), ref, f"decode_noalloc {wl.name}")
    print(f"[result] decode_noalloc {wl.name}: same bits as decode, max abs err {err:.3g}", flush=True)


def test_noalloc_two_calls_second_smaller():
    # first call: the Qwen3-0.6B-shaped batch (64 requests up to 2048 keys,
    # page size 1); second call: a smaller batch of another shape, whose
    # pieces land on what the first call left in the buffer
    _check(W.make("qwen3_06b_p1", poison="nan"), 0)
    _check(W.make_custom([0, 1, 17, 300, 641], 14, 2, 64, 16, dtype="bf16", seed=31), 64)


def test_noalloc_rejects_a_batch_beyond_the_scratch_buffer():
    print("\n[case] decode_noalloc over the scratch limit", flush=True)
    T = torch()
    wl = W.make_custom([100, 200], 32, 8, 128, 16, dtype="bf16", seed=32)
    dw = fresh(wl)
    out = T.zeros_like(dw.q)
    big_q = T.zeros(4096, 32, 128, dtype=T.bfloat16, device="cuda")
    pt = T.zeros(4096, 512, dtype=T.int32, device="cuda")
    sl = T.zeros(4096, dtype=T.int32, device="cuda")
    with pytest.raises(pa().PagedAttnError, match="PA_ERR_SCRATCH"):
        pa().decode_noalloc(big_q, dw.k_pool, dw.v_pool, pt, sl, 8192, wl.scale, T.zeros_like(big_q))
    # nothing was launched, and the next call is unaffected
    pa().decode_noalloc(dw.q, dw.k_pool, dw.v_pool, dw.page_table, dw.seq_lens, wl.max_seq_len, wl.scale, out)
    T.cuda.synchronize()
    kp, vp = stored_oracle_pools(wl)
    ref = oracle.decode(wl.q, kp, vp, wl.page_table, wl.seq_lens, wl.scale, wl.dtype)
    assert_close(f64(out), ref, "decode_noalloc after a refused call")
    assert np.isfinite(f64(out)).all()

"""Fused rotary embedding + KV store on the GPU against the oracle: rotated
rows within one bf16 ulp of the exact float64 rotation (fp32 rows within a
few fp32 ulps), value rows and untouched slots bit-exact, padding rows
skipped; then attention over the rotated pool against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_close, f64, pa, torch

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def dev(x, dtype):
    T = torch()
    if dtype == "bf16":
        return T.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(T.bfloat16).cuda()
    return T.from_numpy(np.ascontiguousarray(x)).cuda()


def rotation_bound(x_pairs_abs, ref, dtype):
    """Allowed |gpu - exact|: one ulp of the storage format (fp32 arithmetic,
    one rounding), plus fp32 rounding of the two products."""
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -21
    return rel * np.abs(ref) + 2.0 ** -22 * x_pairs_abs + 1e-30


def pair_abs(x, dtype):
    xf = oracle.widen(x, dtype)
    half = xf.shape[-1] // 2
    s = np.abs(xf[..., :half]) + np.abs(xf[..., half:])
    return np.concatenate([s, s], axis=-1)


def run_case(wl, max_pos, padding_rows=(), in_place=False):
    dtype = wl.dtype
    cos_t, sin_t = W.rope_tables(max_pos, wl.head_dim)
    pos = wl.positions()
    slots = wl.slot_mapping.copy()
    for r in padding_rows:
        slots[r] = -1
    T = torch()
    kp, vp = dev(wl.k_pool, dtype), dev(wl.v_pool, dtype)
    q = dev(wl.q, dtype)
    q_before = q.clone()
    q_out = q if in_place else T.full_like(q, 7.0)
    out = pa().rope_kv_store(kp, vp, q, dev(wl.k_new, dtype), dev(wl.v_new, dtype),
                             T.from_numpy(pos).cuda(), T.from_numpy(slots).cuda(),
                             T.from_numpy(cos_t).cuda(), T.from_numpy(sin_t).cuda(), q_out=q_out)
    T.cuda.synchronize()
    q_rot, k_rot, live, _, v_ref = oracle.rope_kv_store(wl.k_pool, wl.v_pool, wl.q, wl.k_new, wl.v_new, pos, slots,
                                                        cos_t, sin_t, dtype)
    P = wl.page_size
    k_gpu = W.to_numpy_storage(kp, dtype).reshape(wl.num_pages * P, wl.num_kv_heads, wl.head_dim)
    v_gpu = W.to_numpy_storage(vp, dtype).reshape(wl.num_pages * P, wl.num_kv_heads, wl.head_dim)
    k_old = wl.k_pool.reshape(wl.num_pages * P, wl.num_kv_heads, wl.head_dim)
    written = slots[live]
    # rotated keys in their slots
    got_k = oracle.widen(k_gpu[written], dtype)
    bound = rotation_bound(pair_abs(wl.k_new[live], dtype), k_rot[live], dtype)
    bad = np.abs(got_k - k_rot[live]) > bound
    assert not bad.any(), f"rotated keys: {int(bad.sum())} elements beyond one ulp"
    # values and every other slot byte for byte
    assert v_gpu.tobytes() == v_ref.reshape(v_gpu.shape).tobytes()
    others = np.setdiff1d(np.arange(wl.num_pages * P), written)
    assert k_gpu[others].tobytes() == k_old[others].tobytes()
    # rotated queries; padding rows untouched
    got_q = oracle.widen(W.to_numpy_storage(out, dtype), dtype)
    bq = rotation_bound(pair_abs(wl.q[live], dtype), q_rot[live], dtype)
    assert not (np.abs(got_q[live] - q_rot[live]) > bq).any(), "rotated queries beyond one ulp"
    if (~live).any():
        expect_pad = q_before if in_place else T.full_like(q_before, 7.0)
        assert (out[T.from_numpy(~live).cuda()] == expect_pad[T.from_numpy(~live).cuda()]).all()
    return kp, vp, out, q_rot, k_rot


@pytest.mark.parametrize("dtype,D,P", [("bf16", 128, 16), ("bf16", 64, 1), ("f32", 128, 16), ("f32", 64, 4)])
def test_rope_store_decode_rows(dtype, D, P):
    banner(f"rope+store decode rows {dtype} D={D} P={P}")
    wl = W.make_custom([1, 17, 300, 1000, 2047, 64], 32, 8, D, P, dtype=dtype, seed=400)
    run_case(wl, 4096, padding_rows=(2,))


def test_rope_store_extend_chunk_in_place():
    banner("rope+store extend chunk, q in place")
    wl = W.make_custom([600, 129, 1000], 32, 8, 128, 16, dtype="bf16", kind="extend", n_new=[512, 129, 33],
                       seed=401)
    run_case(wl, 2048, in_place=True)


def test_rope_store_then_attention_matches_oracle():
    """The rotated pool and queries feed decode; the result matches the
    oracle's decode over the oracle's rotated rows (rounded to the pool
    format as the store rounds them)."""
    banner("rope+store then decode")
    wl = W.make_custom([5, 200, 1500, 64], 16, 4, 128, 16, dtype="bf16", seed=402)
    kp, vp, q_out, q_rot, k_rot = run_case(wl, 2048)
    out = pa().decode(q_out, kp, vp, torch().from_numpy(wl.page_table).cuda(),
                      torch().from_numpy(wl.seq_lens).cuda(), wl.max_seq_len, wl.scale)
    torch().cuda.synchronize()
    # oracle pools: the store with k rows replaced by the exact rotation rounded to bf16
    k_rows = W.f32_to_bf16_bits(k_rot.astype(np.float32))
    kp_o, vp_o = oracle.kv_store(wl.k_pool, wl.v_pool, k_rows, wl.v_new, wl.slot_mapping)
    q_o = W.f32_to_bf16_bits(q_rot.astype(np.float32))
    ref = oracle.decode(q_o, kp_o, vp_o, wl.page_table, wl.seq_lens, wl.scale, "bf16")
    assert_close(f64(out), ref, "decode after rope+store")

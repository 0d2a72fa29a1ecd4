"""The seeded input generator: determinism, shapes, page-assignment structure
and poisoning."""
import math

import numpy as np
import pytest

import workloads as W


def test_same_seed_same_bytes():
    a = W.make("qwen25_05b")
    b = W.make("qwen25_05b")
    for f in ("seq_lens", "page_table", "k_pool", "v_pool", "q", "k_new", "v_new", "slot_mapping"):
        assert getattr(a, f).tobytes() == getattr(b, f).tobytes(), f
    c = W.make("qwen25_05b", seed=99)
    assert c.q.tobytes() != a.q.tobytes()


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_config_shapes(name):
    wl = W.make(name, with_values=False)
    spec = {
        "tiny": (4, 2, 1, 64, 16, "f32"),
        "qwen25_05b": (32, 14, 2, 64, 16, "bf16"),
        "qwen3_06b_p1": (64, 16, 8, 128, 1, "bf16"),
        "qwen3_8b_radix": (256, 32, 8, 128, 16, "bf16"),
        "qwen3_8b_extend": (8, 32, 8, 128, 16, "bf16"),
        "qwen3_8b_mixed": (256, 32, 8, 128, 16, "bf16"),
        "qwen3_8b_verify": (64, 32, 8, 128, 16, "bf16"),
    }[name]
    assert (wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype) == spec
    assert wl.page_table.shape[1] * wl.page_size >= wl.max_seq_len
    L = wl.seq_lens
    if name == "tiny":
        assert L.tolist() == [1, 17, 33, 64]
    elif name == "qwen25_05b":
        assert L.min() >= 100 and L.max() <= 640
    elif name == "qwen3_06b_p1":
        assert L.min() >= 256 and L.max() <= 2048 and wl.num_pages == 200_000
    elif name == "qwen3_8b_radix":
        assert L.min() >= 512 and L.max() <= 8192 and wl.num_pages == 65_536
    elif name == "qwen3_8b_verify":
        assert np.all(wl.n_new == 6) and L.min() >= 512 + 6 - 1 and L.max() <= 8192
    elif name == "qwen3_8b_mixed":
        assert np.all(wl.n_new[:8] == 512) and np.all(wl.n_new[8:] == 1)
        assert (L[:8] - 512).min() >= 0 and (L[:8] - 512).max() <= 4096
        assert L[8:].min() >= 512 and L[8:].max() <= 8192
    else:
        p = L - wl.n_new
        assert np.all(wl.n_new == 512) and p.min() >= 0 and p.max() <= 4096
    # new rows go to the slot of each request's newest tokens
    P = wl.page_size
    for b in range(wl.num_seqs):
        Lb, n = int(L[b]), int(wl.n_new[b])
        t = np.arange(Lb - n, Lb)
        expect = wl.page_lists[b][t // P].astype(np.int64) * P + t % P
        np.testing.assert_array_equal(wl.slot_mapping[wl.q_indptr[b]:wl.q_indptr[b + 1]], expect)


@pytest.mark.parametrize("name", ["tiny", "qwen25_05b", "qwen3_06b_p1", "qwen3_8b_extend", "qwen3_8b_mixed",
                                  "qwen3_8b_verify"])
def test_private_pages_are_distinct(name):
    wl = W.make(name, with_values=False)
    allp = np.concatenate(wl.page_lists)
    assert len(np.unique(allp)) == len(allp)
    assert allp.min() >= 0 and allp.max() < wl.num_pages


def test_radix_structure():
    wl = W.make("qwen3_8b_radix", with_values=False)
    P = wl.page_size
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        s = min(64, (L - 1) // P)
        shared = wl.shared_pages[b // 16]
        np.testing.assert_array_equal(wl.page_lists[b][:s], shared[:s])
        # the page with the newest token is private
        assert wl.page_lists[b][(L - 1) // P] not in set(shared.tolist())
    # private pages are distinct across the whole batch
    priv = np.concatenate([wl.page_lists[b][min(64, (int(wl.seq_lens[b]) - 1) // P):]
                           for b in range(wl.num_seqs)])
    assert len(np.unique(priv)) == len(priv)
    # unique bytes are well below logical bytes
    assert wl.kv_bytes_unique() < 0.8 * wl.kv_bytes_logical()


def test_log_uniform_lengths_reading():
    wl = W.make("qwen3_8b_radix", with_values=False)
    u = np.log(wl.seq_lens.astype(np.float64))
    assert u.min() >= math.log(512) and u.max() < math.log(8193)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_poison_marks_exactly_the_non_cached_slots(dtype):
    wl = W.make_custom([5, 16, 17, 1], 4, 2, 8, 4, dtype=dtype, poison="nan", seed=2)
    P = wl.page_size
    cached = set()
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        for t in range(L - 1):
            cached.add(int(wl.page_lists[b][t // P]) * P + t % P)
    flat = wl.k_pool.reshape(wl.num_pages * P, -1)
    if dtype == "bf16":
        isnan = (flat & 0x7FFF) > 0x7F80
    else:
        isnan = np.isnan(flat)
    for s in range(flat.shape[0]):
        assert isnan[s].all() == (s not in cached), s
        assert isnan[s].any() == (s not in cached), s


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6 -> even (1 + 2^-6)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_values_do_not_depend_on_thread_count(monkeypatch):
    a = W._normal_f32(5, 1, 3 * W._CHUNK + 17)
    monkeypatch.setattr(W.os, "cpu_count", lambda: 1)
    b = W._normal_f32(5, 1, 3 * W._CHUNK + 17)
    assert a.tobytes() == b.tobytes()


def test_positions_are_the_new_rows_absolute_positions():
    wl = W.make_custom([10, 3, 7], 4, 2, 64, 4, dtype="bf16", kind="extend", n_new=[4, 1, 7], seed=1)
    assert wl.positions().tolist() == [6, 7, 8, 9, 2, 0, 1, 2, 3, 4, 5, 6]


def test_rope_tables_are_the_standard_schedule():
    c, s = W.rope_tables(5, 8, theta=10000.0)
    assert c.dtype == np.float32 and c.shape == (5, 4)
    assert c[0].tolist() == [1.0] * 4 and s[0].tolist() == [0.0] * 4
    # pair j turns by p * 10000^(-2j/8) at position p
    assert abs(float(s[3, 1]) - math.sin(3 * 10000.0 ** (-0.25))) < 1e-7

"""Pins of the rotary-embedding oracle against what the pages and the
mathematics fix, independently of the oracle's own code: a hand-worked
example, the complex-number form of a plane rotation, closed forms and the
relative-position property, plus planted mistakes that each trip a pin."""
import importlib
import json
import math
from pathlib import Path

import numpy as np
import pytest

R = importlib.import_module("oracle.rope")
GOLDEN = Path(__file__).parent / "golden" / "rope_hand.json"


def standard_tables(max_pos, D, theta=1.0e6):
    """cos/sin of p * theta^(-2i/D), written here from the definition."""
    half = D // 2
    ang = np.array([[p * theta ** (-2.0 * i / D) for i in range(half)] for p in range(max_pos)])
    return np.cos(ang), np.sin(ang)


def f32(a):
    return np.asarray(a, np.float32)


def test_golden_hand_example():
    g = json.loads(GOLDEN.read_text())
    cos_t = np.array(g["cos_table"], float)
    sin_t = np.array(g["sin_table"], float)
    x = f32(np.array(g["x"], float))[:, None, :]
    out1 = R.rope(x, [1], cos_t, sin_t, "f32")
    assert out1[0, 0].tolist() == [float(v) for v in g["position_1_expected"][0]]
    out0 = R.rope(x, [0], cos_t, sin_t, "f32")
    assert out0[0, 0].tolist() == [float(v) for v in g["position_0_expected"][0]]
    st = g["store"]
    P, NP = st["page_size"], st["num_pages"]
    kp = np.full((NP, P, 1, 4), -7, np.float32)
    vp = np.full((NP, P, 1, 4), -8, np.float32)
    q_rot, k_rot, live, kp2, vp2 = R.rope_kv_store(
        kp, vp, f32(np.array(st["q"], float)), f32(np.array(st["k_new"], float)), f32(np.array(st["v_new"], float)),
        st["positions"], st["slot_mapping"], cos_t, sin_t, "f32")
    assert live.tolist() == [True, False]
    assert k_rot[0, 0].tolist() == [float(v) for v in st["expected_k_rot_row0"]]
    assert np.isnan(k_rot[1]).all() and np.isnan(q_rot[1]).all()
    flat_v = vp2.reshape(NP * P, 1, 4)
    assert flat_v[3, 0].tolist() == [float(v) for v in st["expected_v_slot3"]]
    assert (flat_v[:3] == -8).all()
    assert (kp2 == kp).all()  # the oracle reports rotated keys separately


@pytest.mark.parametrize("D,H,N", [(4, 1, 3), (64, 2, 5), (128, 3, 4)])
def test_matches_complex_rotation(D, H, N):
    """(a, b) -> (a + ib) * exp(i*angle), one element at a time."""
    rng = np.random.default_rng(D + H)
    half = D // 2
    ang = rng.uniform(-math.pi, math.pi, (10, half))
    cos_t, sin_t = np.cos(ang), np.sin(ang)
    x = f32(rng.standard_normal((N, H, D)))
    pos = rng.integers(0, 10, N)
    out = R.rope(x, pos, cos_t, sin_t, "f32")
    for n in range(N):
        for h in range(H):
            for i in range(half):
                z = complex(float(x[n, h, i]), float(x[n, h, i + half])) * complex(cos_t[pos[n], i], sin_t[pos[n], i])
                assert abs(out[n, h, i] - z.real) < 1e-12 and abs(out[n, h, i + half] - z.imag) < 1e-12


def test_position_zero_is_identity_and_norms_are_kept():
    D = 128
    cos_t, sin_t = standard_tables(4000, D)
    rng = np.random.default_rng(1)
    x = f32(rng.standard_normal((6, 4, D)))
    assert (R.rope(x, [0] * 6, cos_t, sin_t, "f32") == x.astype(np.float64)).all()
    pos = rng.integers(0, 4000, 6)
    out = R.rope(x, pos, cos_t, sin_t, "f32")
    xf = x.astype(np.float64)
    half = D // 2
    n_in = xf[..., :half] ** 2 + xf[..., half:] ** 2
    n_out = out[..., :half] ** 2 + out[..., half:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12, atol=1e-12)


def test_scores_depend_only_on_relative_position():
    D = 64
    cos_t, sin_t = standard_tables(300, D, theta=10000.0)
    rng = np.random.default_rng(2)
    q = f32(rng.standard_normal((1, 1, D)))
    k = f32(rng.standard_normal((1, 1, D)))
    for m, n, d in [(5, 2, 2), (100, 30, 50), (0, 0, 299), (40, 90, 7)]:
        # the same pair of positions shifted by d gives the same score
        s1 = float(np.sum(R.rope(q, [m], cos_t, sin_t, "f32") * R.rope(k, [n], cos_t, sin_t, "f32")))
        s2 = float(np.sum(R.rope(q, [m + d], cos_t, sin_t, "f32") * R.rope(k, [n + d], cos_t, sin_t, "f32")))
        assert abs(s1 - s2) < 1e-9 * max(1.0, abs(s1))


def test_bf16_rows_are_widened_exactly():
    D = 8
    cos_t, sin_t = standard_tables(4, D)
    x32 = np.array([[[1.5, -2.0, 0.25, 3.0, -0.5, 1.0, 2.5, -1.25]]], np.float32)
    bits = (x32.view(np.uint32) >> 16).astype(np.uint16)  # exact: these values fit bf16
    assert (R.rope(bits, [3], cos_t, sin_t, "bf16") == R.rope(x32, [3], cos_t, sin_t, "f32")).all()


def test_store_skips_padding_rejects_duplicates_and_keeps_other_slots():
    rng = np.random.default_rng(3)
    P, NP, H, D = 4, 3, 2, 8
    cos_t, sin_t = standard_tables(50, D)
    kp = f32(rng.standard_normal((NP, P, H, D)))
    vp = f32(rng.standard_normal((NP, P, H, D)))
    k_new = f32(rng.standard_normal((3, H, D)))
    v_new = f32(rng.standard_normal((3, H, D)))
    q = f32(rng.standard_normal((3, 2 * H, D)))
    q_rot, k_rot, live, kp2, vp2 = R.rope_kv_store(kp, vp, q, k_new, v_new, [7, 9, 11], [5, -1, 10], cos_t, sin_t,
                                                   "f32")
    assert live.tolist() == [True, False, True]
    fv = vp2.reshape(NP * P, H, D)
    assert (fv[5] == v_new[0]).all() and (fv[10] == v_new[2]).all()
    untouched = [s for s in range(NP * P) if s not in (5, 10)]
    assert (fv[untouched] == vp.reshape(NP * P, H, D)[untouched]).all()
    assert np.allclose(k_rot[2], R.rope(k_new[2:3], [11], cos_t, sin_t, "f32")[0])
    assert np.allclose(q_rot[0], R.rope(q[0:1], [7], cos_t, sin_t, "f32")[0])
    with pytest.raises(ValueError):
        R.rope_kv_store(kp, vp, q, k_new, v_new, [1, 2, 3], [5, 5, 6], cos_t, sin_t, "f32")


# ---- planted mistakes: each must trip a pin ------------------------------
def _interleaved(x, positions, cos_table, sin_table, dtype):
    xf = R.widen(x, dtype)
    out = np.empty_like(xf)
    for n, p in enumerate(positions):
        c, s = np.asarray(cos_table, float)[p], np.asarray(sin_table, float)[p]
        a, b = xf[n, :, 0::2], xf[n, :, 1::2]
        out[n, :, 0::2] = a * c - b * s
        out[n, :, 1::2] = b * c + a * s
    return out


def _make(variant):
    orig = R.rope

    def mutant(x, positions, cos_table, sin_table, dtype):
        if variant == "sign":
            return orig(x, positions, cos_table, -np.asarray(sin_table, float), dtype)
        if variant == "swap":
            return orig(x, positions, sin_table, cos_table, dtype)
        if variant == "next_position":
            return orig(x, [min(int(p) + 1, len(cos_table) - 1) for p in positions], cos_table, sin_table, dtype)
        raise AssertionError(variant)
    return mutant


PINS = [test_golden_hand_example, lambda: test_matches_complex_rotation(64, 2, 5),
        test_position_zero_is_identity_and_norms_are_kept, test_scores_depend_only_on_relative_position,
        test_store_skips_padding_rejects_duplicates_and_keeps_other_slots]


@pytest.mark.parametrize("mutation", ["interleaved", "sign", "swap", "next_position"])
def test_planted_mistake_is_caught(mutation, monkeypatch):
    monkeypatch.setattr(R, "rope", _interleaved if mutation == "interleaved" else _make(mutation))
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught the {mutation} mistake"

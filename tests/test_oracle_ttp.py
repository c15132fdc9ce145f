"""Pins of the oracle's Tied Trit-Planes quantizer ([TTP page]: the page
"Новый метод квантования Tied Trit-Planes сжимает DeepSeek-V4 до 4.0625 бит на
вес"): closed forms, brute-force nearest levels, the least-squares scale, the
page's rate. CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ttp_page_numbers.json")))


def _one_group(vals):
    w = np.asarray(vals, dtype=np.float32).reshape(1, 256)
    c, s, r = oracle.ttp_quantize(w, want_rounds=True)
    return w, oracle.ttp_levels(c)[0], s[0, 0], r[0, 0]


def test_rate_and_levels_match_the_page():
    # 4-bit codes plus one fp16 scale per 256 weights
    assert 4 + 16 / oracle.TTP_GROUP == GOLD["bits_per_weight"]
    # two balanced-ternary planes tied by 3 give exactly the 9 integer levels -4..4
    levels = sorted({GOLD["scale_tie"] * t1 + t2 for t1 in GOLD["plane_values"] for t2 in GOLD["plane_values"]})
    assert levels == list(range(-4, 5)) and len(levels) == GOLD["levels"]
    w = synthetic.student_t_rows_f32(8, 1024, seed=3)
    c, s = oracle.ttp_quantize(w)
    assert c.nbytes * 8 + s.nbytes * 8 == pytest.approx(GOLD["bits_per_weight"] * w.size)
    assert (c & 0xF).max() <= 8 and (c >> 4).max() <= 8


def test_exact_grid_group_is_reproduced():
    a = np.float32(0.125)                     # exact in fp16
    q = np.resize(np.arange(-4, 5), 256)      # every level, max |q| = 4
    w, lv, s, r = _one_group(a * q)
    assert np.array_equal(lv, q) and np.float16(a).view(np.uint16) == s and r == 1
    assert np.array_equal(oracle.ttp_dequantize(oracle.ttp_quantize(w)[0], np.array([[s]], np.uint16)), w)


def test_constant_group_closed_form():
    w, lv, s, r = _one_group(np.full(256, 0.3, np.float32))
    a = np.float16(np.float32(0.3) / np.float32(4))   # the start a = max|w| / 4 is already optimal
    assert s == a.view(np.uint16) and np.all(lv == 4) and r == 1
    assert oracle.ttp_dequantize(oracle.ttp_quantize(w)[0], np.array([[s]], np.uint16))[0, 0] == np.float32(a) * 4


def test_two_valued_group_least_squares_step():
    # start a = 0.25 gives levels 4 and 1; the least-squares scale for them is
    # (128*4*1 + 128*1*0.3) / (128*16 + 128*1) = 4.3 / 17, which keeps the levels
    vals = np.r_[np.ones(128), np.full(128, 0.3)].astype(np.float32)
    w, lv, s, r = _one_group(vals)
    a = np.float32((4.0 * 1.0 + float(np.float32(0.3))) / 17.0)
    assert s == np.float16(a).view(np.uint16) and r == 1
    assert np.all(lv[:128] == 4) and np.all(lv[128:] == 1)


def test_levels_are_nearest_for_the_stored_scale():
    w = synthetic.student_t_rows_f32(16, 2048, seed=4)
    c, s = oracle.ttp_quantize(w)
    lv = oracle.ttp_levels(c).reshape(16, 8, 256).astype(np.float64)
    a = s.view(np.float16).astype(np.float64)[:, :, None]
    g = w.reshape(16, 8, 256).astype(np.float64)
    cand = np.arange(-4, 5, dtype=np.float64)
    dist = np.abs(g[..., None] - a[..., None] * cand)           # brute force over the 9 levels
    chosen = np.abs(g - a * lv)
    assert np.all(chosen <= dist.min(axis=-1) * (1 + 1e-6) + 1e-12)


def test_converged_scale_is_the_least_squares_scale():
    w = synthetic.student_t_rows_f32(32, 4096, seed=5)
    c, s, r = oracle.ttp_quantize(w, want_rounds=True)
    lv = oracle.ttp_levels(c).reshape(-1, 256).astype(np.float64)
    g = w.reshape(-1, 256).astype(np.float64)
    a_ls = (g * lv).sum(1) / (lv * lv).sum(1)                   # normal equation of min_a |w - a q|^2
    a_h = s.reshape(-1).view(np.float16).astype(np.float64)
    done = r.reshape(-1) < 8
    assert done.sum() > 10
    rel = np.abs(a_h[done] - a_ls[done]) / a_ls[done]
    assert np.quantile(rel, 0.9) < 2.0 ** -10                   # fp16 rounding of the converged scale


def test_alternating_solver_beats_its_start():
    w = synthetic.student_t_rows_f32(32, 4096, seed=6)
    c, s = oracle.ttp_quantize(w)
    err = np.sum((w.astype(np.float64) - oracle.ttp_dequantize(c, s)) ** 2)
    g = w.reshape(-1, 256)
    a0 = (np.abs(g).max(1, keepdims=True) / np.float32(4)).astype(np.float16).astype(np.float32)
    q0 = np.clip(np.rint(g / a0), -4, 4)
    err0 = np.sum((g.astype(np.float64) - a0 * q0) ** 2)
    assert err < 0.9 * err0


def test_zero_group_and_non_finite_weight():
    w, lv, s, r = _one_group(np.zeros(256))
    assert s == 0 and np.all(lv == 0) and r == 0
    bad = np.zeros((1, 256), np.float32)
    bad[0, 7] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.ttp_quantize(bad)

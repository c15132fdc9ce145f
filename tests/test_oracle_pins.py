"""Pins of the CPU oracle against facts fixed independently of it: closed forms,
exact rational arithmetic, brute force on tiny inputs, invariants of Lloyd's
algorithm, independent library conversions and the numbers printed on the
[VQ3R page] (tests/golden/vq3r_page_numbers.json). CPU only."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import dist8_exact_chain, dist8_real, frac, round_fp32

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "vq3r_page_numbers.json")))


# ------------------------------------------------------------- fp16 format
def test_f16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_bits_to_f32(int(b)) for b in bits], dtype=np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isinf(got[np.isinf(ref)]))


def test_f16_encode_vs_numpy():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(100),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),      # subnormal range
        np.float32([0, -0.0, 65504, 65519.99, 65520, 65536, 1e-8, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                    1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 6.1e-5, 5.96e-8, -2.0 ** -14]),
        # exact fp16 midpoints (ties to even)
        np.float32([(np.float16(1.0).astype(np.float32) + np.float32(2.0 ** -11) * (2 * k + 1)) for k in range(50)]),
    ]).astype(np.float32)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------- row scale
@pytest.mark.parametrize("a,expect", [
    (1.0, 1.0), (0.5, 0.5), (-3.0, 3.0), (1 + 2.0 ** -11, 1.0),            # tie -> even (1.0)
    (1 + 3 * 2.0 ** -11, 1 + 2.0 ** -9),                                   # tie -> even mantissa
    (0.0, 0.0), (2.0 ** -20, 2.0 ** -20),                                  # fp16 subnormal scale
])
def test_row_scale_constant_rows(a, expect):
    w = np.full((1, 64), a, dtype=np.float32)
    s = oracle.row_scales(w)
    assert oracle.f16_bits_to_f32(int(s[0])) == np.float32(expect)


def test_row_scale_closed_form_and_numpy():
    # rows of 3 and 4: mean square 12.5 -> rms sqrt(12.5)
    w = np.tile(np.float32([3, 4]), 32)[None, :]
    s = oracle.row_scales(w)
    assert s[0] == np.float16(np.float32(math.sqrt(12.5))).view(np.uint16)
    # random rows against numpy's independent reductions and conversions
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((64, 1024)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    s = oracle.row_scales(W)
    ref = np.sqrt(np.mean(W.astype(np.float64) ** 2, axis=1)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(s, ref)


def test_row_scale_errors():
    with pytest.raises(oracle.OracleError):
        oracle.row_scales(np.full((1, 8), 70000.0, dtype=np.float32))    # RMS beyond fp16
    w = np.ones((1, 8), dtype=np.float32)
    w[0, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.row_scales(w)


# ------------------------------------------------------------- distance / argmin
def test_dist8_matches_exact_fma_chain():
    rng = np.random.default_rng(3)
    for _ in range(300):
        scale = 10.0 ** rng.integers(-20, 4)
        r = (rng.standard_normal(8) * scale).astype(np.float32)
        c = (rng.standard_normal(8) * scale).astype(np.float32)
        got = oracle.dist8(r, c)
        assert got.view(np.uint32) == dist8_exact_chain(r, c).view(np.uint32)


def test_dist8_sign_and_order_sensitive_cases():
    # a transposed operand or a dropped term changes these values
    r = np.float32([1, 2, 3, 4, 5, 6, 7, 8])
    c = np.zeros(8, np.float32)
    assert oracle.dist8(r, c) == np.float32(204)
    assert oracle.dist8(c, r) == np.float32(204)
    c2 = np.float32([1, 2, 3, 4, 5, 6, 7, 9])
    assert oracle.dist8(r, c2) == np.float32(1)


def _bound(dmin):
    return 40 * 2.0 ** -24 * float(dmin) + 1e-40


def test_argmin_brute_force_exact():
    rng = np.random.default_rng(4)
    for trial in range(60):
        K = int(rng.choice([2, 5, 16, 64, 256]))
        C = rng.standard_normal((K, 8)).astype(np.float32)
        r = rng.standard_normal(8).astype(np.float32)
        got = oracle.argmin(r, C)
        d = [dist8_real(r, C[j]) for j in range(K)]
        dmin = min(d)
        # the oracle's pick is within the fp32 evaluation error of the true minimum
        assert float(d[got] - dmin) <= _bound(dmin)
        order = sorted(range(K), key=lambda j: d[j])
        if float(d[order[1]] - d[order[0]]) > 2 * _bound(d[order[1]]):
            assert got == order[0]


def test_argmin_ties_lowest_index():
    r = np.zeros(8, np.float32)
    C = np.full((8, 8), 10, np.float32)
    C[0] = 0
    C[0, 0] = 5
    C[3] = 0
    C[5] = 0
    C[6] = 0
    C[3, 1] = 1      # distance 1
    C[5, 2] = -1     # distance 1 (exact tie)
    C[6, 1] = 1      # duplicate of 3
    assert oracle.argmin(r, C) == 3
    C[1] = C[5]
    assert oracle.argmin(r, C) == 1


def test_argmin_near_tie_resolved_by_fp32_chain():
    # two codewords whose true distances differ by less than an ulp of d: the
    # fixed fp32 chain decides, and the oracle must follow that chain exactly
    rng = np.random.default_rng(5)
    for _ in range(200):
        r = rng.standard_normal(8).astype(np.float32)
        c0 = rng.standard_normal(8).astype(np.float32)
        c1 = c0.copy()
        k = rng.integers(8)
        c1[k] = np.nextafter(c1[k], np.float32(np.inf))
        C = np.stack([c1, c0]) if rng.integers(2) else np.stack([c0, c1])
        d0 = dist8_exact_chain(r, C[0])
        d1 = dist8_exact_chain(r, C[1])
        want = 1 if d1 < d0 else 0
        assert oracle.argmin(r, C) == want


# ------------------------------------------------------------- greedy encode
def _separated_codebooks(rng, K=16, stages=3):
    """Codewords on three well separated dyadic scales, so that any vector
    C1[a] + C2[b] + C3[c] is greedily decoded back to (a, b, c) exactly."""
    cbs = []
    for t, sc in enumerate([16.0, 2.0, 0.25][:stages]):
        pats = set()
        while len(pats) < K:
            pats.add(tuple(rng.choice([-1.0, 1.0], 8)))
        cbs.append(np.float32(sc) * np.array(sorted(pats), dtype=np.float32))
    return np.stack(cbs).astype(np.float32)


def test_greedy_recovers_exact_sums():
    rng = np.random.default_rng(6)
    cb = _separated_codebooks(rng)
    truth = rng.integers(0, 16, size=(500, 3))
    v = cb[0][truth[:, 0]] + cb[1][truth[:, 1]] + cb[2][truth[:, 2]]
    idx = oracle.encode_vectors(v, cb)
    assert np.array_equal(idx, truth)
    # partial sums: stage 1 alone gives the vq "1-stage" vector exactly C1[a]
    idx1 = oracle.encode_vectors(v, cb[:1])
    assert np.array_equal(idx1[:, 0], truth[:, 0])


def test_greedy_never_better_than_joint_two_stage():
    rng = np.random.default_rng(7)
    for _ in range(40):
        cb = rng.standard_normal((2, 8, 8)).astype(np.float32) * np.float32([[[1.0]], [[0.4]]])
        v = rng.standard_normal((2, 8)).astype(np.float32)
        idx = oracle.encode_vectors(v, cb)
        for n in range(2):
            g = v[n].astype(np.float64) - cb[0, idx[n, 0]] - cb[1, idx[n, 1]]
            greedy = float(g @ g)
            joint = min(float(((v[n].astype(np.float64) - cb[0, a] - cb[1, b]) ** 2).sum())
                        for a in range(8) for b in range(8))
            assert joint <= greedy + 1e-9
            # stage 1 is the exact nearest codeword of v
            d = [dist8_real(v[n], cb[0, j]) for j in range(8)]
            assert float(d[idx[n, 0]] - min(d)) <= _bound(min(d))


def test_encode_matrix_uses_row_scale_and_residual_relay():
    rng = np.random.default_rng(8)
    cb = _separated_codebooks(rng)
    truth = rng.integers(0, 16, size=(4, 16, 3))
    v = (cb[0][truth[..., 0]] + cb[1][truth[..., 1]] + cb[2][truth[..., 2]]).reshape(4, 128)
    # rows whose RMS is an exact power of two times v's: scale by s_r = fp16 RMS(v_r) * 2^k
    idx, s = oracle.encode(v, cb)
    sv = np.array([oracle.f16_bits_to_f32(int(x)) for x in s], dtype=np.float32)
    vn = (v / sv[:, None]).astype(np.float32).reshape(-1, 8)
    assert np.array_equal(idx.reshape(-1, 3), oracle.encode_vectors(vn, cb))
    # an all-zero row encodes like the zero vector
    z = np.zeros((1, 16), np.float32)
    idxz, sz = oracle.encode(z, cb)
    assert sz[0] == 0 and np.array_equal(idxz[0], oracle.encode_vectors(np.zeros((2, 8), np.float32), cb))


# ------------------------------------------------------------- decode
def test_decode_one_hot_and_order():
    K = 16
    cb = np.zeros((3, K, 8), np.float32)
    for t in range(3):
        for j in range(K):
            cb[t, j, j % 8] = np.float32(2.0 ** (j // 8 + 4 * t))
    idx = np.array([[[1, 9, 3]]], dtype=np.int32)
    s = np.array([np.float16(2.0).view(np.uint16)], dtype=np.uint16)
    w = oracle.decode(idx, s, cb)
    expect = np.zeros(8, np.float32)
    expect[1] += 1
    expect[1] += 2.0 ** 5
    expect[3] += 2.0 ** 8
    assert np.array_equal(w[0], 2 * expect)
    # left-to-right fp32 sum: (1 + 2^-24) + 2^-24 == 1, whereas 1 + (2^-24 + 2^-24) != 1
    cb2 = np.zeros((3, 2, 8), np.float32)
    cb2[0, 0, :] = 1.0
    cb2[1, 0, :] = 2.0 ** -24
    cb2[2, 0, :] = 2.0 ** -24
    w2 = oracle.decode(np.zeros((1, 1, 3), np.int32), np.array([0x3C00], np.uint16), cb2)
    assert np.all(w2 == 1.0)
    # partial reconstruction after 2 stages
    w3 = oracle.decode(idx, s, cb, stages_used=2)
    assert np.array_equal(w3[0], 2 * (expect - np.eye(8, dtype=np.float32)[3] * 2.0 ** 8))


def test_decode_inverts_exact_encode():
    rng = np.random.default_rng(9)
    cb = _separated_codebooks(rng)
    truth = rng.integers(0, 16, size=(3, 4, 3)).astype(np.int32)
    s = np.full(3, np.float16(0.5).view(np.uint16), dtype=np.uint16)
    w = oracle.decode(truth, s, cb)
    v = (cb[0][truth[..., 0]] + cb[1][truth[..., 1]] + cb[2][truth[..., 2]]) * np.float32(0.5)
    assert np.array_equal(w, v.reshape(3, 32))


# ------------------------------------------------------------- Lloyd
def test_fixed_point_bits_closed_form():
    assert oracle.fixed_point_bits(1.0, 1) == 61      # 1.0 < 2^1
    assert oracle.fixed_point_bits(0.75, 1024) == 52  # 0.75 < 2^0, ceil log2 1024 = 10
    assert oracle.fixed_point_bits(1.0, 1025) == 50
    assert oracle.fixed_point_bits(84.0, 22020096) == 62 - 7 - 25


def test_lloyd_n_equals_k_gives_zero_residual():
    rng = np.random.default_rng(10)
    R = rng.standard_normal((32, 8)).astype(np.float32)
    C, a, obj, res = oracle.lloyd_on_vectors(R, 32, 3, np.arange(32)[::-1].copy())
    assert np.array_equal(np.sort(a), np.arange(32))
    assert np.all(res == 0)
    assert obj[-1] == 0


def test_lloyd_two_separated_clusters_exact_means():
    rng = np.random.default_rng(11)
    # dyadic points (multiples of 2^-6) around +10 and -10: the fixed-point sums are exact
    A = np.float32(10) + np.round(rng.standard_normal((37, 8)) * 64) / np.float32(64)
    B = np.float32(-10) + np.round(rng.standard_normal((23, 8)) * 64) / np.float32(64)
    R = np.concatenate([A, B]).astype(np.float32)
    C, a, obj, res = oracle.lloyd_on_vectors(R, 2, 4, np.array([5, 40]))
    assert np.array_equal(a, np.r_[np.zeros(37, int), np.ones(23, int)])
    for j, P in enumerate([A, B]):
        for k in range(8):
            exact = sum(frac(x) for x in P[:, k]) / len(P)
            got = frac(C[j, k])
            assert abs(got - exact) <= abs(exact) * Fraction(1, 2 ** 23)
            assert C[j, k] == round_fp32(exact) or abs(got - exact) * 2 ** 24 <= abs(exact)
    # residual = point - its centroid
    assert np.array_equal(res, (R - C[a]).astype(np.float32))


def test_lloyd_empty_cluster_keeps_centroid():
    R = np.zeros((10, 8), np.float32)
    R[:5, 0] = 1
    R[5:, 0] = -1
    # init 0 and 1 hold the same value: cluster 1 loses every tie, stays empty
    # through the updates and keeps its initial centroid
    C, a, obj, res = oracle.lloyd_on_vectors(R, 3, 3, np.array([0, 1, 5]))
    assert not np.any(a == 1)
    assert np.array_equal(C[1], R[1])
    assert np.array_equal(a, np.r_[np.zeros(5, int), 2 * np.ones(5, int)])


def test_lloyd_objective_non_increasing():
    rng = np.random.default_rng(12)
    R = (rng.standard_normal((3000, 8)) * rng.standard_normal((3000, 1))).astype(np.float32)
    init = rng.choice(3000, 32, replace=False)
    C, a, obj, res = oracle.lloyd_on_vectors(R, 32, 12, init)
    assert np.all(np.diff(obj) <= 1e-6 * obj[:-1])
    # the centroids after update n are the means (to fp32 rounding) of the clusters
    # of the assignment made with the centroids of update n-1; empty ones are kept
    Cp, ap, _, _ = oracle.lloyd_on_vectors(R, 32, 11, init)
    for j in range(32):
        m = ap == j
        if m.any():
            assert np.allclose(C[j], R[m].astype(np.float64).mean(0), rtol=1e-6, atol=1e-6)
        else:
            assert np.array_equal(C[j], Cp[j])


def test_fit_stage_energy_non_increasing_and_codebook_shapes():
    rng = np.random.default_rng(13)
    mats = [(rng.standard_normal((16, 64)) * np.exp(0.5 * rng.standard_normal((16, 1)))).astype(np.float32)
            for _ in range(2)]
    n = 2 * 16 * 8
    init = np.stack([rng.choice(n, 16, replace=False) for _ in range(3)])
    cb, out = oracle.fit(mats, 3, 16, 5, init, want_assign=True, want_obj=True, want_energy=True)
    e = out["energy"]
    assert cb.shape == (3, 16, 8)
    assert np.all(np.diff(e) <= 1e-6 * e[:-1])
    assert e[3] < e[0]
    # the final residual energy equals the error of encoding the training vectors
    # with the fitted codebooks (the greedy encode and the fit's last assignment agree)
    idx_all = np.concatenate([oracle.encode(m, cb)[0].reshape(-1, 3) for m in mats])
    assert np.array_equal(idx_all, out["assign"].T)


def test_fit_rejects_bad_init():
    m = [np.ones((4, 16), np.float32)]
    with pytest.raises(oracle.OracleError):
        oracle.fit(m, 1, 4, 1, np.array([[0, 1, 1, 2]]))
    with pytest.raises(oracle.OracleError):
        oracle.fit(m, 1, 4, 1, np.array([[0, 1, 2, 8]]))


# ------------------------------------------------------------- error metric
def test_rel_error_closed_forms():
    rng = np.random.default_rng(14)
    w = rng.standard_normal((4, 16)).astype(np.float32)
    assert oracle.rel_error(w, np.zeros_like(w)) == 1.0
    assert oracle.rel_error(w, w) == 0.0
    assert abs(oracle.rel_error(w, 0.5 * w) - 0.5) < 1e-15
    assert abs(oracle.rel_error(np.float32([[3, 4]]), np.float32([[0, 4]])) - 0.6) < 1e-15


def test_error_sums_closed_forms():
    # (sum (w - w_hat)^2, sum w^2): both sums exact on dyadic values
    w = np.float32([[3, 4], [1, -2]])
    assert oracle.error_sums(w, np.zeros_like(w)) == (30.0, 30.0)
    assert oracle.error_sums(w, w) == (0.0, 30.0)
    # the second sum is over w, not w_hat: swapping the operands changes it
    a, b = np.float32([[1, 1]]), np.float32([[2, 2]])
    assert oracle.error_sums(a, b) == (2.0, 2.0)
    assert oracle.error_sums(b, a) == (2.0, 8.0)
    # constant rows: n d^2 and n c^2
    n, c, d = 1000, 0.75, 0.125
    w = np.full((10, 100), c, np.float32)
    assert oracle.error_sums(w, w - np.float32(d)) == (n * d * d, n * c * c)
    # every element contributes once (no dropped row or column): a single
    # nonzero difference anywhere gives exactly its square
    rng = np.random.default_rng(3)
    for _ in range(20):
        w = np.zeros((7, 9), np.float32)
        w_hat = np.zeros_like(w)
        r, k = rng.integers(7), rng.integers(9)
        w_hat[r, k] = np.float32(-1.5)
        assert oracle.error_sums(w, w_hat) == (2.25, 0.0)


def _gemv_exact(W, x):
    """y and sum_k |W_rk x_k| in exact rational arithmetic."""
    y, s = [], []
    for row in np.asarray(W, dtype=np.float64):
        y.append(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(row, x)))
        s.append(sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(row, x)))
    return y, s


def test_gemv_ref_closed_forms():
    # one-hot rows: y_r = a_r x_{c_r}, and the condition scale is |a_r x_{c_r}|
    rng = np.random.default_rng(5)
    rows, cols = 12, 40
    W = np.zeros((rows, cols), np.float32)
    cr = rng.integers(0, cols, rows)
    a = (rng.integers(-64, 64, rows) / 16.0).astype(np.float32)
    W[np.arange(rows), cr] = a
    x = (rng.integers(-32, 32, cols) / 8.0).astype(np.float32)
    y, s = oracle.gemv_ref(W, x)
    assert np.array_equal(y, a.astype(np.float64) * x[cr])
    assert np.array_equal(s, np.abs(a.astype(np.float64) * x[cr]))
    # rank one u v^T: y = u (v . x), scale = |u| sum |v x|; dyadic values keep fp64 exact
    u = (rng.integers(-8, 8, rows) / 4.0).astype(np.float32)
    v = (rng.integers(-8, 8, cols) / 2.0).astype(np.float32)
    y, s = oracle.gemv_ref(np.outer(u, v).astype(np.float32), x)
    vx = sum(Fraction(float(p)) * Fraction(float(q)) for p, q in zip(v, x))
    avx = sum(abs(Fraction(float(p)) * Fraction(float(q))) for p, q in zip(v, x))
    assert [Fraction(t) for t in y] == [Fraction(float(t)) * vx for t in u]
    assert [Fraction(t) for t in s] == [abs(Fraction(float(t))) * avx for t in u]
    # cancellation: y = 0 while the scale keeps every term
    y, s = oracle.gemv_ref(np.float32([[1, -1, 2, -2]]), np.float32([1, 1, 0.5, 0.5]))
    assert y[0] == 0.0 and s[0] == 4.0
    # a non-square matrix against brute force in exact arithmetic (catches a
    # transposed operand or a dropped row/column)
    W = (rng.integers(-100, 100, (5, 13)) / 32.0).astype(np.float32)
    x = (rng.integers(-100, 100, 13) / 64.0).astype(np.float32)
    y, s = oracle.gemv_ref(W, x)
    ye, se = _gemv_exact(W, x)
    assert [Fraction(t) for t in y] == ye and [Fraction(t) for t in s] == se


def test_gemv_ref_within_fp64_rounding_of_exact_on_random_inputs():
    # general fp32 inputs: the fp64 result is within n * 2^-53 * sum |w x| of the
    # exact rational value (the textbook bound for a length-n fp64 dot product
    # of exactly representable products)
    rng = np.random.default_rng(6)
    W = rng.standard_normal((6, 300)).astype(np.float32)
    x = rng.standard_normal(300).astype(np.float16).astype(np.float32)
    y, s = oracle.gemv_ref(W, x)
    ye, se = _gemv_exact(W, x)
    for r in range(6):
        assert abs(Fraction(float(y[r])) - ye[r]) <= Fraction(300, 2 ** 53) * se[r]
        assert abs(Fraction(float(s[r])) - se[r]) <= Fraction(300, 2 ** 53) * se[r]


# ------------------------------------------------------------- RTN
def test_rtn_grid_exact_and_ties():
    sc = np.float32(np.float16(0.03125))
    q = np.array([[7, -7, 3, 0, -1, 2, 5, -4] * 8], dtype=np.float32)
    w = (q * sc).astype(np.float32)
    w_hat, bpw = oracle.rtn(w, 4, 64)
    assert np.array_equal(w_hat, w) and bpw == 4.25
    # ties to even: w/sc = 0.5, 1.5, 2.5, -2.5 -> 0, 2, 2, -2 (with amax 7*sc fixing sc)
    w = np.array([[7, 0.5, 1.5, 2.5, -2.5, 0, 0, 0]], dtype=np.float32) * sc
    w_hat, _ = oracle.rtn(w, 4, 8)
    assert np.array_equal(w_hat / sc, np.float32([[7, 0, 2, 2, -2, 0, 0, 0]]))
    # a zero group reconstructs to zero; clamp at qmax
    w_hat, _ = oracle.rtn(np.zeros((1, 8), np.float32), 3, 8)
    assert np.all(w_hat == 0)


def test_rtn_bits_per_weight_match_gate3_table():
    rows = {r["scheme"]: r["bpw"] for r in GOLDEN["gate3_table"]["rows"]}
    w = np.ones((2, 2048), np.float32)
    assert oracle.rtn(w, 2, 64)[1] == rows["rtn2-g64"]
    assert oracle.rtn(w, 3, 64)[1] == rows["rtn3-g64"]
    assert round(oracle.rtn(w, 4, None)[1], 2) == rows["rtn4-row"]          # rows of 2048
    k3 = {r["scheme"]: r["bpw"] for r in GOLDEN["k3_gate3_table"]["rows"]}
    assert round(oracle.rtn(np.ones((1, 7168), np.float32), 4, None)[1], 2) == k3["rtn4-row"]  # K3 w1 rows


# ------------------------------------------------------------- MXFP4
def test_mxfp4_values_round_trip_and_rounding():
    for e in (-10, 0, 5):
        X = np.float32(2.0 ** e)
        vals = np.concatenate([oracle.E2M1_VALUES, -oracle.E2M1_VALUES])
        blk = np.zeros(32, np.float32)
        blk[:16] = vals * X
        blk[16] = 6 * X        # amax 6X -> floor(log2) = e + 2 -> scale X
        out = oracle.mxfp4_qdq(blk[None, :])
        assert np.array_equal(out[0], blk)
    X = np.float32(1.0)
    blk = np.zeros(32, np.float32)
    blk[:8] = [4, 5, 2.5, 0.25, 0.75, 1.25, 1.75, 3.5]
    out = oracle.mxfp4_qdq(blk[None, :])[0]
    assert np.array_equal(out[:8], np.float32([4, 4, 2, 0, 1, 1, 2, 4]))
    blk[0] = 7          # amax 7 -> X = 1, 7 saturates to 6
    assert oracle.mxfp4_qdq(blk[None, :])[0][0] == 6
    assert np.all(oracle.mxfp4_qdq(np.zeros((2, 64), np.float32)) == 0)


def test_mxfp4_results_are_exact_in_bf16():
    """Every MXFP4 result (a power-of-two block scale times an E2M1 value) has at
    most two significant bits and is at least 2^-128 in magnitude, so its fp32
    bits end in 16 zero bits: bf16 (the upper half) holds it exactly. Blocks with
    amax across the whole finite fp32 range, subnormal and near-overflow ones
    included."""
    rng = np.random.default_rng(12)
    rows = []
    for e in list(range(-149, 128, 3)) + [127, -126, -127, -128, -133, -140]:
        blk = (rng.standard_normal(32) * 2.0 ** rng.uniform(-24, 0, 32)).astype(np.float64)
        blk[0] = np.sign(blk[0]) * 1.9375
        blk = (blk * 2.0 ** e).astype(np.float32)
        rows.append(np.nan_to_num(blk, posinf=3.4e38, neginf=-3.4e38))
    W = np.stack(rows).astype(np.float32)
    W[-1, :] = np.float32(3.4028235e38) * np.sign(rng.standard_normal(32)).astype(np.float32)   # largest finite
    out = oracle.mxfp4_qdq(W)
    bits = out.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    nz = out[out != 0]
    assert nz.size > 0 and np.abs(nz).min() >= 2.0 ** -128
    assert np.isfinite(out).all() and np.abs(out).max() <= 1.5 * 2.0 ** 127
    # the round trip through bf16 words is the identity
    back = (bits >> 16).astype(np.uint32) << 16
    assert np.array_equal(back.view(np.float32), out)


def test_mxfp4_bits_per_weight_match_pages():
    # 4-bit elements + one 8-bit scale per 32 = 4.25 bits/weight: the K3 release
    # format row of the §1 table and the 190 MB lab fetch of §3.3
    bpw = 4 + 8 / 32
    assert bpw == GOLDEN["k3_record_table"]["rows"][2]["bpw"]
    d = GOLDEN["deepseek_lab_fetch"]
    r, c = d["reading_matrix_shape"]
    mb = d["experts"] * 3 * r * c * bpw / 8 / 1e6
    assert abs(mb - d["MB"]) / d["MB"] < 0.03


# ------------------------------------------------------------- records / sizes
def test_vq4p_pack_exhaustive_round_trip():
    g = np.arange(64, dtype=np.uint8)
    idx = np.stack(np.meshgrid(g, g, g, g, indexing="ij"), axis=-1).reshape(-1, 4)
    rec = oracle.pack_vq4p(idx)
    assert rec.shape == (64 ** 4, 3)
    assert np.array_equal(oracle.unpack_vq4p(rec), idx.astype(np.int32))
    # all 2^24 byte patterns are distinct records
    word = rec[:, 0].astype(np.uint32) | (rec[:, 1].astype(np.uint32) << 8) | (rec[:, 2].astype(np.uint32) << 16)
    assert len(np.unique(word)) == 64 ** 4
    assert list(oracle.pack_vq4p(np.array([1, 2, 3, 4]))) == [0x81, 0x30, 0x10]


def test_record_sizes_match_pages():
    g = GOLDEN
    assert g["vq3r_recipe"]["index_bits"] * g["vq3r_recipe"]["stages"] / g["vq3r_recipe"]["dim"] == 3.0
    assert g["vq4p_recipe"]["index_bits"] * g["vq4p_recipe"]["stages"] / g["vq4p_recipe"]["dim"] == 3.0
    assert oracle.pack_vq3r(np.zeros((5, 3), int)).nbytes == oracle.pack_vq4p(np.zeros((5, 4), int)).nbytes == 15
    assert 256 * 8 * 4 == g["codebook_bytes"]["bytes"]
    t = g["k3_record_table"]
    r, c = t["reading_matrix_shape"]
    n = t["reading_matrices_per_record"] * r * c
    scales = t["reading_matrices_per_record"] * r * 2
    vq2 = n // 8 * 2 + scales                  # two stage bytes per vector
    vq3 = oracle.pack_vq3r(np.zeros((1, 3), int)).nbytes * n // 8 + scales
    mx = n * 4.25 / 8
    for (bytes_, row) in zip([vq2, vq3, mx], t["rows"]):
        assert round(bytes_ / 1e6, 1) == row["record_MB"]
    # bits per weight including the row scales: 2.003 and 3.003, printed as 2.01 and 3.01
    # (the printed values agree with rounding up to two decimals)
    assert math.ceil((vq2 * 8 / n) * 100) / 100 == t["rows"][0]["bpw"]
    assert math.ceil((vq3 * 8 / n) * 100) / 100 == t["rows"][1]["bpw"]

"""Host emulation of the relative-error kernel's fp32 arithmetic (CPU only).

The error kernel (vq_decode.hip, k_error) does not re-form the decoded weights
w_hat_t = fp32(s * fp32 partial sums of codewords) for each stage. It carries
the difference from stage to stage, d_t = fma(-s, C_t[i_t], d_(t-1)) with
d_(-1) = w, sums each 8-weight vector's d_t^2 and w^2 in fp32 (a product, then
fused multiply-adds) and adds those vector sums in fp64. Its comment bounds the
effect on a matrix's ratio ||W - W_hat_t||_F / ||W||_F ([VQ3R page] §3.1) at
about 7 * 2^-24 in absolute terms plus 4 * 2^-24 of the ratio.

These tests emulate that arithmetic in numpy (a fused multiply-add as the fp64
product-sum of fp32 operands rounded once to fp32: exact but for rare double
roundings, each within one fp32 ulp) and compare it with the oracle's fp64
metric on the oracle's decoded weights. The inputs are heavy-tailed rows at
three magnitudes, rows that are themselves decoded weights, and codebooks
whose first two stages cancel (partial sums far larger than the weights). A
formulation mistake (restarting from w at each stage, a wrong sign, a dropped
stage) moves the ratios by orders of magnitude more than the bound.
"""
import numpy as np
import pytest

import oracle
import synthetic

F32 = np.float32
ULP24 = 2.0 ** -24


def _fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F32)


def _vector_sums(x):
    """Per 8-element vector: x0*x0, then fused multiply-adds, in fp32."""
    e = (x[..., 0].astype(np.float64) * x[..., 0]).astype(F32)
    for k in range(1, 8):
        e = _fma32(x[..., k], x[..., k], e)
    return e


def kernel_ratios(W, idx, s_bits, cb):
    """The kernel's ratios after each stage (fp32 fast path)."""
    rows, cols = W.shape
    V, S = cols // 8, cb.shape[0]
    s = s_bits.view(np.float16).astype(F32)
    w = W.reshape(rows, V, 8).astype(F32)
    neg_s = np.broadcast_to(-s[:, None, None], w.shape).astype(F32)
    sum_w = _vector_sums(w).astype(np.float64).sum()
    d = w
    out = []
    for t in range(S):
        d = _fma32(neg_s, cb[t][idx[:, :, t]], d)
        out.append(float(np.sqrt(_vector_sums(d).astype(np.float64).sum() / sum_w)))
    return out


def oracle_ratios(W, idx, s_bits, cb):
    return [oracle.rel_error(W, oracle.decode(idx, s_bits, cb, stages_used=t + 1)) for t in range(cb.shape[0])]


@pytest.fixture(scope="module")
def fitted():
    W = synthetic.student_t_rows_f32(128, 1024, seed=5)
    init = synthetic.forgy_init(128 * 128, 256, 3, seed=1)
    cb, _ = oracle.fit([W], 3, 256, 5, init)
    return W, cb


def _check(W, cb):
    idx, s_bits = oracle.encode(W, cb)
    k = kernel_ratios(W, idx, s_bits, cb)
    o = oracle_ratios(W, idx, s_bits, cb)
    for t, (a, b) in enumerate(zip(k, o)):
        assert abs(a - b) <= 7 * ULP24 + 4 * ULP24 * b, (t, a, b)
    return k, o


@pytest.mark.parametrize("scale", [1.0, 1e5, 1e-3])
def test_carried_difference_heavy_tailed_rows(fitted, scale):
    W, cb = fitted
    _check((W * F32(scale)).astype(F32), cb)


def test_carried_difference_on_decoded_weights(fitted):
    """Rows that are decoded weights themselves (small errors after 3 stages)."""
    W, cb = fitted
    idx, s_bits = oracle.encode(W, cb)
    _check(oracle.decode(idx, s_bits, cb), cb)


def test_carried_difference_cancelling_stages(fitted):
    """Stage-1 and stage-2 codewords that cancel: partial sums about 30x the
    weights, so the first stage's difference dwarfs w."""
    W, cb = fitted
    rng = np.random.default_rng(1)
    big = (rng.standard_normal((256, 8)) * 30).astype(F32)
    cbc = cb.copy()
    cbc[0] = cb[0] + big
    cbc[1] = cb[1] - big[rng.permutation(256)]
    k, o = _check(W, cbc)
    assert o[0] > 5.0  # the first stage alone is far off


def test_a_dropped_stage_is_caught(fitted):
    """The check distinguishes a wrong formulation: restarting each stage's
    difference from w (dropping the earlier stages) misses by far more than
    the bound."""
    W, cb = fitted
    idx, s_bits = oracle.encode(W, cb)
    o = oracle_ratios(W, idx, s_bits, cb)
    rows, cols = W.shape
    s = s_bits.view(np.float16).astype(F32)
    w = W.reshape(rows, cols // 8, 8)
    neg_s = np.broadcast_to(-s[:, None, None], w.shape).astype(F32)
    d = _fma32(neg_s, cb[2][idx[:, :, 2]], w)  # stage 3 alone
    wrong = float(np.sqrt(_vector_sums(d).astype(np.float64).sum() / _vector_sums(w).astype(np.float64).sum()))
    assert abs(wrong - o[2]) > 1e3 * (7 * ULP24 + 4 * ULP24 * o[2])

"""The Lloyd assign kernel accumulates llrint(r 2^F) for each coordinate r with
one fp64 fma, x = r 2^F + 1.5 2^52, taking the integer from the bit pattern:
bits(x) - bits(1.5 2^52) == llrint(r 2^F) (ties to even) whenever
|r 2^F| < 2^51. The product r 2^F is exact, so the fma's single rounding is
the rounding of one fp64 addition, which numpy performs here."""
import numpy as np

BIAS = np.float64(1.5 * 2.0 ** 52)
BIAS_BITS = np.int64(0x4338000000000000)


def _biased(v):
    x = v + BIAS  # v = r 2^F exactly; one rounding, as the fma's
    return x.view(np.int64) - BIAS_BITS


def test_bias_constant():
    assert np.array([BIAS]).view(np.int64)[0] == BIAS_BITS


def test_biased_conversion_equals_llrint():
    rng = np.random.default_rng(11)
    r = rng.standard_normal(2_000_000).astype(np.float32)
    for F in (16, 24, 30, 37, 44, 48):
        v = r.astype(np.float64) * np.float64(2.0 ** F)
        ok = np.abs(v) < 2.0 ** 51
        np.testing.assert_array_equal(_biased(v[ok]), np.rint(v[ok]).astype(np.int64))


def test_ties_and_range_edges():
    # exact halves round to even; the largest magnitudes below 2^51
    v = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.0, -0.0, 1e-300, -1e-300,
                  2.0 ** 51 - 0.5, -(2.0 ** 51) + 0.5, 2.0 ** 51 - 1, -(2.0 ** 51) + 1, 12345.5, -12345.5])
    np.testing.assert_array_equal(_biased(v), np.rint(v).astype(np.int64))


def test_modular_sum_then_bias_removal():
    # the block adds bit patterns mod 2^64 and subtracts count * bits(bias) once
    rng = np.random.default_rng(5)
    v = np.rint(rng.standard_normal(100_000) * 2.0 ** 40)
    pats = (v + BIAS).view(np.uint64)
    with np.errstate(over="ignore"):
        total = np.add.reduce(pats, dtype=np.uint64) - np.uint64(len(v)) * np.uint64(BIAS_BITS)
    assert np.int64(total.astype(np.int64)) == np.int64(v.astype(np.int64).sum())

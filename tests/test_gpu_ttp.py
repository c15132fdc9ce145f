"""Tied Trit-Planes codec ([TTP page]) on the GPU against the oracle: codes
and fp16 scales bit-exact, dequantized weights bit-exact, error sums within
1e-5 of the oracle's relative error and independent of batching."""
import sys

import numpy as np
import pytest

import oracle
import synthetic

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import residual_vector_quantization_amd as vq  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _inputs(dtype, rows, cols, seed):
    if dtype == "bf16":
        bits = synthetic.student_t_rows_bf16(rows, cols, seed=seed)
        return synthetic.bf16_bits_to_f32(bits).reshape(rows, cols), to_dev(bits.view(np.int16)).view(torch.bfloat16)
    w = synthetic.student_t_rows_f32(rows, cols, seed=seed)
    if dtype == "f16":
        h = w.astype(np.float16)
        return h.astype(np.float32), to_dev(h)
    return w, to_dev(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("rows,cols", [(16, 1024), (3, 256), (130, 7168)])
def test_ttp_bit_exact(dtype, rows, cols):
    say("ttp", dtype, rows, cols)
    wf, wd = _inputs(dtype, rows, cols, seed=rows + cols)
    c, s = vq.ttp_quantize(wd)
    c_o, s_o = oracle.ttp_quantize(wf)
    assert np.array_equal(c.cpu().numpy(), c_o)
    assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), s_o)
    assert np.array_equal(vq.ttp_dequantize(c, s).cpu().numpy(), oracle.ttp_dequantize(c_o, s_o))


def test_ttp_special_groups():
    say("ttp special groups")
    w = np.zeros((4, 512), np.float32)
    w[1, :256] = 0.3                                  # constant group
    w[2, :256] = np.float32(0.125) * np.resize(np.arange(-4, 5), 256)   # exact grid
    w[3] = synthetic.student_t_rows_f32(1, 512, seed=9)[0]
    w[3, 256:] *= 1e-30                               # tiny values (fp16-subnormal scale)
    c, s = vq.ttp_quantize(to_dev(w))
    c_o, s_o = oracle.ttp_quantize(w)
    assert np.array_equal(c.cpu().numpy(), c_o)
    assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), s_o)


def test_ttp_flags_non_finite():
    say("ttp non-finite")
    w = np.zeros((1, 256), np.float32)
    w[0, 3] = np.nan
    with pytest.raises(vq.VQError):
        vq.ttp_quantize(to_dev(w))


def test_ttp_full_expert_and_error():
    say("ttp full expert")
    wf, wd = _inputs("bf16", 2048, 7168, seed=77)
    c, s = vq.ttp_quantize(wd)
    c_o, s_o = oracle.ttp_quantize(wf)
    assert np.array_equal(c.cpu().numpy(), c_o)
    assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), s_o)
    sums = vq.ttp_error_sums(wd, c, s).cpu().numpy()[0]
    ref = oracle.rel_error(wf, oracle.ttp_dequantize(c_o, s_o))
    assert abs(np.sqrt(sums[0] / sums[1]) - ref) <= 1e-5
    rtn = oracle.rel_error(wf, oracle.rtn(wf, 4, None)[0])
    say("  rel error ttp %.4f  rtn4-row %.4f" % (ref, rtn))


def test_ttp_error_does_not_depend_on_batching():
    say("ttp error batching")
    wf, wd = _inputs("bf16", 3 * 200, 768, seed=78)
    c, s = vq.ttp_quantize(wd)
    both = vq.ttp_error_sums(wd, c, s, n_mats=3)
    for m in range(3):
        r = slice(200 * m, 200 * (m + 1))
        assert torch.equal(vq.ttp_error_sums(wd[r], c[r], s[r])[0], both[m])


def test_ttp_half_integer_quotients():
    """Weights at and just beside half-integer multiples of the starting scale
    a = max|w| / 4: the nearest level of the rounded quotient is a tie (to
    even) or a near tie, where a level taken from the reciprocal of the scale
    could differ; codes and scales must still be the oracle's."""
    say("ttp half-integer quotients")
    a0 = np.float32(0.0371)
    half = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5], np.float32)
    rows = []
    for rel in (0.0, 2.0 ** -22, -(2.0 ** -22), 2.0 ** -19, -(2.0 ** -19)):
        w = np.resize(half * np.float32(1.0 + rel), 256).astype(np.float32) * a0
        w[0] = 4 * a0                              # sets max|w| = 4 a0
        rows.append(w)
    w = np.stack(rows).astype(np.float32)
    c, s = vq.ttp_quantize(to_dev(w))
    c_o, s_o = oracle.ttp_quantize(w)
    assert np.array_equal(c.cpu().numpy(), c_o)
    assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), s_o)


@pytest.mark.parametrize("seed", [0, 1])
def test_ttp_random_shapes(seed):
    """Seeded random cases: dtype, shape (1-40 rows, 256-4096 columns) and
    magnitude (10^-4 .. 10^3), with some all-zero and constant groups; codes
    and scales bit-exact."""
    say("ttp random sweep", seed)
    rng = np.random.default_rng(500 + seed)
    for case in range(20):
        dtype = ["f32", "bf16", "f16"][rng.integers(3)]
        rows, cols = int(rng.integers(1, 41)), 256 * int(rng.integers(1, 17))
        wf = (synthetic.student_t_rows_f32(rows, cols, seed=6000 + 50 * seed + case) *
              np.float32(10.0 ** rng.uniform(-4, 3))).astype(np.float32)
        if rng.random() < 0.3:
            wf[rng.integers(rows), :256] = 0.0
        if rng.random() < 0.3:
            wf[rng.integers(rows), :256] = np.float32(rng.uniform(-1, 1))
        if dtype == "bf16":
            bits = synthetic.f32_to_bf16_bits(wf)
            wd = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
            wf = synthetic.bf16_bits_to_f32(bits).reshape(rows, cols)
        elif dtype == "f16":
            wf = np.clip(wf, -60000, 60000).astype(np.float16).astype(np.float32)
            wd = to_dev(wf.astype(np.float16))
        else:
            wd = to_dev(wf)
        c, s = vq.ttp_quantize(wd)
        c_o, s_o = oracle.ttp_quantize(wf)
        tag = (case, dtype, rows, cols)
        assert np.array_equal(c.cpu().numpy(), c_o), tag
        assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), s_o), tag

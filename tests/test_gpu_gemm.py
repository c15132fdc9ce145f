"""The batched dequant-GEMM (prompt processing, many tokens per expert)
against the oracle: y = W_hat x in fp64 for every (token, slot) pair, within
1e-3 * sum_c |w_hat_c x_c| per output (the GEMV's bar; the kernel's own bound
is 2^-11 of it plus fp32 accumulation), on ragged and edge shapes and on the
full 256-expert layer."""
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


@pytest.fixture(scope="module")
def books():
    out = {}
    for fmt in ("vq3r", "vq4p"):
        S, K = vq.stages_entries(fmt)
        W = synthetic.student_t_rows_f32(256, 1024, seed=90)
        cb, _ = oracle.fit([W], S, K, 4, synthetic.forgy_init(256 * 128, K, S, seed=91))
        out[fmt] = cb
    return out


def _experts(fmt, cb, E, rows, cols, seed):
    recs, scs, whs = [], [], []
    for e in range(E):
        w = synthetic.student_t_rows_f32(rows, cols, seed=seed + e)
        i, s = oracle.encode(w, cb)
        recs.append(oracle.pack(fmt, i))
        scs.append(s)
        whs.append(oracle.decode(i, s, cb))
    return np.stack(recs), np.stack(scs), whs


def _check(y, whs, xf, route, sample=None):
    ntok, topk = route.shape
    pairs = [(b, k) for b in range(ntok) for k in range(topk)]
    if sample is not None:
        pairs = [pairs[i] for i in sample]
    worst = 0.0
    for b, k in pairs:
        ref, scale = oracle.gemv_ref(whs[route[b, k]], xf[b])
        err = np.abs(y[b, k] - ref)
        worst = max(worst, float((err / scale).max()))
        assert np.all(err <= 1e-3 * scale + 1e-30), (b, k, float((err / scale).max()))
        # and per output vector of at least 64 rows, relative L2 <= 1e-3: the fp16
        # codeword sums err by about 2^-11 / sqrt(3) of |w_hat x| per term with
        # random signs, so over many rows the ratio settles near 3e-4, while a
        # vector of a few rows can be dominated by one cancelling output
        nr = np.linalg.norm(ref)
        if nr > 0 and ref.shape[-1] >= 64:
            assert np.linalg.norm(y[b, k] - ref) <= 1e-3 * nr, (b, k)
    return worst


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("rows,cols,E,ntok,topk", [(256, 1024, 6, 300, 4), (100, 264, 5, 70, 3),
                                                   (130, 64, 3, 257, 2), (32, 8, 2, 5, 2), (1, 512, 4, 40, 4)])
def test_gemm_matches_oracle(books, fmt, rows, cols, E, ntok, topk):
    say("gemm", fmt, rows, cols, E, ntok, topk)
    cb = books[fmt]
    recs, scs, whs = _experts(fmt, cb, E, rows, cols, seed=70)
    x = synthetic.activations_f16(ntok, cols, seed=5)
    route = synthetic.routing(ntok, E, topk, seed=6)
    y = vq.dequant_gemm(to_dev(recs), to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                        to_dev(route), fmt=fmt).cpu().numpy()
    worst = _check(y, whs, synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)
    say("  worst error / sum|w x| = %.2e" % worst)
    assert worst < 2.0 ** -11 * 1.5


def test_gemm_skewed_routing_and_single_expert(books):
    """One expert gets 700 pairs (6 tiles, the last one partial), the others few."""
    say("gemm skewed")
    cb = books["vq3r"]
    rows, cols, E = 192, 512, 4
    recs, scs, whs = _experts("vq3r", cb, E, rows, cols, seed=80)
    ntok, topk = 700, 2
    route = np.zeros((ntok, topk), np.int32)
    route[:, 1] = np.arange(ntok) % 3 + 1
    x = synthetic.activations_f16(ntok, cols, seed=7)
    y = vq.dequant_gemm(to_dev(recs), to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                        to_dev(route)).cpu().numpy()
    _check(y, whs, synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)


def test_gemm_many_experts_global_counters(books):
    """9000 experts (more than the route kernel keeps in LDS), expert e holding
    base expert e % 2."""
    say("gemm 9000 experts")
    cb = books["vq3r"]
    rows, cols, E = 40, 64, 9000
    recs, scs, whs = _experts("vq3r", cb, 2, rows, cols, seed=88)
    idx = to_dev(recs).repeat(E // 2, 1, 1, 1)
    sc = to_dev(scs.view(np.float16)).repeat(E // 2, 1)
    ntok, topk = 600, 4
    route = synthetic.routing(ntok, E, topk, seed=12)
    x = synthetic.activations_f16(ntok, cols, seed=13)
    y = vq.dequant_gemm(idx, sc, to_dev(cb), to_dev(x.view(np.float16)), to_dev(route), check=True).cpu().numpy()
    _check(y, [whs[e % 2] for e in range(E)], synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)


def test_gemm_bad_route_and_empty(books):
    say("gemm bad route / empty")
    cb = books["vq3r"]
    recs, scs, whs = _experts("vq3r", cb, 2, 64, 128, seed=85)
    x = synthetic.activations_f16(3, 128, seed=8)
    route = np.array([[0, 7], [1, -1], [1, 0]], np.int32)
    args = (to_dev(recs), to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)), to_dev(route))
    with pytest.raises(vq.VQError):
        vq.dequant_gemm(*args, check=True)
    y = vq.dequant_gemm(*args).cpu().numpy()
    assert np.all(y[0, 1] == 0) and np.all(y[1, 1] == 0)
    good = route.copy()
    good[good < 0] = 0
    good[good > 1] = 0
    xf = synthetic.f16_bits_to_f32(x).reshape(3, 128)
    for b, k in [(0, 0), (1, 0), (2, 0), (2, 1)]:
        ref, scale = oracle.gemv_ref(whs[route[b, k]], xf[b])
        assert np.all(np.abs(y[b, k] - ref) <= 1e-3 * scale)
        assert np.linalg.norm(y[b, k] - ref) <= 1e-3 * np.linalg.norm(ref)
    y0 = vq.dequant_gemm(args[0], args[1], args[2], args[3][:0], args[4][:0], check=True)
    assert y0.shape == (0, 2, 64)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_gemm_full_layer_sampled(books, fmt):
    """256 experts of [2048 x 7168] (expert e = base expert e % 2), 2048 tokens
    top-8 (64 pairs per expert on average), the oracle checked on 48 pairs."""
    say("gemm full layer", fmt)
    rows, cols, E, ntok, topk = 2048, 7168, 256, 2048, 8
    cb = books[fmt]
    recs, scs, whs = _experts(fmt, cb, 2, rows, cols, seed=95)
    idx = to_dev(recs).repeat(E // 2, 1, 1, 1)
    sc = to_dev(scs.view(np.float16)).repeat(E // 2, 1)
    x = synthetic.activations_f16(ntok, cols, seed=9)
    route = synthetic.routing(ntok, E, topk, seed=10)
    y = vq.dequant_gemm(idx, sc, to_dev(cb), to_dev(x.view(np.float16)), to_dev(route), fmt=fmt)
    torch.cuda.synchronize()
    sample = np.random.default_rng(0).choice(ntok * topk, 48, replace=False)
    yh = y.cpu().numpy()
    _check(yh, [whs[e % 2] for e in range(E)], synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route, sample)


@pytest.mark.parametrize("seed", [0, 1])
def test_gemm_random_shapes(books, seed):
    """Seeded random cases: format, shape (1-299 rows, 8-1600 columns), 1-6
    experts, 1-199 tokens, top-1..4 routing; every pair within 1e-3 of
    sum |w_hat x|."""
    say("gemm random sweep", seed)
    rng = np.random.default_rng(300 + seed)
    for case in range(16):
        fmt = ["vq3r", "vq4p"][rng.integers(2)]
        cb = books[fmt]
        rows, cols = int(rng.integers(1, 300)), 8 * int(rng.integers(1, 201))
        E = int(rng.integers(1, 7))
        ntok, topk = int(rng.integers(1, 200)), int(rng.integers(1, min(E, 4) + 1))
        recs, scs, whs = _experts(fmt, cb, E, rows, cols, seed=4000 + 10 * case + seed)
        x = synthetic.activations_f16(ntok, cols, seed=case)
        route = synthetic.routing(ntok, E, topk, seed=7 + case)
        y = vq.dequant_gemm(to_dev(recs), to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                            to_dev(route), fmt=fmt).cpu().numpy()
        _check(y, whs, synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)

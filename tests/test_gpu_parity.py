"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded
synthetic inputs. Bars: indices, scales, decoded weights and MXFP4 values
bit-exact; Lloyd codebooks bit-exact; relative Frobenius error within 1e-5
absolute; GEMV within 1e-3 of sum_k |w_hat_k x_k| per output."""
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

DEV = "cuda"
ENGINES = ["mfma_f16x", "mfma_f32", "valu_f32", "exact"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.to(dtype)


def bf16_dev(bits):
    return to_dev(bits.view(np.int16)).view(torch.bfloat16)


def rec_to_idx(fmt, rec_dev):
    return oracle.unpack(fmt, rec_dev.cpu().numpy())


def scales_bits(s_dev):
    return s_dev.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(scope="module")
def cfg1():
    """256 x 1024 fp32, N(0,1) x per-row lognormal(0, 0.5), seed 0; codebooks from
    the oracle's Lloyd fit (10 iterations, Forgy init from the shared generator)."""
    W = synthetic.gaussian_rows(256, 1024, seed=0)
    out = {"W": W}
    for fmt in ("vq3r", "vq4p"):
        S, K = vq.stages_entries(fmt)
        init = synthetic.forgy_init(256 * 128, K, S, seed=0)
        cb, _ = oracle.fit([W], S, K, 10, init)
        out[fmt] = (init, cb)
    return out


# ------------------------------------------------------------------ encode
@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("engine", ENGINES)
def test_encode_cfg1_bit_exact(cfg1, fmt, engine):
    say("encode cfg1", fmt, engine)
    W = cfg1["W"]
    init, cb = cfg1[fmt]
    idx_o, s_o = oracle.encode(W, cb)
    rec, s = vq.encode(to_dev(W), to_dev(cb), fmt=fmt, engine=engine)
    torch.cuda.synchronize()
    assert np.array_equal(scales_bits(s), s_o)
    got = rec_to_idx(fmt, rec)
    mism = np.argwhere(np.any(got != idx_o, axis=-1))
    assert len(mism) == 0, "%d vectors differ, first %s" % (len(mism), mism[:5].tolist())


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("shape", [(1, 8), (3, 24), (5, 264), (7, 2056), (33, 512)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_encode_ragged_shapes_and_dtypes(cfg1, fmt, shape, dtype):
    say("encode ragged", fmt, shape, dtype)
    rows, cols = shape
    _, cb = cfg1[fmt]
    W = synthetic.gaussian_rows(rows, cols, seed=rows * 7 + cols)
    if dtype == "bf16":
        bits = synthetic.f32_to_bf16_bits(W)
        Wd = bf16_dev(bits)
        W = synthetic.bf16_bits_to_f32(bits).reshape(rows, cols)
    elif dtype == "f16":
        W = W.astype(np.float16).astype(np.float32)
        Wd = to_dev(W.astype(np.float16))
    else:
        Wd = to_dev(W)
    idx_o, s_o = oracle.encode(W, cb)
    rec, s = vq.encode(Wd, to_dev(cb), fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(scales_bits(s), s_o)
    assert np.array_equal(rec_to_idx(fmt, rec), idx_o)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_encode_near_ties_and_duplicates(cfg1, fmt):
    """Duplicate codewords (exact ties) and vectors placed on bisectors of
    codeword pairs: the certification must route them to the exact search."""
    say("encode near ties", fmt)
    S, K = vq.stages_entries(fmt)
    _, cb = cfg1[fmt]
    cb = cb.copy()
    rng = np.random.default_rng(11)
    for t in range(S):
        for q in range(K // 8):
            cb[t, rng.integers(K)] = cb[t, rng.integers(K)]
    # rows made of midpoints between two stage-1 codewords (times a row factor)
    rows, V = 64, 32
    a = rng.integers(0, K, size=(rows, V))
    b = rng.integers(0, K, size=(rows, V))
    mid = 0.5 * (cb[0][a] + cb[0][b])
    W = (mid.reshape(rows, V * 8) * rng.uniform(0.5, 2, size=(rows, 1))).astype(np.float32)
    idx_o, s_o = oracle.encode(W, cb)
    for engine in ENGINES[:3]:
        rec, s = vq.encode(to_dev(W), to_dev(cb), fmt=fmt, engine=engine)
        torch.cuda.synchronize()
        assert np.array_equal(scales_bits(s), s_o), engine
        assert np.array_equal(rec_to_idx(fmt, rec), idx_o), engine


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_encode_all_ties_overflows_queue_and_stays_exact(fmt):
    """Every codeword identical: every vector is a tie, the exact-pass queue
    overflows and the exact pass covers all vectors; answer = index 0."""
    say("encode all ties", fmt)
    S, K = vq.stages_entries(fmt)
    cb = np.zeros((S, K, 8), np.float32)
    cb[:] = np.float32(0.25)
    W = synthetic.gaussian_rows(512, 1024, seed=3)      # 65536 vectors > 16 * 4096
    rec, s = vq.encode(to_dev(W), to_dev(cb), fmt=fmt)
    ws = vq.encode_workspace(fmt, 512, 1024)
    rec, s = vq.encode(to_dev(W), to_dev(cb), fmt=fmt, workspace=ws)
    flags = vq.read_status(ws)
    assert flags & (1 << 8)     # the exact pass covered every vector
    assert np.all(rec_to_idx(fmt, rec) == 0)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("rows,cols", [(16, 2048), (8, 4096), (13, 1544)])
def test_encode_flag_list_complete(fmt, rows, cols):
    """Every vector a tie but the queue does not overflow: each wave stages 256+
    flagged ids in LDS and flushes them in batches. The list (after the 256-byte
    header, count in header word 1) must hold every vector id exactly once."""
    say("encode flag list", fmt, rows, cols)
    S, K = vq.stages_entries(fmt)
    cb = np.zeros((S, K, 8), np.float32)
    cb[:] = np.float32(0.25)
    W = synthetic.gaussian_rows(rows, cols, seed=4)
    nvec = rows * cols // 8
    assert nvec <= 4096                                  # the smallest queue capacity
    ws = vq.encode_workspace(fmt, rows, cols)
    rec, s = vq.encode(to_dev(W), to_dev(cb), fmt=fmt, workspace=ws)
    torch.cuda.synchronize()
    assert vq.read_status(ws) == 0
    words = ws[: 256 + 4 * nvec].cpu().numpy().view(np.uint32)
    assert int(words[1]) == nvec
    ids = np.sort(words[64:64 + nvec])
    assert np.array_equal(ids, np.arange(nvec, dtype=np.uint32))
    assert np.all(rec_to_idx(fmt, rec) == 0)


def test_encode_edge_rows_and_errors(cfg1):
    say("encode edge rows")
    _, cb = cfg1["vq3r"]
    W = synthetic.gaussian_rows(6, 64, seed=5)
    W[1] = 0.0                      # zero row: scale 0, vectors encoded as 0
    W[2] = 1e-30                    # RMS below fp16 range: scale 0
    W[3, :8] = 3e4                  # large row
    idx_o, s_o = oracle.encode(W, cb)
    rec, s = vq.encode(to_dev(W), to_dev(cb))
    torch.cuda.synchronize()
    assert np.array_equal(scales_bits(s), s_o)
    assert np.array_equal(rec_to_idx("vq3r", rec), idx_o)
    # a non-finite weight and an RMS beyond fp16 are data errors
    for bad in (np.nan, np.inf):
        Wb = W.copy()
        Wb[4, 7] = bad
        with pytest.raises(vq.VQError) as e:
            vq.encode(to_dev(Wb), to_dev(cb))
        assert e.value.status == 5
    Wb = np.full((2, 64), 1e5, np.float32)
    with pytest.raises(vq.VQError):
        vq.encode(to_dev(Wb), to_dev(cb))
    # codebook entries beyond |c| <= 2048 are rejected
    cbb = cb.copy()
    cbb[1, 3, 2] = 5000.0
    with pytest.raises(vq.VQError):
        vq.encode(to_dev(W), to_dev(cbb))
    # empty input
    rec, s = vq.encode(torch.empty((0, 64), device=DEV), to_dev(cb))
    assert rec.shape == (0, 8, 3)


def _normalization_edge_matrix():
    """48 x 64 fp32 rows where vectors leave the reciprocal normalization's
    range |w| in [2^-100, 2^100] (zeros, -0, fp32 subnormals, 2^-101) or sit on
    its edge (2^-100), rows with an fp16-subnormal scale, large rows."""
    W = synthetic.gaussian_rows(48, 64, seed=31)
    W[0, ::3] = 0.0
    W[0, 1::5] = -0.0
    W[1] = W[1] * np.float32(1e-6)                  # scale below fp16's normal range
    W[1, 3], W[1, 17], W[1, 40] = 1e-42, -1e-31, 2.0 ** -101
    W[2, 5], W[2, 6], W[2, 7] = 2.0 ** -100, -(2.0 ** -100), np.float32(2.0 ** -100) * np.float32(1 - 2 ** -24)
    W[2, 20], W[2, 21] = 2.0 ** -99, 2.0 ** -60
    W[3] = W[3] * np.float32(1e3)
    W[4, 8:16] = 0.0                                 # a whole zero vector
    W[5] = W[5] * np.float32(3e-8)                   # smallest fp16 subnormal scales
    return W.astype(np.float32)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_encode_and_fit_normalization_edges(cfg1, fmt):
    say("normalization edges", fmt)
    W = _normalization_edge_matrix()
    _, cb = cfg1[fmt]
    idx_o, s_o = oracle.encode(W, cb)
    rec, s = vq.encode(to_dev(W), to_dev(cb), fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(scales_bits(s), s_o)
    assert np.array_equal(rec_to_idx(fmt, rec), idx_o)
    S, K = vq.stages_entries(fmt)
    init = synthetic.forgy_init(48 * 8, K, S, seed=12)
    cb_o, _ = oracle.fit([W], S, K, 3, init)
    cb_g = vq.fit_codebooks([to_dev(W)], init, fmt=fmt, iters=3)
    assert np.array_equal(cb_g.cpu().numpy().view(np.uint32), cb_o.view(np.uint32))


def test_encode_deterministic(cfg1):
    say("encode determinism")
    _, cb = cfg1["vq3r"]
    Wd = to_dev(cfg1["W"])
    r1, s1 = vq.encode(Wd, to_dev(cb))
    r2, s2 = vq.encode(Wd, to_dev(cb))
    assert torch.equal(r1, r2) and torch.equal(s1.view(torch.int16), s2.view(torch.int16))


# ------------------------------------------------------------------ decode / error
@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_decode_bit_exact_and_error(cfg1, fmt):
    say("decode + error", fmt)
    S, _ = vq.stages_entries(fmt)
    W = cfg1["W"]
    _, cb = cfg1[fmt]
    idx_o, s_o = oracle.encode(W, cb)
    rec = to_dev(oracle.pack(fmt, idx_o))
    sd = to_dev(s_o.view(np.float16))
    cbd = to_dev(cb)
    for su in range(1, S + 1):
        got = vq.decode(rec, sd, cbd, fmt=fmt, stages_used=su).cpu().numpy()
        ref = oracle.decode(idx_o, s_o, cb, stages_used=su)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), su
    rel, rel_all, sums = vq.rel_errors(to_dev(W), rec, sd, cbd, fmt=fmt)
    e = rel.cpu().numpy()[0]
    sums = sums.cpu().numpy()[0]
    for su in range(1, S + 1):
        ref = oracle.rel_error(W, oracle.decode(idx_o, s_o, cb, stages_used=su))
        assert abs(e[su - 1] - ref) < 1e-5
        # the library's ratio is the correctly rounded sqrt(sum / sum) of its own sums
        assert e[su - 1] == np.sqrt(sums[su - 1] / sums[S])
    assert np.array_equal(rel_all.cpu().numpy(), e)  # one matrix: the aggregate is the same
    # error is non-increasing over the stages on the fit data
    assert np.all(np.diff(e) <= 1e-12)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_encode_decode_error_full_layer_sampled(cfg1, fmt):
    """The launches the benchmark times: the 256-expert layer of [2048 x 7168]
    bf16 (generated on the GPU as the benchmark does) encoded, decoded and
    measured in one call each. 64 sampled rows are checked bit-exact against
    the oracle (indices, scales, decoded weights); two whole experts' error
    sums against the oracle's relative error within 1e-5."""
    say("full layer encode/decode/error", fmt)
    E, R, C = 256, 2048, 7168
    S, _ = vq.stages_entries(fmt)
    _, cb = cfg1[fmt]
    W = torch.empty((E * R, C), dtype=torch.bfloat16, device=DEV)
    for e in range(E):
        synthetic.student_t_expert_torch(synthetic.expert_seed(3, e), R, C, device=DEV, out=W[e * R:(e + 1) * R])
    cbd = to_dev(cb)
    rec, sc = vq.encode(W, cbd, fmt=fmt)
    w_hat = vq.decode(rec, sc, cbd, fmt=fmt)
    rel_d, rel_all_d, sums_d = vq.rel_errors(W, rec, sc, cbd, fmt=fmt, n_mats=E)
    rel, rel_all, sums = rel_d.cpu().numpy(), rel_all_d.cpu().numpy(), sums_d.cpu().numpy()
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7).choice(E * R, 64, replace=False))
    rt = torch.from_numpy(rows).to(DEV)
    wf = W[rt].float().cpu().numpy()
    idx_o, s_o = oracle.encode(wf, cb)
    assert np.array_equal(rec_to_idx(fmt, rec[rt]), idx_o)
    assert np.array_equal(scales_bits(sc[rt]), s_o)
    assert np.array_equal(w_hat[rt].cpu().numpy().view(np.uint32), oracle.decode(idx_o, s_o, cb).view(np.uint32))
    del w_hat
    for e in (5, 201):
        we = W[e * R:(e + 1) * R].float().cpu().numpy()
        i_e, s_e = oracle.encode(we, cb)
        for su in range(1, S + 1):
            ref = oracle.rel_error(we, oracle.decode(i_e, s_e, cb, stages_used=su))
            assert abs(rel[e, su - 1] - ref) <= 1e-5, (e, su)
    # the aggregate over the layer: ratio of the summed sums, in matrix order
    tot = np.zeros(S + 1)
    for m in range(E):
        tot = tot + sums[m]
    assert np.array_equal(rel_all, np.sqrt(tot[:S] / tot[S]))


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_decode_ragged_rows_and_unaligned_records(cfg1, fmt):
    """The decoder works on chunks of 256 consecutive vectors. Covered here:
    rows of 13 vectors (several rows per chunk), rows of 256, 257 and 512
    vectors (chunk starts inside a row), a ragged last chunk, a matrix smaller
    than one chunk, records starting at an odd byte address (byte-wise record
    loads), and the partial reconstructions of the aligned cases. All must stay
    bit-exact."""
    say("decode ragged / unaligned", fmt)
    S, _ = vq.stages_entries(fmt)
    _, cb = cfg1[fmt]
    cbd = to_dev(cb)
    for rows, cols, offset in ((37, 104, 0), (16, 256, 1), (5, 104, 3), (300, 2056, 0), (9, 2048, 2), (9, 2048, 0),
                               (41, 4096, 0), (1, 2056, 0)):
        W = synthetic.student_t_rows_f32(rows, cols, seed=rows + cols)
        idx_o, s_o = oracle.encode(W, cb)
        packed = oracle.pack(fmt, idx_o).reshape(-1)
        buf = torch.zeros(packed.size + 8, dtype=torch.uint8, device=DEV)
        buf[offset:offset + packed.size] = to_dev(packed)
        rec = buf[offset:offset + packed.size].view(rows, cols // 8, 3)
        for su in ((1, S - 1, S) if offset == 0 else (S,)):
            got = vq.decode(rec, to_dev(s_o.view(np.float16)), cbd, fmt=fmt, stages_used=su).cpu().numpy()
            ref = oracle.decode(idx_o, s_o, cb, stages_used=su)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (rows, cols, offset, su)


def test_error_multi_matrix_bf16(cfg1):
    say("error multi matrix bf16")
    _, cb = cfg1["vq3r"]
    mats = [synthetic.student_t_rows_bf16(32, 512, seed=s) for s in range(3)]
    Wf = [synthetic.bf16_bits_to_f32(m).reshape(32, 512) for m in mats]
    recs, scs = [], []
    for w in Wf:
        i, s = oracle.encode(w, cb)
        recs.append(oracle.pack("vq3r", i))
        scs.append(s)
    sums = vq.error_sums(bf16_dev(np.concatenate(mats)), to_dev(np.concatenate(recs)),
                         to_dev(np.concatenate(scs).view(np.float16)), to_dev(cb), n_mats=3).cpu().numpy()
    for m in range(3):
        i = oracle.unpack("vq3r", recs[m])
        ref = oracle.rel_error(Wf[m], oracle.decode(i, scs[m], cb))
        assert abs(np.sqrt(sums[m, 2] / sums[m, 3]) - ref) < 1e-5


def test_error_extreme_magnitudes(cfg1):
    """Vectors whose squares leave fp32's range still give the oracle's relative
    errors (the kernel sums such vectors in fp64): a tiny matrix (its scales
    underflow to 0), entries near 1e30 against ordinary records, and rows of
    1e-19 / 1 / 1e12 in one matrix."""
    say("error extreme magnitudes")
    _, cb = cfg1["vq3r"]
    base = synthetic.gaussian_rows(24, 256, seed=21)
    idx_b, s_b = oracle.encode(base, cb)
    tiny = (base * np.float32(1e-19)).astype(np.float32)
    idx_t, s_t = oracle.encode(tiny, cb)
    huge = base.copy()
    huge[::3, ::5] *= np.float32(1e30)
    mixed = (base * np.array([1e-19] * 8 + [1.0] * 8 + [1e12] * 8, np.float32)[:, None]).astype(np.float32)
    for tag, W, idx_o, s_o in (("tiny", tiny, idx_t, s_t), ("huge", huge, idx_b, s_b), ("mixed", mixed, idx_b, s_b)):
        rec, sd, cbd = to_dev(oracle.pack("vq3r", idx_o)), to_dev(s_o.view(np.float16)), to_dev(cb)
        rel = vq.rel_errors(to_dev(W), rec, sd, cbd, fmt="vq3r")[0].cpu().numpy()[0]
        for su in (1, 2, 3):
            ref = oracle.rel_error(W, oracle.decode(idx_o, s_o, cb, stages_used=su))
            assert np.isfinite(rel[su - 1]) and abs(rel[su - 1] - ref) <= 1e-5, (tag, su, rel[su - 1], ref)


def test_error_flags_non_finite_weights(cfg1):
    """A non-finite weight is a data error of the error call (status 5);
    finite weights up to the fp32 maximum are not."""
    say("error non-finite")
    _, cb = cfg1["vq3r"]
    W = synthetic.gaussian_rows(40, 256, seed=12)
    idx_o, s_o = oracle.encode(W, cb)
    rec, sd, cbd = to_dev(oracle.pack("vq3r", idx_o)), to_dev(s_o.view(np.float16)), to_dev(cb)
    for bad, where in ((np.nan, (3, 17)), (np.inf, (39, 255)), (-np.inf, (0, 0))):
        Wb = W.copy()
        Wb[where] = bad
        with pytest.raises(vq.VQError) as e:
            vq.error_sums(to_dev(Wb), rec, sd, cbd)
        assert e.value.status == 5, (bad, where)
    Wb = W.copy()
    Wb[5, 9] = np.float32(3.4e38)
    ws = vq.error_workspace("vq3r", 1, 40, 256)
    sums = vq.error_sums(to_dev(Wb), rec, sd, cbd, workspace=ws).cpu().numpy()[0]
    assert np.all(np.isfinite(sums))
    assert vq.lib().vq_read_device_status(ws.data_ptr(), vq._stream()) == 0
    Wb[5, 9] = np.nan
    vq.error_sums(to_dev(Wb), rec, sd, cbd, workspace=ws, check=False)
    assert vq.lib().vq_read_device_status(ws.data_ptr(), vq._stream()) == 5


@pytest.mark.parametrize("rows,cols,n", [(2048, 7168, 3), (100, 264, 70), (1, 8, 5)])
def test_error_sums_do_not_depend_on_batching(rows, cols, n):
    """A matrix's fp64 sums are bit-identical alone and inside a multi-matrix
    call (the per-matrix summation order is fixed by its row count)."""
    say("error batching", rows, cols, n)
    g = torch.Generator(device=DEV)
    g.manual_seed(rows + n)
    W = torch.randn((n * rows, cols), generator=g, device=DEV).to(torch.bfloat16)
    cb = torch.randn((3, 256, 8), generator=g, device=DEV) * 0.5
    idx, sc = vq.encode(W, cb)
    both = vq.error_sums(W, idx, sc, cb, n_mats=n)
    for m in range(n):
        r = slice(m * rows, (m + 1) * rows)
        one = vq.error_sums(W[r], idx[r], sc[r], cb, n_mats=1)
        assert torch.equal(one[0], both[m]), m


# ------------------------------------------------------------------ fit
@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("engine", ["mfma_f16x", "mfma_f32", "valu_f32"])
def test_fit_cfg1_bit_exact(cfg1, fmt, engine):
    say("fit cfg1", fmt, engine)
    init, cb_o = cfg1[fmt]
    cb = vq.fit_codebooks([to_dev(cfg1["W"])], init, fmt=fmt, iters=10, engine=engine)
    torch.cuda.synchronize()
    got = cb.cpu().numpy()
    diff = np.argwhere(got.view(np.uint32) != cb_o.view(np.uint32))
    assert len(diff) == 0, "codebook entries differ: %d, first %s" % (len(diff), diff[:5].tolist())


def test_fit_multi_matrix_bf16_bit_exact():
    say("fit multi bf16")
    mats = [synthetic.student_t_rows_bf16(64, 512, seed=100 + s) for s in range(3)]
    Wf = [synthetic.bf16_bits_to_f32(m).reshape(64, 512) for m in mats]
    n = 3 * 64 * 64
    for fmt in ("vq3r", "vq4p"):
        S, K = vq.stages_entries(fmt)
        init = synthetic.forgy_init(n, K, S, seed=9)
        cb_o, _ = oracle.fit(Wf, S, K, 4, init)
        cb = vq.fit_codebooks([bf16_dev(m) for m in mats], init, fmt=fmt, iters=4)
        assert np.array_equal(cb.cpu().numpy().view(np.uint32), cb_o.view(np.uint32)), fmt


def test_fit_zero_iterations_and_duplicate_values():
    say("fit iters=0 + duplicate-valued init")
    W = synthetic.gaussian_rows(16, 256, seed=21)
    W[:4] = W[4]                                  # identical rows -> identical vectors
    n = 16 * 32
    init = synthetic.forgy_init(n, 64, 4, seed=2)
    rest = np.setdiff1d(init[0], [0, 32, 64])[:61]
    init[0] = np.r_[[0, 32, 64], rest]             # three indices with equal vectors
    for iters in (0, 3):
        cb_o, _ = oracle.fit([W], 4, 64, iters, init)
        cb = vq.fit_codebooks([to_dev(W)], init, fmt="vq4p", iters=iters)
        assert np.array_equal(cb.cpu().numpy().view(np.uint32), cb_o.view(np.uint32)), iters


@pytest.mark.parametrize("seed", [0, 1])
def test_fit_random_shapes_bit_exact(seed):
    """Seeded random fits: format, engine (fp16 split, fp32 matrix cores, fp32
    VALU), shape (up to 400 rows, 8-2072 columns, at least K vectors),
    magnitude (10^-2 .. 10^2) and 1-4 iterations; codebooks bit for bit
    against the oracle's Lloyd fit."""
    say("fit random sweep", seed)
    rng = np.random.default_rng(300 + seed)
    for case in range(20):
        fmt = ["vq3r", "vq4p"][rng.integers(2)]
        S, K = vq.stages_entries(fmt)
        eng = ["auto", "mfma_f32", "valu_f32"][rng.integers(3)]
        V = int(rng.integers(1, 260))
        cols = 8 * V
        rows = int(rng.integers(max(1, -(-K // V)), 400))
        iters = int(rng.integers(1, 5))
        W = (synthetic.student_t_rows_f32(rows, cols, seed=7000 + 100 * seed + case) *
             float(10.0 ** rng.uniform(-2, 2))).astype(np.float32)
        init = synthetic.forgy_init(rows * V, K, S, seed=case)
        cb_o, _ = oracle.fit([W], S, K, iters, init)
        cb = vq.fit_codebooks([to_dev(W)], init, fmt=fmt, iters=iters, engine=eng)
        assert np.array_equal(cb.cpu().numpy().view(np.uint32), cb_o.view(np.uint32)), \
            (case, fmt, eng, rows, cols, iters)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_fit_flag_list_overflow_bit_exact(fmt):
    """Seven eighths of the rows are copies of one row made of 4 distinct
    vectors, so most Forgy codewords coincide and every copied vector ties. The
    assign kernel resolves up to 128 flagged vectors per wave itself; with
    786,432 vectors each wave searches 3 groups of 64, so its stage overflows
    into the exact-pass list, which (capacity 49,152) overflows in turn: the
    exact pass covers every vector and the update must skip the search's
    partial slots."""
    say("fit list overflow", fmt)
    S, K = vq.stages_entries(fmt)
    rows, cols = 4096, 1536
    W = synthetic.gaussian_rows(rows, cols, seed=41)
    base = synthetic.gaussian_rows(4, 8, seed=42)
    W[rows // 8:] = np.tile(base.reshape(-1), cols // 32)[None, :]
    init = synthetic.forgy_init(rows * cols // 8, K, S, seed=43)
    cb_o, _ = oracle.fit([W], S, K, 3, init)
    ws = vq.fit_workspace(fmt, 1, rows, cols)
    cb = vq.fit_codebooks([to_dev(W)], init, fmt=fmt, iters=3, workspace=ws)
    flags = vq.read_status(ws)
    assert flags & (1 << 8)
    assert np.array_equal(cb.cpu().numpy().view(np.uint32), cb_o.view(np.uint32))


def _unit_rms_rows(vals, rng):
    """Rows whose RMS rounds to fp16 1.0 (so the normalized row is the row
    itself): one element per row, at a random position, is set so that the sum
    of squares is cols."""
    W = np.array(vals, dtype=np.float64)
    rows, cols = W.shape
    for r in range(rows):
        k = rng.integers(0, cols)
        W[r, k] = 0.0
        assert np.sum(W[r] ** 2) < cols / 2
        W[r, k] = np.sqrt(cols - np.sum(W[r] ** 2)) * rng.choice([-1.0, 1.0])
    return W.astype(np.float32)


def _extreme_codebooks(rng, S, K):
    C = np.empty((S, K, 8))
    for t in range(S):
        c = rng.standard_normal((K, 8))
        q = K // 8
        c[q:2 * q] *= 0.01
        c[q:2 * q, rng.integers(0, 8)] = rng.choice([2048.0, -2048.0], q)       # the codebook limit
        c[2 * q:3 * q] *= 30.0
        base = rng.choice([1.0, -1.0, 0.5, 2.0, 3.0], (2 * q, 8))
        c[3 * q:5 * q] = base * (1.0 + rng.integers(1, 2 ** 10, (2 * q, 8)) * 2.0 ** -23)  # subnormal lo parts
        c[5 * q:6 * q] = rng.standard_normal((q, 8)) * 2.0 ** -16                 # below fp16's normal range
        C[t] = c
    return np.clip(C, -2048, 2048).astype(np.float32)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("engine", ENGINES)
def test_encode_outlier_rows_and_extreme_codebooks(fmt, engine):
    """Normalized rows at the extremes of the fp16 hi/lo split: all of a row's
    energy in one element (|v| = sqrt(cols)), values whose lo part is an fp16
    subnormal, small rows beside one outlier; codebooks with entries at
    +-2048, scaled by 30, with subnormal lo parts and below 2^-14."""
    say("encode outlier rows", fmt, engine)
    S, K = vq.stages_entries(fmt)
    rng = np.random.default_rng(44)
    rows, cols = 48, 1024
    v = np.empty((rows, cols))
    v[:16] = rng.standard_normal((16, cols)) * 0.01                            # -> one element near 32
    base = rng.choice([1.0, -1.0, 0.5, -0.5, 0.25, -0.25, 0.125], (16, cols))
    v[16:32] = base * (1.0 + rng.integers(1, 2 ** 12, (16, cols)) * 2.0 ** -23)
    v[32:] = rng.standard_normal((16, cols)) * rng.choice([1.0, 2.0 ** -15, 30.0], (16, cols)) * 0.01
    W = _unit_rms_rows(v, rng)
    cb = _extreme_codebooks(rng, S, K)
    idx_o, s_o = oracle.encode(W, cb)
    assert np.all(s_o == 0x3C00)                 # the construction: every row scale is 1.0
    rec, s = vq.encode(to_dev(W), to_dev(cb), fmt=fmt, engine=engine)
    assert np.array_equal(scales_bits(s), s_o)
    got = rec_to_idx(fmt, rec)
    bad = np.argwhere(got != idx_o)
    assert len(bad) == 0, "indices differ: %d, first %s" % (len(bad), bad[:5].tolist())


# ------------------------------------------------------------------ GEMV
def _experts(fmt, cb, E, rows, cols, seed):
    recs, scs, whs = [], [], []
    for e in range(E):
        w = synthetic.student_t_rows_f32(rows, cols, seed=seed + e)
        i, s = oracle.encode(w, cb)
        recs.append(oracle.pack(fmt, i))
        scs.append(s)
        whs.append(oracle.decode(i, s, cb))
    return np.stack(recs), np.stack(scs), whs


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("shape", [(64, 256), (96, 2056), (256, 1024), (32, 448), (1100, 896), (64, 7168),
                                   (2600, 264), (2112, 64), (4160, 136), (2049, 24), (1100, 7168), (300, 7168),
                                   (700, 3976)])
def test_gemv_matches_oracle(cfg1, fmt, shape):
    say("gemv", fmt, shape)
    rows, cols = shape
    _, cb = cfg1[fmt]
    E, ntok, topk = 6, 5, 3
    recs, scs, whs = _experts(fmt, cb, E, rows, cols, seed=40)
    x = synthetic.activations_f16(ntok, cols, seed=1)
    route = synthetic.routing(ntok, E, topk, seed=2)
    packed = vq.gemv_pack(to_dev(recs), fmt=fmt)
    y = vq.dequant_gemv_packed(packed, to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                               to_dev(route), rows, cols, fmt=fmt).cpu().numpy()
    _check_gemv(y, whs, synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)
    # the stored-record call: same kernels on its own packed copies, same bits
    ys = vq.dequant_gemv(to_dev(recs), to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                         to_dev(route), fmt=fmt).cpu().numpy()
    assert np.array_equal(ys.view(np.uint32), y.view(np.uint32))


def _check_gemv(y, whs, xf, route):
    """Per element within 1e-3 * sum_k |w_hat_k x_k| (the condition-aware bar),
    and per output vector ||y - y_ref|| / ||y_ref|| <= 1e-3."""
    ntok, topk = route.shape
    for b in range(ntok):
        for k in range(topk):
            ref, scale = oracle.gemv_ref(whs[route[b, k]], xf[b])
            err = np.abs(y[b, k] - ref)
            assert np.all(err <= 1e-3 * scale + 1e-30), (b, k, float((err / scale).max()))
            nr = np.linalg.norm(ref)
            if nr > 0:
                assert np.linalg.norm(y[b, k] - ref) <= 1e-3 * nr, (b, k)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_gemv_many_slots(cfg1, fmt):
    """Many token slots (1120), each slot a workgroup column of its own."""
    say("gemv many slots", fmt)
    rows, cols = 64, 64
    _, cb = cfg1[fmt]
    E, ntok, topk = 6, 140, 8
    recs, scs, whs = _experts(fmt, cb, E, rows, cols, seed=50)
    x = synthetic.activations_f16(ntok, cols, seed=3)
    route = synthetic.routing(ntok, E, 4, seed=4)
    route = np.concatenate([route, route[::-1]], axis=1).astype(np.int32)
    packed = vq.gemv_pack(to_dev(recs), fmt=fmt)
    y = vq.dequant_gemv_packed(packed, to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                        to_dev(route), rows, cols, fmt=fmt).cpu().numpy()
    _check_gemv(y, whs, synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_gemv_full_layer_sampled(cfg1, fmt):
    """The launch the benchmark times: 256 experts of [2048 x 7168], 16 tokens,
    top-8 routing. Expert e holds the records of base expert e % 2 (two experts
    encoded by the oracle), so every one of the 128 outputs has an oracle value."""
    say("gemv full layer", fmt)
    rows, cols, E, ntok, topk = 2048, 7168, 256, 16, 8
    _, cb = cfg1[fmt]
    recs, scs, whs = _experts(fmt, cb, 2, rows, cols, seed=60)
    rec_d = to_dev(recs)
    packed = torch.empty((E, vq.lib().vq_gemv_packed_size(vq.FORMATS[fmt], rows, cols)), dtype=torch.uint8,
                         device="cuda")
    vq.gemv_pack(rec_d, fmt=fmt, out=packed[:2])
    packed[2:] = packed[:2].repeat(E // 2 - 1, 1)
    scales = to_dev(scs.view(np.float16)).repeat(E // 2, 1)
    x = synthetic.activations_f16(ntok, cols, seed=11)
    route = synthetic.routing(ntok, E, topk, seed=12)
    y = vq.dequant_gemv_packed(packed, scales, to_dev(cb), to_dev(x.view(np.float16)), to_dev(route), rows, cols,
                        fmt=fmt).cpu().numpy()
    _check_gemv(y, [whs[e % 2] for e in range(E)], synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_gemv_full_layer_w2_sampled(cfg1, fmt):
    """The w2 shape of the same layer: 256 experts of [7168 x 2048] (rows cut
    into 4 chunks of 28 row groups), 16 tokens, top-8. Expert e holds the records
    of base expert e % 2."""
    say("gemv full layer w2", fmt)
    rows, cols, E, ntok, topk = 7168, 2048, 256, 16, 8
    _, cb = cfg1[fmt]
    recs, scs, whs = _experts(fmt, cb, 2, rows, cols, seed=64)
    packed = torch.empty((E, vq.lib().vq_gemv_packed_size(vq.FORMATS[fmt], rows, cols)), dtype=torch.uint8,
                         device="cuda")
    vq.gemv_pack(to_dev(recs), fmt=fmt, out=packed[:2])
    packed[2:] = packed[:2].repeat(E // 2 - 1, 1)
    scales = to_dev(scs.view(np.float16)).repeat(E // 2, 1)
    x = synthetic.activations_f16(ntok, cols, seed=13)
    route = synthetic.routing(ntok, E, topk, seed=14)
    y = vq.dequant_gemv_packed(packed, scales, to_dev(cb), to_dev(x.view(np.float16)), to_dev(route), rows, cols,
                        fmt=fmt).cpu().numpy()
    _check_gemv(y, [whs[e % 2] for e in range(E)], synthetic.f16_bits_to_f32(x).reshape(ntok, cols), route)


def test_gemv_bad_route_flagged(cfg1):
    say("gemv bad route")
    _, cb = cfg1["vq3r"]
    recs, scs, _ = _experts("vq3r", cb, 2, 32, 64, seed=3)
    x = synthetic.activations_f16(1, 64, seed=1)
    route = np.array([[0, 5]], np.int32)
    packed = vq.gemv_pack(to_dev(recs))
    with pytest.raises(vq.VQError):
        vq.dequant_gemv_packed(packed, to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                        to_dev(route), 32, 64, check=True)
    # the valid slot is still computed; the bad one is zero
    y = vq.dequant_gemv_packed(packed, to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                        to_dev(route), 32, 64).cpu().numpy()
    assert np.all(y[0, 1] == 0) and np.any(y[0, 0] != 0)
    # the stored-record call reads no expert for the bad id, flags it, zeroes its slot
    with pytest.raises(vq.VQError):
        vq.dequant_gemv(to_dev(recs), to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                        to_dev(route), check=True)
    for bad in (-1, 2, 1 << 30):
        r2 = np.array([[bad, 0, 1, bad]], np.int32)
        ys = vq.dequant_gemv(to_dev(recs), to_dev(scs.view(np.float16)), to_dev(cb), to_dev(x.view(np.float16)),
                             to_dev(r2)).cpu().numpy()
        assert np.all(ys[0, 0] == 0) and np.all(ys[0, 3] == 0)
        assert np.array_equal(ys[0, 1].view(np.uint32), y[0, 0].view(np.uint32))


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("shape", [(1, 8), (64, 224), (70, 456), (128, 7168), (65, 640), (3, 1152)])
def test_gemv_pack_layout(fmt, shape):
    """The packed layout is a pure permutation of the stored records: blocks of 16
    slices x 64-row groups, 4 records (12 bytes) per lane chunk, each row's slices
    rotated by its lane, zero padding. The shapes take the repack's byte, dword
    and 16-byte load paths, with full and partial runs of 4 blocks."""
    say("gemv pack layout", fmt, shape)
    rows, cols = shape
    V = cols // 8
    J = 16
    rng = np.random.default_rng(rows + cols)
    E = 2
    rec = rng.integers(0, 256, size=(E, rows, V, 3), dtype=np.uint8)
    got = vq.gemv_pack(to_dev(rec), fmt=fmt).cpu().numpy()
    nblk, ng = -(-V // J), -(-rows // 64)
    pad = np.zeros((E, ng * 64, nblk * J, 3), np.uint8)
    pad[:, :rows, :V] = rec
    b, g, c, lane, q = np.meshgrid(np.arange(nblk), np.arange(ng), np.arange(J // 4), np.arange(64), np.arange(4),
                                   indexing="ij")
    row = 64 * g + lane
    sl = J * b + (4 * c + q + lane) % J
    want = pad[:, row, sl, :].reshape(E, -1)
    assert got.shape == want.shape and np.array_equal(got, want)


# ------------------------------------------------------------------ MXFP4
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_mxfp4_bit_exact(dtype):
    """Aligned inputs take the 4-elements-per-lane kernel, an input one element
    off its alignment the one-element-per-lane kernel; both bit-exact, with fp32
    and with bf16 output."""
    say("mxfp4", dtype)
    W = synthetic.student_t_rows_f32(64, 1024, seed=8)
    W[3, :32] = 0.0
    W[4, :32] = 1e-42 if dtype != "f16" else 1e-7    # subnormal block
    if dtype != "f16":
        W[5, 64:96] = np.float32(2.0) ** 120         # large exponent
        W[6, 0] = np.float32(3.0e38)                 # largest block scale
        W[6, 1:32] = np.float32(1e-30)               # tiny next to it: flushed to the smallest codes
    else:
        W[5, 64:96] = 60000.0
    if dtype == "bf16":
        bits = synthetic.f32_to_bf16_bits(W)
        Wd = bf16_dev(bits)
        W = synthetic.bf16_bits_to_f32(bits).reshape(W.shape)
    elif dtype == "f16":
        W = W.astype(np.float16).astype(np.float32)
        Wd = to_dev(W.astype(np.float16))
    else:
        Wd = to_dev(W)
    ref = oracle.mxfp4_qdq(W)
    got = vq.mxfp4_qdq(Wd).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    buf = torch.empty(Wd.numel() + 8, dtype=Wd.dtype, device=DEV)
    Wu = buf[1:1 + Wd.numel()].view(Wd.shape)
    Wu.copy_(Wd)
    got = vq.mxfp4_qdq(Wu).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # bf16 output: the upper halves of the oracle's fp32 bits (exact, its lower
    # halves are zero); an output one element off its 8-byte alignment takes
    # the one-element-per-lane kernel
    want = (ref.view(np.uint32) >> 16).astype(np.uint16)
    assert np.all((ref.view(np.uint32) & 0xFFFF) == 0)
    ob = torch.empty(W.shape, dtype=torch.bfloat16, device=DEV)
    got = vq.mxfp4_qdq(Wd, out=ob).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    obuf = torch.zeros(ob.numel() + 4, dtype=torch.bfloat16, device=DEV)
    ou = obuf[1:1 + ob.numel()].view(ob.shape)
    got = vq.mxfp4_qdq(Wu, out=ou).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert float(obuf[0]) == 0.0 and float(obuf[-3:].abs().sum()) == 0.0   # nothing written outside


# ------------------------------------------------------------------ random sweep
@pytest.mark.parametrize("seed", [0, 1])
def test_random_shapes_parity(cfg1, seed):
    """Seeded random cases: format, dtype, shape (1-199 rows, 8-2392 columns),
    magnitude (10^-3 .. 10^2) and zero rows, each through encode (indices and
    scales bit-exact), decode (bit-exact), error (within 1e-5) and the
    dequant-GEMV over 1-4 copies of the matrix with random routing (within
    1e-3 of sum |w_hat x|)."""
    say("random sweep", seed)
    rng = np.random.default_rng(100 + seed)
    for case in range(60):
        fmt = ["vq3r", "vq4p"][rng.integers(2)]
        _, cb = cfg1[fmt]
        S = cb.shape[0]
        rows, V = int(rng.integers(1, 200)), int(rng.integers(1, 300))
        cols = 8 * V
        dt = ["f32", "bf16", "f16"][rng.integers(3)]
        W = (synthetic.gaussian_rows(rows, cols, seed=5000 + 100 * seed + case) *
             float(10.0 ** rng.uniform(-3, 2))).astype(np.float32)
        if rng.random() < 0.2:
            W[rng.integers(rows)] = 0.0
        if dt == "bf16":
            bits = synthetic.f32_to_bf16_bits(W)
            Wd = bf16_dev(bits)
            W = synthetic.bf16_bits_to_f32(bits).reshape(rows, cols)
        elif dt == "f16":
            W = np.clip(W, -60000, 60000).astype(np.float16).astype(np.float32)
            Wd = to_dev(W.astype(np.float16))
        else:
            Wd = to_dev(W)
        tag = (case, fmt, rows, cols, dt)
        idx_o, s_o = oracle.encode(W, cb)
        cbd = to_dev(cb)
        rec, s = vq.encode(Wd, cbd, fmt=fmt)
        assert np.array_equal(rec_to_idx(fmt, rec), idx_o), tag
        assert np.array_equal(scales_bits(s), s_o), tag
        w_ref = oracle.decode(idx_o, s_o, cb)
        got = vq.decode(rec, s, cbd, fmt=fmt).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), w_ref.view(np.uint32)), tag
        rel = vq.rel_errors(Wd, rec, s, cbd, fmt=fmt)[0].cpu().numpy()[0]
        if np.any(W):
            for su in range(1, S + 1):
                ref = oracle.rel_error(W, oracle.decode(idx_o, s_o, cb, stages_used=su))
                assert abs(rel[su - 1] - ref) <= 1e-5, tag + (su,)
        else:
            assert np.all(rel == 0), tag  # zeros reconstructed as zeros
        E, ntok = int(rng.integers(1, 5)), int(rng.integers(1, 6))
        topk = int(rng.integers(1, E + 1))
        packed = vq.gemv_pack(rec[None].expand(E, -1, -1, -1).contiguous(), fmt=fmt)
        x = synthetic.activations_f16(ntok, cols, seed=case)
        route = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(ntok)]).astype(np.int32)
        sE = s[None].expand(E, -1).contiguous()
        y = vq.dequant_gemv_packed(packed, sE, cbd, to_dev(x.view(np.float16)),
                                   to_dev(route), rows, cols, fmt=fmt).cpu().numpy()
        # the stored-record call runs the same kernels on its own packed copies
        ys = vq.dequant_gemv(rec[None].expand(E, -1, -1, -1).contiguous(), sE, cbd, to_dev(x.view(np.float16)),
                             to_dev(route), fmt=fmt).cpu().numpy()
        assert np.array_equal(ys.view(np.uint32), y.view(np.uint32)), tag
        xf = synthetic.f16_bits_to_f32(x).reshape(ntok, cols)
        for b in range(ntok):
            ref, scale = oracle.gemv_ref(w_ref, xf[b])
            for k in range(topk):
                assert np.all(np.abs(y[b, k] - ref) <= 1e-3 * scale), tag + (b, k)
                nr = np.linalg.norm(ref)
                if nr > 0:
                    assert np.linalg.norm(y[b, k] - ref) <= 1e-3 * nr, tag + (b, k)

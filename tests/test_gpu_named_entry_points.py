"""The C ABI's hot-path entry points called by name through ctypes (not through
the Python helpers): vq_fit_codebooks, vq_fit_codebooks_seeded, vq3r_encode / vq4p_encode,
vq3r_decode / vq4p_decode, vq3r_dequant_gemv / vq4p_dequant_gemv (stored
records), vq_error with its relative errors, vq_read_device_status and
vq_status_string, each against the oracle to the parity bar of its operation."""
import ctypes

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def ws(n):
    return torch.zeros(max(int(n), 256), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_named_entry_points_against_oracle(fmt):
    print("named entry points", fmt, flush=True)
    L = vq.lib()
    S, K = vq.stages_entries(fmt)
    F = vq.FORMATS[fmt]
    rows, cols, iters = 96, 1032, 4
    W = synthetic.gaussian_rows(rows, cols, seed=21)
    Wd = dev(W)
    init = synthetic.forgy_init(rows * cols // 8, K, S, seed=22)

    # vq_fit_codebooks: codebooks bit-exact
    cb = torch.empty((S, K, 8), dtype=torch.float32, device=DEV)
    w_fit = ws(L.vq_fit_workspace_size(F, 1, rows, cols))
    mats = (ctypes.c_void_p * 1)(Wd.data_ptr())
    init_h = np.ascontiguousarray(init, dtype=np.int64)
    st = L.vq_fit_codebooks(F, mats, 0, 1, rows, cols, iters, init_h.ctypes.data_as(ctypes.c_void_p), P(cb), P(w_fit),
                            w_fit.numel(), 0, stream())
    assert st == 0, L.vq_status_string(st)
    assert L.vq_read_device_status(P(w_fit), stream()) == 0
    cb_o, _ = oracle.fit([W], S, K, iters, init)
    assert np.array_equal(cb.cpu().numpy().view(np.uint32), cb_o.view(np.uint32))

    # vq_fit_codebooks_seeded: the library draws the init (vq_forgy_init); bit-exact
    # against the oracle started from its own seeded init
    cb_s = torch.empty((S, K, 8), dtype=torch.float32, device=DEV)
    st = L.vq_fit_codebooks_seeded(F, mats, 0, 1, rows, cols, iters, 4242, P(cb_s), P(w_fit), w_fit.numel(), 0,
                                   stream())
    assert st == 0, L.vq_status_string(st)
    assert L.vq_read_device_status(P(w_fit), stream()) == 0
    cb_so, _ = oracle.fit([W], S, K, iters, oracle.forgy_init_seeded(rows * cols // 8, K, S, 4242))
    assert np.array_equal(cb_s.cpu().numpy().view(np.uint32), cb_so.view(np.uint32))

    # vq3r_encode / vq4p_encode: indices and scales bit-exact
    enc = L.vq3r_encode if fmt == "vq3r" else L.vq4p_encode
    idx = torch.empty((rows, cols // 8, 3), dtype=torch.uint8, device=DEV)
    sc = torch.empty(rows, dtype=torch.float16, device=DEV)
    w_enc = ws(L.vq_encode_workspace_size(F, rows, cols))
    assert enc(P(Wd), 0, rows, cols, P(cb), P(idx), P(sc), P(w_enc), w_enc.numel(), stream()) == 0
    assert L.vq_read_device_status(P(w_enc), stream()) == 0
    idx_o, s_o = oracle.encode(W, cb_o)
    assert np.array_equal(oracle.unpack(fmt, idx.cpu().numpy()), idx_o)
    assert np.array_equal(sc.cpu().view(torch.int16).numpy().view(np.uint16), s_o)

    # vq3r_decode / vq4p_decode: decoded weights bit-exact
    dec = L.vq3r_decode if fmt == "vq3r" else L.vq4p_decode
    w_hat = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    assert dec(P(idx), P(sc), P(cb), rows, cols, P(w_hat), stream()) == 0
    ref = oracle.decode(idx_o, s_o, cb_o)
    assert np.array_equal(w_hat.cpu().numpy().view(np.uint32), ref.view(np.uint32))

    # vq_error: relative errors within 1e-5 of the oracle's
    sums = torch.empty((1, S + 1), dtype=torch.float64, device=DEV)
    rel = torch.empty((1, S), dtype=torch.float64, device=DEV)
    rel_all = torch.empty(S, dtype=torch.float64, device=DEV)
    w_err = ws(L.vq_error_workspace_size(F, 1, rows, cols))
    assert L.vq_error(F, P(Wd), 0, P(idx), P(sc), P(cb), 1, rows, cols, P(sums), P(rel), P(rel_all), P(w_err),
                      w_err.numel(), stream()) == 0
    assert L.vq_read_device_status(P(w_err), stream()) == 0
    for su in range(1, S + 1):
        r_o = oracle.rel_error(W, oracle.decode(idx_o, s_o, cb_o, stages_used=su))
        assert abs(float(rel[0, su - 1]) - r_o) <= 1e-5
        assert float(rel_all[su - 1]) == float(rel[0, su - 1])

    # vq3r_dequant_gemv / vq4p_dequant_gemv on stored records: 3 experts (the
    # encoded one, and two more encoded by the oracle), 4 tokens, top-2
    E, ntok, topk = 3, 4, 2
    recs, scs, whs = [oracle.pack(fmt, idx_o)], [s_o], [ref]
    for e in (1, 2):
        We = synthetic.gaussian_rows(rows, cols, seed=30 + e)
        i_e, s_e = oracle.encode(We, cb_o)
        recs.append(oracle.pack(fmt, i_e))
        scs.append(s_e)
        whs.append(oracle.decode(i_e, s_e, cb_o))
    rec_d = dev(np.stack(recs))
    sc_d = dev(np.stack(scs).view(np.float16))
    x = synthetic.activations_f16(ntok, cols, seed=23)
    route = np.array([[0, 2], [1, 0], [2, 2], [1, 2]], np.int32)
    y = torch.empty((ntok, topk, rows), dtype=torch.float32, device=DEV)
    w_g = ws(L.vq_gemv_workspace_size(F, rows, cols, ntok, topk, E))
    gemv = L.vq3r_dequant_gemv if fmt == "vq3r" else L.vq4p_dequant_gemv
    assert gemv(P(rec_d), rows * (cols // 8) * 3, P(sc_d), rows, P(cb), rows, cols, E, P(dev(x.view(np.float16))), ntok,
                P(dev(route)), topk, P(y), P(w_g), w_g.numel(), stream()) == 0
    assert L.vq_read_device_status(P(w_g), stream()) == 0
    yh = y.cpu().numpy()
    xf = synthetic.f16_bits_to_f32(x).reshape(ntok, cols)
    for b in range(ntok):
        for k in range(topk):
            r_y, scale = oracle.gemv_ref(whs[route[b, k]], xf[b])
            assert np.all(np.abs(yh[b, k] - r_y) <= 1e-3 * scale)
            assert np.linalg.norm(yh[b, k] - r_y) <= 1e-3 * np.linalg.norm(r_y)
    # a data error is reported by name: a route id past the experts
    route_bad = route.copy()
    route_bad[0, 1] = E
    assert gemv(P(rec_d), rows * (cols // 8) * 3, P(sc_d), rows, P(cb), rows, cols, E, P(dev(x.view(np.float16))),
                ntok, P(dev(route_bad)), topk, P(y), P(w_g), w_g.numel(), stream()) == 0
    st = L.vq_read_device_status(P(w_g), stream())
    assert st == 5 and L.vq_status_string(st) == b"data error flagged on the device"

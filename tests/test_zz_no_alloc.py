"""vq_dequant_gemv_packed_noalloc, the GEMV entry point for callers that cannot
allocate device memory, called by name through ctypes. Its output must equal
vq_dequant_gemv_packed's on the same inputs bit for bit (same kernels, same
launch geometry) and the oracle's fp64 product within 1e-3 of
sum_c |w_hat[r][c] x[c]| per element, on two calls in a row, the second on a
smaller input (ragged slices, fewer experts, rows and tokens); the status word
reaches the caller's buffer; a call whose partial sums exceed the static
scratch is refused before anything runs."""
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


def P(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_case(fmt, E, rows, cols, ntok, topk, seed):
    S, K = vq.stages_entries(fmt)
    rng = np.random.default_rng(seed)
    V = cols // 8
    idx = [rng.integers(0, K, (rows, V, S)) for _ in range(E)]
    sc = [(rng.uniform(0.5, 2.0, rows) * 0.01).astype(np.float16).view(np.uint16) for _ in range(E)]
    cb = rng.standard_normal((S, K, 8)).astype(np.float32)
    rec = np.stack([oracle.pack(fmt, i) for i in idx])
    x = synthetic.activations_f16(ntok, cols, seed=seed + 1)
    route = synthetic.routing(ntok, E, topk, seed=seed + 2)
    L = vq.lib()
    F = vq.FORMATS[fmt]
    packed = torch.empty((E, L.vq_gemv_packed_size(F, rows, cols)), dtype=torch.uint8, device=DEV)
    rec_d = torch.from_numpy(rec).to(DEV)
    assert L.vq_gemv_pack(F, P(rec_d), rows, cols, E, P(packed), stream()) == 0
    d = {"fmt": fmt, "F": F, "E": E, "rows": rows, "cols": cols, "ntok": ntok, "topk": topk, "packed": packed,
         "sc": torch.from_numpy(np.stack(sc).view(np.int16)).to(DEV), "cb": torch.from_numpy(cb).to(DEV),
         "x": torch.from_numpy(x.view(np.int16)).to(DEV), "route": torch.from_numpy(route).to(DEV),
         "idx": idx, "sc_h": sc, "cb_h": cb, "x_h": synthetic.f16_bits_to_f32(x).reshape(ntok, cols),
         "route_h": route}
    return d


def run_noalloc(c, status, route=None):
    L = vq.lib()
    y = torch.full((c["ntok"], c["topk"], c["rows"]), float("nan"), dtype=torch.float32, device=DEV)
    st = L.vq_dequant_gemv_packed_noalloc(c["F"], P(c["packed"]), c["packed"].shape[1], P(c["sc"]), c["rows"],
                                          P(c["cb"]), c["rows"], c["cols"], c["E"], P(c["x"]), c["ntok"],
                                          P(c["route"] if route is None else route), c["topk"], P(y), P(status),
                                          stream())
    return st, y


def run_packed(c):
    L = vq.lib()
    y = torch.full((c["ntok"], c["topk"], c["rows"]), float("nan"), dtype=torch.float32, device=DEV)
    n = L.vq_gemv_packed_workspace_size(c["F"], c["rows"], c["cols"], c["ntok"], c["topk"])
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
    st = L.vq_dequant_gemv_packed(c["F"], P(c["packed"]), c["packed"].shape[1], P(c["sc"]), c["rows"], P(c["cb"]),
                                  c["rows"], c["cols"], c["E"], P(c["x"]), c["ntok"], P(c["route"]), c["topk"], P(y),
                                  P(ws), ws.numel(), stream())
    assert st == 0, vq.lib().vq_status_string(st)
    assert L.vq_read_device_status(P(ws), stream()) == 0
    return y


def check_oracle(c, y):
    yh = y.cpu().numpy()
    w_hat = {}
    for b in range(c["ntok"]):
        for k in range(c["topk"]):
            e = int(c["route_h"][b, k])
            if e not in w_hat:
                w_hat[e] = oracle.decode(c["idx"][e], c["sc_h"][e], c["cb_h"])
            r_y, scale = oracle.gemv_ref(w_hat[e], c["x_h"][b])
            assert np.all(np.abs(yh[b, k] - r_y) <= 1e-3 * scale), (b, k)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_noalloc_gemv_matches_packed_entry_point(fmt):
    print("no-alloc GEMV", fmt, flush=True)
    L = vq.lib()
    big = make_case(fmt, 12, 1024, 4096, 16, 4, seed=70)
    small = make_case(fmt, 5, 320, 1032, 3, 2, seed=80)
    status = torch.full((256,), 0xAB, dtype=torch.uint8, device=DEV)
    for c, stat in ((big, status), (small, None)):
        print("  case rows=%d cols=%d pairs=%d" % (c["rows"], c["cols"], c["ntok"] * c["topk"]), flush=True)
        st, y = run_noalloc(c, stat)
        assert st == 0, L.vq_status_string(st)
        torch.cuda.synchronize()
        if stat is not None:
            assert L.vq_read_device_status(P(stat), stream()) == 0
        y_ref = run_packed(c)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32))
        check_oracle(c, y)
    # a route id past the experts reaches the caller's status word; its slot is 0
    bad = small["route"].clone()
    bad[1, 0] = small["E"]
    st, y = run_noalloc(small, status, route=bad)
    assert st == 0
    assert L.vq_read_device_status(P(status), stream()) == 5
    assert np.all(y[1, 0].cpu().numpy() == 0.0)
    # the same call again is clean (the status word is rewritten by every call)
    st, y = run_noalloc(small, status)
    assert st == 0 and L.vq_read_device_status(P(status), stream()) == 0


def test_noalloc_gemv_refuses_calls_beyond_the_scratch():
    """4096 pairs x 2048 rows of partial sums need at least 32 MiB (one range
    per pair at the least), twice the scratch: refused, nothing launched."""
    print("no-alloc GEMV size refusal", flush=True)
    L = vq.lib()
    rows, cols, ntok, topk = 2048, 64, 512, 8
    c = {"F": 0, "E": 1, "rows": rows, "cols": cols, "ntok": ntok, "topk": topk}
    c["packed"] = torch.zeros((1, L.vq_gemv_packed_size(0, rows, cols)), dtype=torch.uint8, device=DEV)
    c["sc"] = torch.zeros((1, rows), dtype=torch.int16, device=DEV)
    c["cb"] = torch.zeros((3, 256, 8), dtype=torch.float32, device=DEV)
    c["x"] = torch.zeros((ntok, cols), dtype=torch.int16, device=DEV)
    c["route"] = torch.zeros((ntok, topk), dtype=torch.int32, device=DEV)
    assert ntok * topk * rows * 4 >= 2 * (16 << 20)   # VQ_NOALLOC_SCRATCH_BYTES = 16 MiB
    st, _ = run_noalloc(c, None)
    assert st == 8 and L.vq_status_string(st) == b"call too large for the no-allocation scratch"

"""The decode-time entry points allocate nothing and issue no memsets, so a
caller can capture them in a HIP graph. Each captured call is replayed
several times, with eager work and synchronizations between the replays, and
every replay must equal the eager call bit for bit."""
import sys

import numpy as np
import pytest

import synthetic

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import residual_vector_quantization_amd as vq  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def check_replays(g, outs, refs, clobber):
    for rep in range(3):
        for o in outs:
            clobber(o)
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), rep
        torch.randn(1024, device="cuda").sum().item()  # eager work between replays


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_encode_decode_gemv_replay_bit_exact(fmt):
    say("graph replay", fmt)
    S, K = vq.stages_entries(fmt)
    E, rows, cols, ntok, topk = 4, 256, 1024, 3, 2
    bits = np.stack([synthetic.student_t_rows_bf16(rows, cols, seed=900 + e) for e in range(E)])
    W = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16).reshape(E * rows, cols)
    g0 = torch.Generator(device="cuda")
    g0.manual_seed(4)
    cb = torch.randn((S, K, 8), device="cuda", generator=g0) * 0.5
    ws = vq.encode_workspace(fmt, E * rows, cols)
    idx = torch.empty((E * rows, cols // 8, 3), dtype=torch.uint8, device="cuda")
    sc = torch.empty(E * rows, dtype=torch.float16, device="cuda")
    enc = lambda: vq.encode(W, cb, fmt=fmt, idx=idx, scales=sc, workspace=ws, check=False)  # noqa: E731
    enc()
    torch.cuda.synchronize()
    assert vq.read_status(ws) & 0xFF == 0
    idx_ref, sc_ref = idx.clone(), sc.clone()
    g = capture(enc)
    check_replays(g, [idx, sc], [idx_ref, sc_ref], lambda t: t.view(torch.uint8).fill_(0xAB))

    out = torch.empty((E * rows, cols), dtype=torch.float32, device="cuda")
    dec = lambda: vq.decode(idx, sc, cb, fmt=fmt, out=out)  # noqa: E731
    dec()
    torch.cuda.synchronize()
    out_ref = out.clone()
    g = capture(dec)
    check_replays(g, [out], [out_ref], lambda t: t.fill_(float("nan")))

    packed = vq.gemv_pack(idx.view(E, rows, cols // 8, 3), fmt=fmt)
    x = torch.from_numpy(synthetic.activations_f16(ntok, cols, seed=3).view(np.float16)).cuda()
    route = torch.from_numpy(synthetic.routing(ntok, E, topk, seed=5)).cuda()
    y = torch.empty((ntok, topk, rows), device="cuda")
    wsg = vq.gemv_packed_workspace(fmt, rows, cols, ntok, topk)
    gemv = lambda: vq.dequant_gemv_packed(packed, sc.view(E, rows), cb, x, route, rows, cols, fmt=fmt, y=y,  # noqa: E731
                                   workspace=wsg)
    gemv()
    torch.cuda.synchronize()
    y_ref = y.clone()
    g = capture(gemv)
    check_replays(g, [y], [y_ref], lambda t: t.fill_(float("nan")))

"""Lloyd fit parity at the sizes the layer workload runs ([VQ3R page] §2 and
§4: codebooks fit by Lloyd k-means on 12 sampled experts).

The expected codebooks, index and scale hashes and errors were written by
tests/golden/make_fit_goldens.py, which calls only the CPU oracle and the seeded
generators (its oracle run times are in fit_config2_vq3r.json). The inputs are
drawn here with the same numpy generators, so both sides see the same bf16
experts.

  * one full [2048 x 7168] expert (1,835,008 vectors, 3 iterations), VQ3R and
    VQ4P: the assign kernel runs several 64-vector groups per wave with the
    next group's registers prefetched, and the update sums 1,024 partial slots
  * the 12-expert layer slice (22,020,096 vectors, 20 iterations, VQ3R), then
    the encode of all 12 experts with the oracle's codebooks: indices and scales
    compared through sha256 of the oracle's layout, errors within 1e-5
"""
import hashlib
import json
import os

import numpy as np
import pytest

import oracle
import synthetic

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import residual_vector_quantization_amd as vq  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ROWS, COLS = 2048, 7168
NVEC = ROWS * COLS // 8


def expert_bf16_dev(seed):
    bits = synthetic.student_t_rows_bf16(ROWS, COLS, seed=seed)
    return torch.from_numpy(bits.view(np.int16).reshape(ROWS, COLS)).to("cuda").view(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_fit_full_expert_bit_exact(fmt):
    print("fit full expert", fmt, flush=True)
    S, K = vq.stages_entries(fmt)
    want = np.load(os.path.join(GOLDEN, "fit_full_expert_%s.npy" % fmt))
    W = expert_bf16_dev(2901)
    init = synthetic.forgy_init(NVEC, K, S, seed=2902)
    ws = vq.fit_workspace(fmt, 1, ROWS, COLS)
    cb = vq.fit_codebooks([W], init, fmt=fmt, iters=3, workspace=ws)
    assert vq.read_status(ws) & 0xFF == 0
    diff = np.argwhere(cb.cpu().numpy().view(np.uint32) != want.view(np.uint32))
    assert len(diff) == 0, "codebook entries differ: %d, first %s" % (len(diff), diff[:5].tolist())


def test_fit_and_encode_layer_slice_12_experts():
    print("fit 12-expert slice", flush=True)
    meta = json.load(open(os.path.join(GOLDEN, "fit_config2_vq3r.json")))
    want = np.load(os.path.join(GOLDEN, "fit_config2_vq3r.npy"))
    mats = [expert_bf16_dev(s) for s in meta["expert_seeds"]]
    assert meta["experts"] == [int(e) for e in synthetic.sample_experts(256, 12, seed=2)]
    init = synthetic.forgy_init(len(mats) * NVEC, 256, 3, seed=meta["init_seed"])
    cb = vq.fit_codebooks(mats, init, fmt="vq3r", iters=meta["iters"])
    diff = np.argwhere(cb.cpu().numpy().view(np.uint32) != want.view(np.uint32))
    assert len(diff) == 0, "codebook entries differ: %d, first %s" % (len(diff), diff[:5].tolist())
    print("encode 12-expert slice", flush=True)
    cb_o = torch.from_numpy(want).to("cuda")
    flat = torch.cat(mats, dim=0)
    idx, sc = vq.encode(flat, cb_o, fmt="vq3r")
    h_idx, h_sc = hashlib.sha256(), hashlib.sha256()
    for e in range(len(mats)):
        rec = idx[e * ROWS:(e + 1) * ROWS].cpu().numpy()
        h_idx.update(np.ascontiguousarray(oracle.unpack("vq3r", rec), dtype=np.uint8).tobytes())
        h_sc.update(sc[e * ROWS:(e + 1) * ROWS].cpu().view(torch.int16).numpy().view(np.uint16).tobytes())
    assert h_idx.hexdigest() == meta["indices_sha256"]
    assert h_sc.hexdigest() == meta["scales_sha256"]
    _, rel_all, _ = vq.rel_errors(flat, idx, sc, cb_o, fmt="vq3r", n_mats=len(mats))
    for t in range(3):
        assert abs(float(rel_all[t]) - meta["rel_err_after_stage"][t]) <= 1e-5

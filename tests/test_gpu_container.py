"""The expert-record container on the GPU: records encoded by the HIP path,
written to a container, streamed back into device memory through the pinned
staging buffer (vqc_load_records), parsed by the oracle's independent reader,
and verified record by record against the source weights ([VQ3R page] §4).
Bars: every byte identical; the container's records equal the oracle's encode
of the same weights; recomputed errors equal the stored ones exactly and the
oracle's within 1e-5."""
import sys

import numpy as np
import pytest

import oracle
import synthetic
from oracle import container as oc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import residual_vector_quantization_amd as vq  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.fixture(scope="module", params=["vq3r", "vq4p"])
def converted(request, tmp_path_factory):
    """Three [256 x 1024] bf16 Student-t experts, codebooks from a short oracle
    fit on the first, encoded on the GPU and written to a container."""
    fmt = request.param
    say("container case", fmt)
    S, K = vq.stages_entries(fmt)
    Wb = [synthetic.student_t_rows_bf16(256, 1024, seed=40 + e) for e in range(3)]
    Wf = [synthetic.bf16_bits_to_f32(w) for w in Wb]
    init = synthetic.forgy_init(256 * 128, K, S, seed=9)
    cb, _ = oracle.fit([Wf[0]], S, K, 3, init)
    cbd = torch.from_numpy(cb).to(DEV)
    Wd = [bf16_dev(w) for w in Wb]
    recs, scs, errs = [], [], []
    for w in Wd:
        rec, s = vq.encode(w, cbd, fmt=fmt)
        recs.append(rec)
        scs.append(s)
        errs.append(vq.rel_errors(w, rec, s, cbd, fmt=fmt)[0][0])
    rec, sc, rel = torch.stack(recs), torch.stack(scs), torch.stack(errs)
    path = tmp_path_factory.mktemp("c") / ("%s.vqc" % fmt)
    vq.write_container(path, fmt, cbd, rec, sc, rel_err=rel)
    torch.cuda.synchronize()
    return {"fmt": fmt, "cb": cb, "Wf": Wf, "Wd": Wd, "rec": rec, "sc": sc, "rel": rel.cpu().numpy(), "path": path}


@pytest.mark.parametrize("staging_strides", [2, 3, 64])
def test_load_records_to_device_is_bit_exact(converted, staging_strides):
    fmt, path = converted["fmt"], converted["path"]
    stride = vq.container_layout(fmt, 256, 1024, 3)["record_stride"]
    say("load", fmt, "staging", staging_strides, "strides")
    cb, rec, sc, rel = vq.load_container(path, staging_bytes=staging_strides * stride)
    torch.cuda.synchronize()
    assert torch.equal(rec, converted["rec"])
    assert torch.equal(sc.view(torch.int16), converted["sc"].view(torch.int16))
    assert np.array_equal(cb.cpu().numpy(), converted["cb"])
    assert np.array_equal(rel, converted["rel"])
    _, rec1, sc1, _ = vq.load_container(path, first=1, count=2, staging_bytes=2 * stride)
    assert torch.equal(rec1, converted["rec"][1:])


def test_container_holds_the_oracle_encode(converted):
    fmt = converted["fmt"]
    say("oracle reader", fmt)
    got = oc.read(converted["path"])
    for e, w in enumerate(converted["Wf"]):
        idx_o, s_o = oracle.encode(w, converted["cb"])
        assert np.array_equal(got["idx"][e], oracle.pack(fmt, idx_o))
        assert np.array_equal(got["scales"][e], s_o)


def test_verify_container(converted):
    fmt = converted["fmt"]
    say("verify", fmt)
    v = vq.verify_container(converted["path"], converted["Wd"])
    assert v["match"]
    got = oc.read(converted["path"])
    S = vq.stages_entries(fmt)[0]
    for e, w in enumerate(converted["Wf"]):
        idx = oracle.unpack(fmt, got["idx"][e])
        for su in range(1, S + 1):
            ref = oracle.rel_error(w, oracle.decode(idx, got["scales"][e], got["codebooks"], stages_used=su))
            assert abs(v["measured"][e, su - 1] - ref) <= 1e-5


def test_verify_detects_a_changed_source(converted):
    say("verify mismatch", converted["fmt"])
    W = [w.clone() for w in converted["Wd"]]
    W[2][5, 7] = W[2][5, 7] * 2 + 0.01
    v = vq.verify_container(converted["path"], W)
    assert not v["match"]
    assert np.array_equal(v["measured"][:2], v["stored"][:2])


def test_corrupt_record_fails_the_device_load(converted, tmp_path):
    fmt = converted["fmt"]
    say("corrupt load", fmt)
    raw = bytearray(open(converted["path"], "rb").read())
    L = oc.layout(fmt, 256, 1024, 3)
    raw[L["rec_off"] + 2 * L["stride"] + L["idx_off"] + 77] ^= 1
    p = tmp_path / "bad.vqc"
    p.write_bytes(bytes(raw))
    with pytest.raises(vq.VQError) as e:
        vq.load_container(p, staging_bytes=2 * L["stride"])
    assert e.value.status == 7
    _, rec, _, _ = vq.load_container(p, first=0, count=2, staging_bytes=2 * L["stride"])
    assert torch.equal(rec, converted["rec"][:2])

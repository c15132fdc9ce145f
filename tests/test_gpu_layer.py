"""Per-layer conversion (w1, w3 and the transposed shape w2, each family with
its own codebooks; [VQ3R page] §2, §4, §3.2) against the oracle, on a small
seeded layer. Bars: codebooks, indices and scales bit-exact; per-expert and
per-family relative errors within 1e-5; the written containers hold exactly
the converted records."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_convert_layer_matches_oracle(fmt, tmp_path):
    say("convert layer", fmt)
    E, d, f = 4, 256, 64          # w1, w3: [f x d]; w2: [d x f]
    S, K = vq.stages_entries(fmt)
    shapes = {"w1": (f, d), "w3": (f, d), "w2": (d, f)}
    sample = [1, 3]
    host, dev, inits = {}, {}, {}
    for j, (name, (rows, cols)) in enumerate(shapes.items()):
        bits = np.stack([synthetic.student_t_rows_bf16(rows, cols, seed=500 + 10 * j + e) for e in range(E)])
        host[name] = synthetic.bf16_bits_to_f32(bits).reshape(E, rows, cols)
        dev[name] = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        inits[name] = synthetic.forgy_init(len(sample) * rows * cols // 8, K, S, seed=7 + j)
    res = vq.convert_layer(dev, inits, sample, fmt=fmt, iters=5, out_dir=tmp_path)
    for name in shapes:
        W = host[name]
        cb_o, _ = oracle.fit([W[e] for e in sample], S, K, 5, inits[name])
        r = res[name]
        assert np.array_equal(r["codebooks"].cpu().numpy().view(np.uint32), cb_o.view(np.uint32)), name
        d2, wsq = np.zeros(S), 0.0
        got = oc.read(tmp_path / (name + ".vqc"))
        for e in range(E):
            idx_o, s_o = oracle.encode(W[e], cb_o)
            assert np.array_equal(oracle.unpack(fmt, r["idx"][e].cpu().numpy()), idx_o), (name, e)
            assert np.array_equal(r["scales"][e].cpu().view(torch.int16).numpy().view(np.uint16), s_o)
            assert np.array_equal(got["idx"][e], r["idx"][e].cpu().numpy())
            for su in range(1, S + 1):
                wh = oracle.decode(idx_o, s_o, cb_o, stages_used=su)
                ref = oracle.rel_error(W[e], wh)
                assert abs(float(r["rel_err"][e, su - 1]) - ref) <= 1e-5, (name, e, su)
                dd, ww = oracle.error_sums(W[e], wh)
                d2[su - 1] += dd
            wsq += ww
        assert np.allclose(r["rel_err_all"].cpu().numpy(), np.sqrt(d2 / wsq), rtol=0, atol=1e-5), name
        assert np.array_equal(got["rel_err"], r["rel_err"].cpu().numpy())

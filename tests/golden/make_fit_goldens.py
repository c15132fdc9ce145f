#!/usr/bin/env python3
"""Writes the stored expected values of the at-size Lloyd fit tests, computed by
the CPU oracle alone (oracle/ + the seeded generators of synthetic/):

  fit_full_expert_<fmt>.npy   codebooks of a 3-iteration fit on one full
                              [2048 x 7168] bf16 expert (Student-t recipe,
                              seed 2901; Forgy init seed 2902), VQ3R and VQ4P
  fit_config2_vq3r.npy        codebooks of the 12-expert, 20-iteration VQ3R fit
                              of the layer slice (experts sample_experts(256, 12,
                              seed 2), expert seeds 2000 + e; Forgy init seed 2)
  fit_config2_vq3r.json       the slice's oracle encode: sha256 of the indices and
                              of the fp16 scale bits of all 12 experts, relative
                              Frobenius error after stages 1-3, and run times

Run from the repository root: python tests/golden/make_fit_goldens.py [expert|config2]
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synthetic  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
ROWS, COLS = 2048, 7168
NVEC = ROWS * COLS // 8

EXPERT_SEED, EXPERT_INIT_SEED, EXPERT_ITERS = 2901, 2902, 3
CFG2_ITERS, CFG2_INIT_SEED = 20, 2


def expert_f32(seed):
    return synthetic.bf16_bits_to_f32(synthetic.student_t_rows_bf16(ROWS, COLS, seed=seed)).reshape(ROWS, COLS)


def config2_experts():
    return [int(e) for e in synthetic.sample_experts(256, 12, seed=2)]


def full_expert():
    w = expert_f32(EXPERT_SEED)
    for fmt, S, K in (("vq3r", 3, 256), ("vq4p", 4, 64)):
        init = synthetic.forgy_init(NVEC, K, S, seed=EXPERT_INIT_SEED)
        t0 = time.time()
        cb, _ = oracle.fit([w], S, K, EXPERT_ITERS, init)
        print("full expert %s: %.1f s" % (fmt, time.time() - t0), flush=True)
        np.save(os.path.join(HERE, "fit_full_expert_%s.npy" % fmt), cb)


def config2():
    experts = config2_experts()
    mats = [expert_f32(synthetic.expert_seed(2, e)) for e in experts]
    init = synthetic.forgy_init(len(mats) * NVEC, 256, 3, seed=CFG2_INIT_SEED)
    t0 = time.time()
    cb, _ = oracle.fit(mats, 3, 256, CFG2_ITERS, init)
    t_fit = time.time() - t0
    print("config 2 fit: %.1f s" % t_fit, flush=True)
    np.save(os.path.join(HERE, "fit_config2_vq3r.npy"), cb)
    h_idx, h_sc = hashlib.sha256(), hashlib.sha256()
    num = np.zeros(3)
    den = 0.0
    t0 = time.time()
    for w in mats:
        idx, s = oracle.encode(w, cb)
        h_idx.update(np.ascontiguousarray(idx, dtype=np.uint8).tobytes())
        h_sc.update(np.ascontiguousarray(s, dtype=np.uint16).tobytes())
        for su in range(1, 4):
            num[su - 1] += oracle.error_sums(w, oracle.decode(idx, s, cb, stages_used=su))[0]
        den += float(np.sum(w.astype(np.float64) ** 2))
    t_enc = time.time() - t0
    meta = {"experts": experts, "expert_seeds": [synthetic.expert_seed(2, e) for e in experts],
            "iters": CFG2_ITERS, "init_seed": CFG2_INIT_SEED,
            "indices_layout": "per expert, oracle.encode order: uint8 [rows, cols/8, stages]",
            "indices_sha256": h_idx.hexdigest(), "scales_sha256": h_sc.hexdigest(),
            "rel_err_after_stage": [float(np.sqrt(v / den)) for v in num],
            "oracle_fit_seconds": round(t_fit, 1), "oracle_encode_seconds": round(t_enc, 1),
            "oracle_threads": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))}
    with open(os.path.join(HERE, "fit_config2_vq3r.json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(json.dumps(meta), flush=True)


if __name__ == "__main__":
    what = sys.argv[1:] or ["expert", "config2"]
    if "expert" in what:
        full_expert()
    if "config2" in what:
        config2()

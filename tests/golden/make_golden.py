"""Writes tests/golden/oracle_tiny.json: oracle outputs on the seeded one-layer
workload (hidden 256, 4/2 heads, head_dim 64, FFN 688, batch 4, contexts in
[1, 64], block size 16).  Calls only oracle/ and the seeded input generator.

Regenerate with:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import pkv_inputs as inp  # noqa: E402


def tiny_outputs():
    case = inp.tiny_layer_case(seed=1001)
    s = inp.TINY
    cfg = oracle.ModelConfig(s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab, 1)
    kp, vp = case["k_pool"].copy(), case["v_pool"].copy()
    h = oracle.decode_layer(cfg, case["weights"]["layers"][0], case["hidden"], kp, vp,
                            case["block_tables"], case["ctx_lens"])
    return case, h, kp, vp


def appended(case, kp, vp):
    """The K and V the layer stored, [B, Hkv, D] each, read back at pos = c - 1."""
    ks, vs = [], []
    for b, c in enumerate(case["ctx_lens"]):
        blk = case["block_tables"][b][(c - 1) // 16]
        ks.append(kp[blk, :, (c - 1) % 16, :])
        vs.append(vp[blk, :, (c - 1) % 16, :])
    return np.stack(ks), np.stack(vs)


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main():
    case, h, kp, vp = tiny_outputs()
    k_new, v_new = appended(case, kp, vp)
    out = {
        "workload": "one decoder layer, hidden 256, 4/2 heads, D 64, FFN 688, batch 4, seed 1001",
        "ctx_lens": case["ctx_lens"].tolist(),
        "hidden_out": [float(x) for x in h.ravel()],
        "k_appended": [float(x) for x in k_new.ravel()],
        "v_appended": [float(x) for x in v_new.ravel()],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print(path)


if __name__ == "__main__":
    main()

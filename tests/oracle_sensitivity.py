"""How far a 1-ulp perturbation of the input, or fp32 instead of fp64 arithmetic,
moves the final pre-norm hidden state and the logits of the 28-layer
random-weight Qwen2.5-1.5B-shape model, evaluated with the oracle alone (CPU,
a few minutes; not collected by pytest).

The numbers set the envelope that the full-model GPU test applies to the final
hidden state:  python tests/oracle_sensitivity.py
"""
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import pkv_inputs as inp  # noqa: E402


def _report(a, b, name):
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    err = np.abs(a - b)
    bad = err > 2e-2 + 1e-2 * np.abs(b)
    print(f"{name}: max abs {err.max():.4f}  mean {err.mean():.5f}  outside the bar {bad.sum()} / {bad.size}"
          f"  (|ref| max {np.abs(b).max():.2f})")


def main():
    shape = inp.QWEN15
    t0 = time.time()
    w = inp.model_weights_torch(shape, seed=5456, device="cpu")
    host = {"embed": w["embed"].numpy(), "w_final_norm": w["w_final_norm"].numpy(),
            "w_lm_head": w["w_lm_head"].numpy(),
            "layers": [{k: (None if t is None else t.numpy()) for k, t in lw.items()} for lw in w["layers"]]}
    cfg = oracle.ModelConfig(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                             shape.vocab, shape.n_layers)
    rng = np.random.default_rng(1)
    lens = np.array([140, 150], np.int32)
    bt, nb = inp.deal_block_tables(rng, lens, 150)
    valid = inp.valid_slot_masks(bt, lens - 1, nb)
    pools = [inp.random_pools(rng, nb, shape.n_kv_heads, shape.head_dim, valid) for _ in range(shape.n_layers)]
    tok = np.array([5, 77], np.int32)

    def run(acc, perturb=False):
        kps = [p[0].copy() for p in pools]
        vps = [p[1].copy() for p in pools]
        h2 = dict(host)
        if perturb:  # flip the last mantissa bit of every 97th embedding element of both rows
            e = host["embed"].copy()
            for t in tok:
                e[t].view(np.uint16)[::97] ^= 1
            h2["embed"] = e
        return oracle.decode_step(cfg, h2, kps, vps, tok, bt, lens, acc=acc)

    l64, h64 = run(np.float64)
    l32, h32 = run(np.float32)
    lp, hp = run(np.float64, perturb=True)
    print(f"({time.time() - t0:.0f} s)")
    _report(h32, h64, "final hidden, fp32 vs fp64 oracle")
    _report(l32, l64, "logits, fp32 vs fp64 oracle")
    _report(hp, h64, "final hidden, 1-ulp input perturbation")
    _report(lp, l64, "logits, 1-ulp input perturbation")


if __name__ == "__main__":
    main()

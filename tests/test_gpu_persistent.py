"""The persistent batch-1 decode step (every layer's five fused ops in one
kernel with grid-wide barriers) against the per-op kernels, through the C ABI:
the same model and inputs stepped both ways give the same logits, final hidden
state and cache bytes, bit for bit, over many steps (contexts growing across
block boundaries; 4-wave attention partitions of 64 and 32 tokens per wave),
for f16 and E4M3 caches, eagerly and through a captured graph; and the
oracle's step agrees within the parity bar."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import dev, assert_parity, oracle_config, k_from_lib, v_from_lib

pytestmark = pytest.mark.gpu

# a few layers of the 1.5B and 7B shapes (their batch-1 projection plans are the
# ones the persistent kernel carries), small vocabularies
S15 = inp.Shape(1536, 12, 2, 128, 8960, 4096, 3)
S7 = inp.Shape(3584, 28, 4, 128, 18944, 2048, 2)


class Twin:
    def __init__(self, lib, shape, mc, seed, fp8=False):
        self.lib, self.shape, self.mc = lib, shape, mc
        self.w = inp.model_weights_torch(shape, seed=seed)
        self.m_on = lib.Model(shape, self.w, max_positions=mc + 1)
        self.m_on.set_persistent_batch1(True)
        self.m_off = lib.Model(shape, self.w, max_positions=mc + 1)  # per-op kernels: the default
        stride = (mc + 15) // 16
        self.nb = stride + 3
        kw = dict(dtype=lib.KV_FP8_E4M3, k_scales=[0.02] * shape.n_layers, v_scales=[0.015] * shape.n_layers) \
            if fp8 else {}
        self.caches = [lib.KVCache(shape.n_layers, self.nb, shape.n_kv_heads, shape.head_dim, **kw) for _ in range(2)]
        for c in self.caches:
            for layer in range(shape.n_layers):
                for t in c.layer(layer):
                    t.zero_()
        rng = np.random.default_rng(seed + 1)
        self.bt = rng.permutation(self.nb).astype(np.int32)[:stride].reshape(1, stride)
        self.tokens = rng.integers(0, shape.vocab, size=mc).astype(np.int32)
        self.ws = [torch.zeros(lib.step_workspace_bytes(m, c, 1, mc), dtype=torch.uint8, device="cuda")
                   for m, c in ((self.m_on, self.caches[0]), (self.m_off, self.caches[1]))]
        self.logits = [torch.empty(1, shape.vocab, dtype=torch.float16, device="cuda") for _ in range(2)]
        self.hidden = [torch.empty(1, shape.hidden, dtype=torch.float16, device="cuda") for _ in range(2)]
        self.d_bt = dev(self.bt)

    def step(self, t):
        lens = dev(np.array([t + 1], np.int32))
        tok = dev(self.tokens[t:t + 1])
        for i, m in enumerate((self.m_on, self.m_off)):
            self.lib.decode_step(m, self.caches[i], tok, self.d_bt, lens, self.mc, self.logits[i], self.ws[i],
                                 hidden_out=self.hidden[i])
        torch.cuda.synchronize()

    def same(self):
        eq = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))
        if not (eq(self.logits[0], self.logits[1]) and eq(self.hidden[0], self.hidden[1])):
            return False
        for layer in range(self.shape.n_layers):
            for a, b in zip(self.caches[0].layer(layer), self.caches[1].layer(layer)):
                if not torch.equal(a, b):
                    return False
        return True


def ran_persistent(ws, n_layers):
    """Whether the last step in this workspace ran the persistent kernel: its
    barrier words (zeroed at the step's start, 256-byte aligned) then hold the
    release count 5 L - 1 at word 64 and 32 times it at the root (word 128)."""
    w = ws.view(torch.int32).cpu().numpy()
    nbar = 5 * n_layers - 1
    for c in np.flatnonzero(w == nbar):
        o = c - 64
        if o >= 0 and o % 64 == 0 and w[o] == 0 and o + 128 < w.size and w[o + 128] == 32 * nbar:
            return True
    return False


@pytest.mark.parametrize("shape,mc,steps,fp8", [(S15, 200, 40, False), (S7, 600, 24, False), (S15, 200, 20, True)])
def test_persistent_batch1_step_equals_per_op_step(lib, shape, mc, steps, fp8):
    rig = Twin(lib, shape, mc, seed=8100 + shape.hidden + int(fp8), fp8=fp8)
    for t in range(steps):
        rig.step(t)
        assert rig.same(), f"step {t}"
        if t == 0:
            assert ran_persistent(rig.ws[0], shape.n_layers) and not ran_persistent(rig.ws[1], shape.n_layers)
    assert torch.isfinite(rig.logits[0].float()).all().item()


def test_persistent_batch1_graph_and_oracle(lib):
    """Replays of a captured persistent step equal the per-op eager step, and
    the oracle's step (over the GPU's cache history) is within the bar."""
    shape, mc = S15, 200
    rig = Twin(lib, shape, mc, seed=8200)
    tok_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = lib.Graph(rig.m_on, rig.caches[0], tok_d, rig.d_bt, lens_d, mc, rig.logits[0], rig.ws[0],
                  hidden_out=rig.hidden[0])
    host = {"embed": rig.w["embed"].cpu().numpy(), "w_final_norm": rig.w["w_final_norm"].cpu().numpy(),
            "w_lm_head": rig.w["w_lm_head"].cpu().numpy(),
            "layers": [{k: (None if t is None else t.cpu().numpy()) for k, t in lw.items()} for lw in rig.w["layers"]]}
    cfg = oracle_config(shape)
    for t in range(18):
        tok_d.copy_(torch.from_numpy(rig.tokens[t:t + 1]))
        lens_d.copy_(torch.from_numpy(np.array([t + 1], np.int32)))
        g.replay()
        lib.decode_step(rig.m_off, rig.caches[1], dev(rig.tokens[t:t + 1]), rig.d_bt,
                        dev(np.array([t + 1], np.int32)), mc, rig.logits[1], rig.ws[1], hidden_out=rig.hidden[1])
        torch.cuda.synchronize()
        assert rig.same(), f"replay {t}"
    # the oracle's next step over the GPU's cache (token t = 18)
    kp = [k_from_lib(rig.caches[0].layer(i)[0].cpu().numpy()) for i in range(shape.n_layers)]
    vp = [v_from_lib(rig.caches[0].layer(i)[1].cpu().numpy()) for i in range(shape.n_layers)]
    rig.step(18)
    rl, rh = oracle.decode_step(cfg, host, kp, vp, rig.tokens[18:19], rig.bt, np.array([19], np.int32),
                                acc=np.float32)
    assert_parity(rig.logits[0].cpu().numpy(), rl, "persistent step logits")
    assert_parity(rig.hidden[0].cpu().numpy(), rh, "persistent step hidden")
    g.close()


def test_persistent_option_errors(lib):
    shape = inp.Shape(256, 4, 2, 64, 688, 64, 1)
    m = lib.Model(shape, inp.model_weights_torch(shape, seed=1), max_positions=64)
    m.set_persistent_batch1(False)
    m.set_persistent_batch1(True)
    assert lib.lib().pkv_model_set_option(m.handle, 0, 5) == 1     # PKV_E_ARG: value
    assert lib.lib().pkv_model_set_option(m.handle, 7, 1) == 1     # PKV_E_ARG: option

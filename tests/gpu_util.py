"""Helpers shared by the GPU tests: move seeded inputs to the device and compare
with the oracle at the tolerance of the parity bar."""
import numpy as np
import torch

ATOL, RTOL = 2e-2, 1e-2   # |gpu - ref| <= 2e-2 + 1e-2 |ref| on f16 outputs


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def k_to_lib(k):
    """K pool [NB, Hkv, 16, D] (numpy or torch) -> the library's tile layout
    [NB, Hkv, D/c, 16, c] with 16-byte chunks: c = 8 (f16) or 16 (fp8 codes)."""
    nb, hkv, bs, d = k.shape
    c = 16 if k.dtype in (np.uint8, torch.uint8) else 8
    if isinstance(k, torch.Tensor):
        return k.reshape(nb, hkv, bs, d // c, c).permute(0, 1, 3, 2, 4).contiguous()
    return np.ascontiguousarray(k.reshape(nb, hkv, bs, d // c, c).transpose(0, 1, 3, 2, 4))


def k_from_lib(k):
    """Inverse of k_to_lib: [NB, Hkv, D/c, 16, c] -> [NB, Hkv, 16, D]."""
    nb, hkv, nc, bs, c = k.shape
    if isinstance(k, torch.Tensor):
        return k.permute(0, 1, 3, 2, 4).reshape(nb, hkv, bs, nc * c)
    return np.ascontiguousarray(k.transpose(0, 1, 3, 2, 4).reshape(nb, hkv, bs, nc * c))


def v_to_lib(v):
    """V pool [NB, Hkv, 16, D] (numpy or torch; token-major like K) -> the
    library's tile layout: f16 dim-major [NB, Hkv, D, 16]; fp8 codes
    [NB, Hkv, D/64, 4, 16, 4, 4] where dim d = 64 jj + 16 r + n and token
    t = 4 q4 + tt sit at [jj, q4, n, r, tt]."""
    nb, hkv, bs, d = v.shape
    if isinstance(v, torch.Tensor):
        if v.dtype != torch.uint8:
            return v.transpose(2, 3).contiguous()
        return v.reshape(nb, hkv, 4, 4, d // 64, 4, 16).permute(0, 1, 4, 2, 6, 5, 3).contiguous()
    if v.dtype != np.uint8:
        return np.ascontiguousarray(v.transpose(0, 1, 3, 2))
    return np.ascontiguousarray(v.reshape(nb, hkv, 4, 4, d // 64, 4, 16).transpose(0, 1, 4, 2, 6, 5, 3))


def v_from_lib(v):
    """Inverse of v_to_lib: the library's f16 [NB, Hkv, D, 16] or fp8
    [NB, Hkv, D/64, 4, 16, 4, 4] view -> [NB, Hkv, 16, D]."""
    if isinstance(v, torch.Tensor):
        if v.ndim == 4:
            return v.transpose(2, 3).contiguous()
        nb, hkv, ng = v.shape[:3]
        return v.permute(0, 1, 3, 6, 2, 5, 4).reshape(nb, hkv, 16, ng * 64).contiguous()
    if v.ndim == 4:
        return np.ascontiguousarray(v.transpose(0, 1, 3, 2))
    nb, hkv, ng = v.shape[:3]
    return np.ascontiguousarray(v.transpose(0, 1, 3, 6, 2, 5, 4).reshape(nb, hkv, 16, ng * 64))


def load_case_into_cache(pkv, case, num_layers=1, layer=0, cache=None):
    """A KVCache holding the case's pools at `layer` (other layers left uninitialised)."""
    fp8 = case.k_pool.dtype == np.uint8
    if cache is None:
        kw = {}
        if fp8:
            kw = dict(dtype=pkv.KV_FP8_E4M3, k_scales=[case.k_scale] * num_layers,
                      v_scales=[case.v_scale] * num_layers)
        cache = pkv.KVCache(num_layers, case.num_blocks, case.k_pool.shape[1], case.k_pool.shape[3], **kw)
    k, v = cache.layer(layer)
    k.copy_(torch.from_numpy(k_to_lib(case.k_pool)))
    v.copy_(torch.from_numpy(v_to_lib(case.v_pool)))
    return cache


def assert_parity(gpu, ref, what, atol=ATOL, rtol=RTOL):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside atol {atol} + rtol {rtol}; "
                           f"max abs err {err.max():.3e}")
    return float(err.max())


def weights_to_device(w):
    """numpy weight dict (pkv_inputs.model_weights) -> same structure of CUDA tensors."""
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return {
        "embed": t(w["embed"]),
        "w_final_norm": t(w["w_final_norm"]),
        "w_lm_head": t(w["w_lm_head"]),
        "layers": [{k: t(v) for k, v in lw.items()} for lw in w["layers"]],
    }


def oracle_config(shape, n_layers=None):
    import oracle
    return oracle.ModelConfig(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                              shape.vocab, shape.n_layers if n_layers is None else n_layers,
                              shape.rms_eps, shape.rope_theta)


def tie_aware_agree(gpu_tok, ref_logits):
    """Per row: the GPU's greedy token is the oracle's, or its oracle logit is
    within the parity bar of the oracle's maximum (a tie at the bar)."""
    ref = ref_logits.astype(np.float64)
    best = ref.max(-1)
    got = ref[np.arange(len(gpu_tok)), gpu_tok]
    return got >= best - (ATOL + RTOL * np.abs(best))


def calibrated(gpu, ref, ref_pert, what, min_inside=0.0):
    """GPU within the per-element bar, or within twice the oracle's own change
    under a 1-ulp perturbation of the same row's input (ref_pert; the largest
    change over that row's elements, rows being independent), and at least
    min_inside of all elements inside the per-element bar itself."""
    g, r, rp = (np.asarray(a, np.float64) for a in (gpu, ref, ref_pert))
    assert np.all(np.isfinite(g)), what
    err = np.abs(g - r)
    bar = ATOL + RTOL * np.abs(r)
    sens = np.abs(rp - r).max(axis=-1, keepdims=True)
    inside = np.mean(err <= bar)
    print(f"{what}: max abs err {err.max():.4f}, {100 * inside:.4f} % inside the bar, "
          f"oracle 1-ulp sensitivity per row {sens.min():.4f} .. {sens.max():.4f}")
    assert np.all(err <= np.maximum(bar, 2 * sens)), (what, err.max(), sens.max())
    assert inside >= min_inside, (what, inside)

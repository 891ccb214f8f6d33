"""Shared helpers for GPU parity tests: layer cache and oracle comparisons."""
import gc

import numpy as np
import torch

import oracle
from mixture_experts_layer_biased_amd import inputs, lcmoe
from tests.helpers import bf16_values, expert_getter

_cache = {}


def layer(name, **overrides):
    """(cfg, layer tensors on cuda) for a named config; at most one
    LongCat-shape layer is kept resident at a time."""
    cfg = inputs.CONFIGS[name].with_(**overrides)
    key = (name, tuple(sorted(overrides.items())))
    if key not in _cache:
        if cfg.d * cfg.n_ffn * cfg.inter >= 2 ** 30:
            for k in [k for k, (c, _) in _cache.items() if c.d * c.n_ffn * c.inter >= 2 ** 30]:
                del _cache[k]
            gc.collect()
            torch.cuda.empty_cache()
        _cache[key] = (cfg, inputs.make_layer(cfg, "cuda"))
    return _cache[key]


def max_rel_err(y, y_ref):
    """max_t ||y_t - yref_t||_inf / max(||yref_t||_inf, 1e-6 max_t ||yref_t||_inf)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    ref_n = np.abs(y_ref).max(axis=1)
    floor = 1e-6 * max(ref_n.max(), 1e-300)
    return float((np.abs(y - y_ref).max(axis=1) / np.maximum(ref_n, floor)).max())


def oracle_forward_rows(cfg, L, x, idx_gpu, tokens, cache=None):
    """Oracle output rows for `tokens`, evaluated on the GPU's selection
    (gates from the oracle's fp64 logits at those experts)."""
    xv = bf16_values(x[tokens])
    z = oracle.router_logits(xv, L["w_router"].cpu().numpy())
    idx = idx_gpu[tokens]
    g, _ = oracle.softmax_gates(z, idx)
    get = expert_getter(L, cfg.wdtype, cache=cache)
    return oracle.combine_given_routing(xv, idx, g, cfg.n_ffn, get, a8=cfg.wdtype == "fp8a8")


def router_error_scale(x_vals, w_router, d):
    """Per (token, expert) bound on |z_gpu - z_exact| for the router kernel.

    The kernel accumulates each split of the k range as a chain of MFMA
    updates (three per 16 k: lo, mid and hi bf16 planes of W_r), each adding
    exactly computed products to one fp32 accumulator, then sums the splits.
    Chain length <= 3*d/16 plus split adds; bound: (3*d/16 + 24) * 2^-24 *
    sum_k |W_ik x_tk|.
    """
    absdot = np.abs(x_vals) @ np.abs(np.asarray(w_router, dtype=np.float64)).T
    return (3 * d / 16 + 24) * 2.0 ** -24 * absdot

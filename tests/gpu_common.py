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
    experts = np.unique(idx[idx < cfg.n_ffn])  # the oracle's combine visits them in this order
    get = expert_getter(L, cfg.wdtype, cache=cache, prefetch=None if cache is not None else experts)
    return oracle.combine_given_routing(xv, idx, g, cfg.n_ffn, get, a8=cfg.wdtype == "fp8a8")


def cover_tokens(idx, n_ffn, extra=()):
    """Tokens whose selections together touch every FFN expert that any
    token selected: for each touched expert in id order not yet covered,
    its first token. Returns (sorted tokens including `extra`, number of
    touched FFN experts, number covered)."""
    idx = np.asarray(idx)
    touched = np.unique(idx[idx < n_ffn])
    covered = set()
    toks = set(int(t) for t in extra)
    for t in toks:
        covered.update(int(e) for e in idx[t] if e < n_ffn)
    for e in touched:
        if int(e) in covered:
            continue
        t = int(np.flatnonzero((idx == e).any(axis=1))[0])
        toks.add(t)
        covered.update(int(v) for v in idx[t] if v < n_ffn)
    return np.array(sorted(toks)), len(touched), len(covered & set(int(e) for e in touched))


def check_fp8a8_chain(cfg, L, x, res, tokens, tol_h=2e-2, tol_y=5e-2):
    """Stage-by-stage parity of the fp8-activation forward on `tokens`, from
    lcmoe_forward_inspect's intermediates (res), each stage checked on the
    GPU's own inputs to it so that an fp8 rounding flip upstream cannot
    consume the tolerance downstream:
      x codes and scales == the oracle's per-row quantizer, bit for bit;
      H (before quantization) vs the oracle's gate/up half on the GPU's x
        codes (one bf16 rounding of fp32-accumulated exact products: tol_h);
      H codes and scales == the oracle's quantizer on the GPU's H, bit for bit;
      y vs the oracle's MoE sum with each FFN slot's down half evaluated on
        the GPU's H codes (tol_y, the fp8 bar).
    Returns (max relative error of H, of y, FFN slot rows checked)."""
    tokens = np.asarray(sorted(set(int(t) for t in tokens)))
    K, N = cfg.k, cfg.n_ffn
    idx_all = res["idx"].cpu().numpy()
    idx = idx_all[tokens]
    xv = bf16_values(x[tokens])
    tsel = torch.as_tensor(tokens, device=x.device)
    # 1. token rows: codes and scales
    xq_ref, xs_ref = oracle.quantize_rows_fp8(xv.astype(np.float32))
    xq = res["xq"][tsel].cpu().numpy()
    xs = res["xs"][tsel].cpu().numpy()
    assert np.array_equal(xq, xq_ref), "x codes differ from the oracle's quantizer"
    assert np.array_equal(xs.view(np.uint32), xs_ref.view(np.uint32)), "x scales differ"
    # 2. the FFN slot rows of these tokens, in the expert-grouped slot order
    _, _, row_of_slot = oracle.permutation(idx_all, N)
    slots = (tokens[:, None] * K + np.arange(K)[None, :])
    rows = row_of_slot[slots]                       # [n, K], -1 for zero slots
    ffn = rows >= 0
    assert np.array_equal(ffn, idx < N)
    r_sel = torch.as_tensor(rows[ffn], device=x.device)
    h = bf16_values(res["h"][r_sel])
    hq = res["hq"][r_sel].cpu().numpy()
    hs = res["hs"][r_sel].cpu().numpy()
    # 3. H codes and scales: the oracle's quantizer on the GPU's own H
    hq_ref, hs_ref = oracle.quantize_rows_fp8(h.astype(np.float32))
    assert np.array_equal(hq, hq_ref), "H codes differ from the oracle's quantizer"
    assert np.array_equal(hs.view(np.uint32), hs_ref.view(np.uint32)), "H scales differ"
    # 4. per expert: gate/up half on the GPU's x codes, down half on its H codes
    xhat = oracle.dequant_rows_fp8(xq, xs)
    pos_t, pos_k = np.nonzero(ffn)                 # same order as rows[ffn]
    exp_of = idx[pos_t, pos_k]
    h_ref = np.zeros_like(h)
    out = np.zeros((len(tokens), K, cfg.d))
    experts = np.unique(exp_of)
    get = expert_getter(L, cfg.wdtype, prefetch=experts)
    for e in experts:
        sel = np.flatnonzero(exp_of == e)
        w13, w2 = get(e)
        h_ref[sel] = oracle.expert_gate_up(xhat[pos_t[sel]], w13)
        out[pos_t[sel], pos_k[sel]] = oracle.expert_down_fp8_rows(hq[sel], hs[sel], w2)
    err_h = max_rel_err(h, h_ref) if len(h) else 0.0  # no FFN slot among these tokens
    z = oracle.router_logits(xv, L["w_router"].cpu().numpy())
    g, _ = oracle.softmax_gates(z, idx)
    y_ref = oracle.combine_given_expert_outputs(xv, idx, g, N, out)
    err_y = max_rel_err(bf16_values(res["y"][tsel]), y_ref)
    print(f"{cfg.name} T={x.shape[0]} fp8 activations: {len(tokens)} tokens, {int(ffn.sum())} FFN "
          f"slot rows over {len(experts)} experts; codes and scales bit-exact; H max rel err "
          f"{err_h:.3e}, y max rel err {err_y:.3e}")
    assert err_h < tol_h, err_h
    assert err_y < tol_y, err_y
    return err_h, err_y, int(ffn.sum())


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

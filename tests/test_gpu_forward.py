"""GPU parity of the whole layer (routing, permutation, grouped SiLU-gated
expert GEMMs, combine with the zero-expert identity) against the oracle.

Tolerance (max relative error per token, infinity norm): 2e-2 with bf16
weights, 5e-2 with fp8 weights, against the fp64 oracle evaluated on the
GPU's own selection (selection parity is checked separately, bit-exact).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_biased_amd import inputs, lcmoe
from tests.gpu_common import (check_fp8a8_chain, cover_tokens, layer, max_rel_err,
                              oracle_forward_rows)
from tests.helpers import bf16_values

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp8": 5e-2, "fp8a8": 5e-2}


def run_forward(cfg, L, x):
    """lcmoe_forward; with fp8 activations lcmoe_forward_inspect, whose
    outputs are checked to be those of lcmoe_forward bit for bit and which
    also returns the activation codes, scales and pre-quantization H."""
    shape = lcmoe.shape_of(cfg)
    res = lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"],
                        L["w13_scale"], L["w2_scale"])
    if cfg.wdtype == "fp8a8":
        ins = lcmoe.forward_inspect(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"],
                                    L["w13_scale"], L["w2_scale"])
        torch.cuda.synchronize()
        for k in ("y", "idx", "gate", "counts"):
            assert torch.equal(ins[k], res[k]), f"lcmoe_forward_inspect {k} differs"
        res = ins
    torch.cuda.synchronize()
    return res


def check_rows(cfg, L, x, res, tokens, cache=None):
    if cfg.wdtype == "fp8a8":
        # stage by stage on the GPU's own intermediates (check_fp8a8_chain)
        return check_fp8a8_chain(cfg, L, x, res, tokens)[1]
    idx = res["idx"].cpu().numpy()
    y_ref = oracle_forward_rows(cfg, L, x, idx, tokens, cache=cache)
    y = bf16_values(res["y"][torch.as_tensor(tokens, device=x.device)])
    err = max_rel_err(y, y_ref)
    print(f"{cfg.name} T={x.shape[0]}: max rel err {err:.3e} over {len(tokens)} tokens")
    assert err < TOL[cfg.wdtype], err
    return err


def check_routing_consistent(cfg, L, x, res):
    # forward's selection and counts are those of the routing entry point
    r = lcmoe.route(lcmoe.shape_of(cfg), x, L["w_router"], L["bias"])
    torch.cuda.synchronize()
    assert torch.equal(r["idx"], res["idx"]) and torch.equal(r["gate"], res["gate"])
    cnt = np.bincount(res["idx"].cpu().numpy().ravel(), minlength=cfg.n_experts)
    assert np.array_equal(res["counts"].cpu().numpy(), cnt)


@pytest.mark.parametrize("name,T", [("tiny", 16), ("tiny", 1), ("tiny", 200), ("tiny", 777),
                                    ("small", 33), ("small", 300), ("small", 4096)])
def test_forward_all_tokens(name, T):
    # T spans a few rows per expert (decode-like), the mixed regime, and
    # experts split into several M-tiles.
    cfg, L = layer(name)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    res = run_forward(cfg, L, x)
    check_routing_consistent(cfg, L, x, res)
    check_rows(cfg, L, x, res, np.arange(T), cache={})


@pytest.mark.parametrize("inter", [128, 256, 384, 512])
@pytest.mark.parametrize("T", [1, 33, 300, 4096])
def test_forward_fp8_activations_all_tokens(T, inter):
    # fp8 weights and fp8 activations at the small shape, at every intermediate
    # size from the smallest the boundary accepts (128), from a few rows per
    # expert to several M-tiles, on the fp8-MFMA kernel.
    cfg, L = layer("small", wdtype="fp8a8", inter=inter)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    res = run_forward(cfg, L, x)
    check_routing_consistent(cfg, L, x, res)
    check_rows(cfg, L, x, res, np.arange(T), cache={})


@pytest.mark.parametrize("d,inter,T", [(96, 160, 1500), (160, 96, 1500), (1056, 544, 700)])
def test_forward_k_odd_multiple_of_32(d, inter, T):
    # d or I an odd multiple of 32: the large-M kernel's last k stage holds
    # 32 of its 64 k; T puts 2 M-tiles on some experts (tiny) or one (1056).
    cfg, L = layer("tiny", d=d, inter=inter)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    res = run_forward(cfg, L, x)
    counts = res["counts"].cpu().numpy()[: cfg.n_ffn]
    assert counts.max() > 32
    check_rows(cfg, L, x, res, np.arange(T), cache={})


@pytest.mark.parametrize("kw,T", [
    (dict(d=128, n_ffn=1, n_zero=0, k=1, inter=64), 100),      # one FFN expert: g = 1, y = FFN(x)
    (dict(n_ffn=8, n_zero=4, k=12), 50),                        # K = E: a dense mixture
    (dict(n_ffn=1536, n_zero=512, k=64, inter=32), 64),          # the largest E and K accepted
    (dict(n_ffn=2, n_zero=2040, k=2), 200),                      # almost only zero experts
])
def test_forward_degenerate_shapes(kw, T):
    cfg, L = layer("tiny", **kw)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    res = run_forward(cfg, L, x)
    check_routing_consistent(cfg, L, x, res)
    check_rows(cfg, L, x, res, np.arange(T), cache={})
    if cfg.n_ffn == 1 and cfg.n_zero == 0:
        assert np.all(res["gate"].cpu().numpy() == 1.0)


def _sample(x, n, extra_large=0):
    T = x.shape[0]
    toks = list(np.linspace(0, T - 1, n).astype(int))
    if extra_large:
        norms = x.float().norm(dim=1)
        toks += norms.topk(extra_large).indices.cpu().tolist()
    return np.array(sorted(set(toks)))


@pytest.mark.parametrize("name,n_sample,n_skew", [("decode", 64, 0), ("prefill", 6, 2),
                                                  ("fp8", 5, 0), ("fp8a8", 5, 0),
                                                  ("prefill32k", 4, 0), ("ep8_shard", 6, 0)])
def test_forward_longcat_shape_every_expert(name, n_sample, n_skew):
    # At the LongCat shape, in the launch configuration the bench times: every
    # decode token; at the larger batches a set of tokens whose selections
    # touch every FFN expert that the batch touches (so every expert's
    # weights, M-tiles and column slices feed a checked output), plus evenly
    # spaced tokens and the x20-scaled ones.
    cfg, L = layer(name)
    x = inputs.make_tokens(cfg, "cuda")
    res = run_forward(cfg, L, x)
    check_routing_consistent(cfg, L, x, res)
    counts = res["counts"].cpu().numpy()
    toks, touched, covered = cover_tokens(res["idx"].cpu().numpy(), cfg.n_ffn,
                                          extra=_sample(x, n_sample, n_skew))
    print(f"{name}: mean FFN experts/token {counts[:cfg.n_ffn].sum() / cfg.tokens:.3f}, "
          f"max rows {counts[:cfg.n_ffn].max()}; checking {len(toks)} tokens covering "
          f"{covered} of {touched} touched FFN experts")
    assert covered == touched == int((counts[:cfg.n_ffn] > 0).sum())
    check_rows(cfg, L, x, res, toks)


@pytest.mark.parametrize("name", ["prefill", "fp8", "fp8a8"])
def test_forward_maximum_tokens(name):
    # The largest batch the boundary accepts at the LongCat shape: the
    # large-M GEMMs address gathered x rows (bf16, or fp8 codes with fp8
    # activations) with 32-bit byte offsets, so T * d * 2 < 2^32 gives
    # T = 349,525 (about 5,500 rows per FFN expert, 18 M-tiles each). The
    # last tokens (x offsets just under 4 GiB) are checked along with the
    # first, for bf16 weights, fp8 weights and fp8 weights and activations
    # (stage by stage, through lcmoe_forward_inspect only: its equality with
    # lcmoe_forward is checked at the other sizes); one token more is
    # rejected.
    cfg, L = layer(name)
    T = (2 ** 32 - 1) // (cfg.d * 2)
    shape = lcmoe.shape_of(cfg)
    x = inputs.make_tokens(cfg, "cuda", tokens=T, skew=False)
    if cfg.wdtype == "fp8a8":
        res = lcmoe.forward_inspect(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"],
                                    L["w13_scale"], L["w2_scale"])
        torch.cuda.synchronize()
    else:
        res = run_forward(cfg, L, x)
    counts = res["counts"].cpu().numpy()
    assert counts.sum() == T * cfg.k
    print(f"{name} T={T}: FFN slots {counts[:cfg.n_ffn].sum()}, max rows {counts[:cfg.n_ffn].max()}")
    check_rows(cfg, L, x, res, np.array([0, 1, T // 2, T - 2, T - 1]))
    del res
    torch.cuda.empty_cache()
    # T + 1 tokens: UNSUPPORTED before anything is read or enqueued
    p = [t.data_ptr() for t in (x, L["w_router"], L["bias"], L["w13"], L["w2"])]
    s13 = L["w13_scale"].data_ptr() if L["w13_scale"] is not None else None
    s2 = L["w2_scale"].data_ptr() if L["w2_scale"] is not None else None
    st = lcmoe.lib().lcmoe_forward(ctypes.byref(shape), T + 1, p[0], p[1], p[2], p[3], s13, p[4],
                                   s2, p[0], p[0], p[0], p[0], p[0], 1 << 40, None)
    assert st == lcmoe.ERR_UNSUPPORTED
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,T", [("tiny", 16), ("small", 1000), ("decode", 64)])
def test_closed_form_all_zero_routing_gpu(name, T):
    # P-Y1: FFN experts biased out (K <= Z): y_t = (sum_k g_tk) x_t, rounded
    # once to bf16 (unit roundoff 2^-8) from an fp32 accumulation.
    cfg, L = layer(name)
    b = L["bias"].clone()
    b[: cfg.n_ffn] = -1e4
    L2 = dict(L, bias=b)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    res = run_forward(cfg, L2, x)
    idx = res["idx"].cpu().numpy()
    assert np.all(idx >= cfg.n_ffn)
    xv = bf16_values(x)
    z = oracle.router_logits(xv, L["w_router"].cpu().numpy())
    g, _ = oracle.softmax_gates(z, idx)
    want = g.sum(1)[:, None] * xv
    y = bf16_values(res["y"])
    assert np.all(np.abs(y - want) <= 2.0 ** -8 * np.abs(want) + 1e-5 * np.abs(want).max())
    # mirror: zero experts biased out -> no identity term
    bm = L["bias"].clone()
    bm[cfg.n_ffn:] = -1e4
    res_m = run_forward(cfg, dict(L, bias=bm), x)
    assert np.all(res_m["idx"].cpu().numpy() < cfg.n_ffn)
    n = min(T, 8)
    check_rows(cfg, dict(L, bias=bm), x, res_m, np.arange(n))


def test_forward_zero_tokens_and_determinism():
    cfg, L = layer("small")
    shape = lcmoe.shape_of(cfg)
    x0 = torch.empty(0, cfg.d, dtype=torch.bfloat16, device="cuda")
    counts = torch.full((cfg.n_experts,), 3, dtype=torch.int32, device="cuda")
    lcmoe.forward(shape, x0, L["w_router"], L["bias"], L["w13"], L["w2"],
                  out=dict(counts=counts))
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0
    # P-Y5: identical inputs give bitwise identical outputs
    x = inputs.make_tokens(cfg, "cuda", tokens=2500)
    a = run_forward(cfg, L, x)
    b = run_forward(cfg, L, x)
    for k in ("y", "idx", "gate", "counts"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("wdtype", ["bf16", "fp8a8"])
def test_forward_staged_matches_and_records_every_stage(wdtype):
    # lcmoe_forward_staged: the outputs of lcmoe_forward bit for bit, and one
    # event per stage boundary (NUM_STAGES + 1 caller events), in order
    cfg, L = layer("small", wdtype=wdtype)
    x = inputs.make_tokens(cfg, "cuda", tokens=777)
    shape = lcmoe.shape_of(cfg)
    ref = lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"],
                        L["w13_scale"], L["w2_scale"])
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    n = lcmoe.NUM_STAGES
    ev = (ctypes.c_void_p * (n + 1))()
    for i in range(n + 1):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        ev[i] = h
    got = lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"],
                        L["w13_scale"], L["w2_scale"], stage_events=ev)
    torch.cuda.synchronize()
    for k in ("y", "idx", "gate", "counts"):
        assert torch.equal(ref[k], got[k]), k
    ms = ctypes.c_float()
    for i in range(n):
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[i], ev[i + 1]) == 0
        assert ms.value >= 0, lcmoe.STAGES[i]
    for i in range(n + 1):
        hip.hipEventDestroy(ev[i])

"""GPU parity of the layer backward against the oracle.

The GPU computes the gradients of <dy, y> for the layer's forward; the oracle
(fp64) does the same on the GPU's own selection (the selection itself is
checked bit-exact elsewhere). Tolerances, max relative error per row against
the row's infinity norm:
  dx, dW_r (fp32 outputs): 2e-2. The expert operands are bf16 (x, dy, the
    weights), the slot-row intermediates dU are rounded to bf16 once before
    the dU W13 product (unit roundoff 2^-9), the rest accumulates in fp32.
  dW13, dW2 (bf16 outputs): 2e-2, the same rounding of dU / g*h plus one
    bf16 rounding of the result.
Untouched experts' weight gradients must be exactly zero.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_biased_amd import inputs, lcmoe
from tests.gpu_common import layer, max_rel_err
from tests.helpers import bf16_values, expert_getter

pytestmark = pytest.mark.gpu

TOL = 2e-2


def run_backward(cfg, L, x, dy, **kw):
    shape = lcmoe.shape_of(cfg)
    res = lcmoe.backward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], dy, **kw)
    torch.cuda.synchronize()
    return res


def gpu_selection(cfg, L, x):
    r = lcmoe.route(lcmoe.shape_of(cfg), x, L["w_router"], L["bias"])
    torch.cuda.synchronize()
    return r["idx"].cpu().numpy()


def oracle_backward(cfg, L, x, dy, idx, cache=None):
    get = expert_getter(L, "bf16", cache=cache)
    return oracle.layer_backward(bf16_values(x), L["w_router"].cpu().numpy(),
                                 L["bias"].cpu().numpy(), cfg.k, cfg.n_ffn, get,
                                 bf16_values(dy), idx=idx)


def untouched_are_zero(res, touched, n_ffn):
    mask = torch.ones(n_ffn, dtype=torch.bool, device=res["dw13"].device)
    mask[torch.as_tensor(sorted(touched), dtype=torch.long, device=mask.device)] = False
    z13 = res["dw13"].view(n_ffn, -1)[mask].view(torch.int16).abs().amax() if mask.any() else 0
    z2 = res["dw2"].view(n_ffn, -1)[mask].view(torch.int16).abs().amax() if mask.any() else 0
    return int(z13) == 0 and int(z2) == 0


def check_all(cfg, L, x, dy, res, idx, experts=None, cache=None, tol=TOL):
    ref = oracle_backward(cfg, L, x, dy, idx, cache=cache)
    errs = {"dx": max_rel_err(res["dx"].cpu().numpy(), ref["dx"]),
            "dw_router": max_rel_err(res["dw_router"].cpu().numpy(), ref["dw_router"])}
    touched = sorted(ref["dw13"])
    for e in touched if experts is None else [e for e in experts if e in ref["dw13"]]:
        errs[f"dw13[{e}]"] = max_rel_err(bf16_values(res["dw13"][e]), ref["dw13"][e])
        errs[f"dw2[{e}]"] = max_rel_err(bf16_values(res["dw2"][e]), ref["dw2"][e])
    worst = max(errs, key=errs.get)
    print(f"{cfg.name} T={x.shape[0]}: {len(touched)} experts touched, "
          f"worst {worst} {errs[worst]:.3e}, dx {errs['dx']:.3e}, dW_r {errs['dw_router']:.3e}")
    assert errs[worst] < tol, (worst, errs[worst])
    assert untouched_are_zero(res, touched, cfg.n_ffn)
    return errs


@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 16), ("tiny", 777),
                                    ("small", 33), ("small", 300), ("small", 4096)])
def test_backward_all_tokens(name, T):
    # T spans one token, several 128-row M tiles per expert and ragged tails
    # in every grouped GEMM (slot rows in the dgrad GEMMs, the reduction over
    # slots in the wgrad GEMMs).
    cfg, L = layer(name)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=T)
    res = run_backward(cfg, L, x, dy)
    check_all(cfg, L, x, dy, res, gpu_selection(cfg, L, x), cache={})


@pytest.mark.parametrize("d,inter,T", [(96, 160, 1500), (160, 96, 300)])
def test_backward_odd_multiples_of_32(d, inter, T):
    # d and I not multiples of the 128-wide tiles: partial N tiles and a
    # k range ending inside a 32-wide stage.
    cfg, L = layer("tiny", d=d, inter=inter)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=T)
    res = run_backward(cfg, L, x, dy)
    check_all(cfg, L, x, dy, res, gpu_selection(cfg, L, x), cache={})


@pytest.mark.parametrize("kw,T", [
    (dict(d=128, n_ffn=1, n_zero=0, k=1, inter=64), 100),      # one FFN expert: dz = 0
    (dict(d=128, n_ffn=1, n_zero=0, k=1, inter=64), 1000),     # every token on it: four 256-row
                                                                # dgrad tiles, a 16-stage wgrad k
    (dict(n_ffn=8, n_zero=4, k=12), 50),                        # K = E: a dense mixture
    (dict(n_ffn=1536, n_zero=512, k=64, inter=32), 64),          # the largest E and K accepted
])
def test_backward_degenerate_shapes(kw, T):
    cfg, L = layer("tiny", **kw)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=T)
    res = run_backward(cfg, L, x, dy)
    check_all(cfg, L, x, dy, res, gpu_selection(cfg, L, x), cache={})
    if cfg.n_ffn == 1 and cfg.n_zero == 0:
        # one expert: the softmax is constant, so the router gets no gradient
        assert float(res["dw_router"].abs().max()) == 0.0


def test_backward_zero_routing_closed_form():
    # FFN experts biased out: y_t = (sum_k g_tk) x_t, so
    # dx_t = G_t dy_t + W_r^T dz_t and every expert weight gradient is zero.
    cfg, L = layer("small")
    b = L["bias"].clone()
    b[: cfg.n_ffn] = -1e4
    L2 = dict(L, bias=b)
    T = 500
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=T)
    res = run_backward(cfg, L2, x, dy)
    idx = gpu_selection(cfg, L2, x)
    assert np.all(idx >= cfg.n_ffn)
    assert untouched_are_zero(res, [], cfg.n_ffn)
    check_all(cfg, L2, x, dy, res, idx, cache={})


def dw13_excess(xv, dyv, g, w13, w2, got, ref, tol=TOL):
    """Largest |GPU - oracle| / allowance over the elements of one expert's
    dW13 = sum over its slots of du x^T, where allowance = max(tol times the
    reference row's infinity norm, the fp32 error envelope of the element).

    A row of dW13 is tied to one entry of du per slot, du = [dh c silu'(a);
    dh silu(a)], and where that entry is small by cancellation (silu' has a
    root near a = -1.28; a, c or Q = W2^T dy near zero) the row's relative
    error is that of fp32 sums evaluated next to a root, not of the kernel.
    The envelope propagates, to first order, the GPU's documented arithmetic:
    a, c and Q accumulate exact bf16 products in fp32 (within
    (k/16 + 32) 2^-24 sum |products| for a reduction of length k, the bound
    used for the router's fp32 sums), silu and silu' are evaluated in fp32
    (a few ulps of their terms), du is rounded once to bf16 (2^-9, taken as
    2^-8 with the fp32 products), and dW13 once to bf16 (2^-8).
    With got=None, returns (envelope, tol bar) per element instead."""
    xv, dyv, g = np.asarray(xv), np.asarray(dyv), np.asarray(g)
    d = xv.shape[1]
    inter = w2.shape[1]
    u = xv @ w13.T
    a, c = u[:, :inter], u[:, inter:]
    Q = dyv @ w2
    dh = g[:, None] * Q
    gam = (d / 16 + 32) * 2.0 ** -24
    su = np.abs(xv) @ np.abs(w13).T
    da, dc = gam * su[:, :inter], gam * su[:, inter:]
    ddh = np.abs(g)[:, None] * gam * (np.abs(dyv) @ np.abs(w2)) + 2.0 ** -22 * np.abs(dh)
    sg = 1.0 / (1.0 + np.exp(-a))
    s1 = sg * (1.0 + a * (1.0 - sg))                   # silu'
    s2 = sg * (1.0 - sg) * (2.0 + a * (1.0 - 2.0 * sg))  # silu''
    ef = 8 * 2.0 ** -24
    du_g = dh * c * s1
    du_u = dh * a * sg
    e_g = (np.abs(dh * c) * (np.abs(s2) * da + ef * (sg + np.abs(a) * sg * (1 - sg)))
           + np.abs(dh * s1) * dc + np.abs(c * s1) * ddh + 2.0 ** -8 * np.abs(du_g))
    e_u = np.abs(dh * s1) * da + np.abs(a * sg) * ddh + 2.0 ** -8 * np.abs(du_u)
    env = np.concatenate([e_g, e_u], axis=1).T @ np.abs(xv) + 2.0 ** -8 * np.abs(ref)
    rown = np.abs(ref).max(axis=1, keepdims=True)
    bar = tol * np.maximum(rown, 1e-6 * rown.max())
    if got is None:
        return env, bar
    return float((np.abs(got - ref) / np.maximum(bar, env)).max())


def _sample(T, n):
    return np.array(sorted(set(np.linspace(0, T - 1, n).astype(int))))


@pytest.mark.parametrize("name", ["decode", "prefill", "prefill32k"])
def test_backward_longcat_shape(name):
    # LongCat shape. (1) A handful of tokens on their own: every output
    # checked (dW13/dW2 on three touched experts, the rest zero). (2) The
    # full batch: dx on sampled tokens and dW13/dW2 of at least 32 experts
    # against the oracle, and dW_r equal to the sum of the two half batches'
    # dW_r.
    cfg, L = layer(name)
    x = inputs.make_tokens(cfg, "cuda")
    dy = inputs.make_upstream_grad(cfg, "cuda")
    T = x.shape[0]
    toks = _sample(T, 4)
    xs, dys = x[torch.as_tensor(toks, device="cuda")], dy[torch.as_tensor(toks, device="cuda")]
    res = run_backward(cfg, L, xs, dys)
    idx_s = gpu_selection(cfg, L, xs)
    ffn = sorted(set(idx_s[idx_s < cfg.n_ffn].tolist()))
    check_all(cfg, L, xs, dys, res, idx_s, experts=[ffn[0], ffn[len(ffn) // 2], ffn[-1]])
    del res

    res = run_backward(cfg, L, x, dy)
    idx = gpu_selection(cfg, L, x)
    # dx on sampled tokens: a token's dx depends on that token alone
    toks = _sample(T, 6)
    ref = oracle_backward(cfg, L, x[torch.as_tensor(toks, device="cuda")],
                          dy[torch.as_tensor(toks, device="cuda")], idx[toks])
    err_dx = max_rel_err(res["dx"][torch.as_tensor(toks, device="cuda")].cpu().numpy(), ref["dx"])
    # weight gradients of at least 32 touched experts spread over the expert
    # ids and over the row counts (so over the weight-gradient kernel's k
    # lengths and the dgrad kernel's M tiles): 16 evenly spaced in id order,
    # 16 evenly spaced in row-count order (the least and most loaded among
    # them), and the last touched one; every touched expert at decode
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)[: cfg.n_ffn]
    touched = np.nonzero(counts)[0]
    if len(touched) <= 400 and T <= 64:
        pick = set(int(e) for e in touched)
    else:
        by_count = touched[np.argsort(counts[touched], kind="stable")]
        pick = set(int(e) for e in touched[np.linspace(0, len(touched) - 1, 16).astype(int)])
        pick |= set(int(e) for e in by_count[np.linspace(0, len(touched) - 1, 16).astype(int)])
        pick.add(int(touched[-1]))
    pick = sorted(pick)
    assert len(pick) >= min(32, len(touched))
    get = expert_getter(L, "bf16", prefetch=pick)
    wr = L["w_router"].cpu().numpy()
    errs, rel13 = {}, {}
    for e in pick:
        rows, ks = np.nonzero(idx == e)
        xe = x[torch.as_tensor(rows, device="cuda")]
        dye = dy[torch.as_tensor(rows, device="cuda")]
        xv, dyv = bf16_values(xe), bf16_values(dye)
        z = oracle.router_logits(xv, wr)
        g, _ = oracle.softmax_gates(z, idx[rows])
        w13_e, w2_e = get(e)
        ge = g[np.arange(len(rows)), ks]
        _, dw13, dw2, _ = oracle.expert_backward(xv, ge, dyv, w13_e, w2_e)
        got13 = bf16_values(res["dw13"][e])
        rel13[e] = max_rel_err(got13, dw13)
        # dW13 against tol or its fp32 error envelope (dw13_excess; 1 = at the allowance)
        errs[(e, int(counts[e]), "dw13")] = TOL * dw13_excess(xv, dyv, ge, w13_e, w2_e, got13, dw13)
        errs[(e, int(counts[e]), "dw2")] = max_rel_err(bf16_values(res["dw2"][e]), dw2)
    worst = max(errs, key=errs.get)
    rc = counts[pick]
    w13r = max(rel13, key=rel13.get)
    print(f"{name} T={T}: dx {err_dx:.3e} over {len(toks)} tokens; dW13/dW2 of {len(pick)} of "
          f"{len(touched)} touched experts (ids {pick[0]}..{pick[-1]}, {rc.min()}..{rc.max()} "
          f"rows): worst {worst} {errs[worst]:.3e} (dW13 as tol x allowance ratio; plain "
          f"per-row dW13 worst: expert {w13r} {rel13[w13r]:.3e})")
    assert err_dx < TOL
    assert errs[worst] < TOL, (worst, errs[worst])
    # dW_r is a sum over tokens: full batch = first half + second half. The
    # router's fp32 split-K summation order depends on the batch size, so a
    # token at a near tie may be routed differently in a half batch; such
    # tokens get dy = 0, which removes them from every gradient exactly.
    h = T // 2
    halves = np.concatenate([gpu_selection(cfg, L, x[:h]), gpu_selection(cfg, L, x[h:])])
    flipped = np.nonzero((np.sort(halves, 1) != np.sort(idx, 1)).any(1))[0]
    dy2 = dy.clone()
    dy2[torch.as_tensor(flipped, dtype=torch.long, device="cuda")] = 0
    out = dict(dw13=res["dw13"], dw2=res["dw2"])
    full = run_backward(cfg, L, x, dy2, out=out)["dw_router"].double()
    a = run_backward(cfg, L, x[:h], dy2[:h], out=out)["dw_router"].double()
    b = run_backward(cfg, L, x[h:], dy2[h:], out=out)["dw_router"].double()
    err_r = max_rel_err((a + b).cpu().numpy(), full.cpu().numpy())
    print(f"{name}: dW_r additivity {err_r:.3e} ({len(flipped)} tokens routed differently "
          f"in the half batches)")
    assert len(flipped) <= max(2, T // 1000)
    assert err_r < 1e-3


def test_backward_slot_buffers_past_4gib():
    # The LongCat shape at T = 65,536 (about 524k FFN slot rows): the gathered
    # slot-row buffers (x and dy rows, 6.4 GB each; the fp32 dX rows, 12.9 GB)
    # pass 4 GiB, so the later experts' rows sit past 2^32 bytes from the
    # buffer start and are reached through each expert's 64-bit base. dx on
    # tokens whose slot rows lie there, and dW13/dW2 of the first touched
    # expert and of the last two, against the oracle.
    cfg, L = layer("prefill")
    T = 65536
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=T)
    res = run_backward(cfg, L, x, dy)
    idx = gpu_selection(cfg, L, x)
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)[: cfg.n_ffn]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    row_bytes = cfg.d * 2
    touched = np.nonzero(counts)[0]
    pick = [int(touched[0]), int(touched[-2]), int(touched[-1])]
    assert offsets[pick[1]] * row_bytes >= 2 ** 32  # rows past 4 GiB in the x and dy slot buffers
    # tokens with a slot on the last touched expert (rows past 4 GiB), plus the first token
    t_last = np.nonzero((idx == pick[-1]).any(1))[0]
    toks = np.array(sorted(set([0] + t_last[:: max(1, len(t_last) // 4)][:4].tolist())))
    ref = oracle_backward(cfg, L, x[torch.as_tensor(toks, device="cuda")],
                          dy[torch.as_tensor(toks, device="cuda")], idx[toks])
    err_dx = max_rel_err(res["dx"][torch.as_tensor(toks, device="cuda")].cpu().numpy(), ref["dx"])
    get = expert_getter(L, "bf16", prefetch=pick)
    wr = L["w_router"].cpu().numpy()
    errs = {}
    for e in pick:
        rows, ks = np.nonzero(idx == e)
        xv = bf16_values(x[torch.as_tensor(rows, device="cuda")])
        dyv = bf16_values(dy[torch.as_tensor(rows, device="cuda")])
        z = oracle.router_logits(xv, wr)
        g, _ = oracle.softmax_gates(z, idx[rows])
        w13_e, w2_e = get(e)
        ge = g[np.arange(len(rows)), ks]
        _, dw13, dw2, _ = oracle.expert_backward(xv, ge, dyv, w13_e, w2_e)
        got13 = bf16_values(res["dw13"][e])
        errs[(e, "dw13")] = TOL * dw13_excess(xv, dyv, ge, w13_e, w2_e, got13, dw13)
        errs[(e, "dw2")] = max_rel_err(bf16_values(res["dw2"][e]), dw2)
    worst = max(errs, key=errs.get)
    print(f"T={T}: {int(counts.sum())} FFN slot rows; experts {pick} start at byte "
          f"{[int(offsets[e] * row_bytes) for e in pick]} of the slot buffers; dx {err_dx:.3e} over "
          f"{len(toks)} tokens; worst weight gradient {worst} {errs[worst]:.3e}")
    assert err_dx < TOL
    assert errs[worst] < TOL, (worst, errs[worst])
    del res
    torch.cuda.empty_cache()


def test_backward_zero_tokens_and_determinism():
    cfg, L = layer("small")
    shape = lcmoe.shape_of(cfg)
    x0 = torch.empty(0, cfg.d, dtype=torch.bfloat16, device="cuda")
    out = dict(dw_router=torch.full((cfg.n_experts, cfg.d), 7.0, device="cuda"),
               dw13=torch.ones(cfg.n_ffn, 2 * cfg.inter, cfg.d, dtype=torch.bfloat16,
                               device="cuda"),
               dw2=torch.ones(cfg.n_ffn, cfg.d, cfg.inter, dtype=torch.bfloat16, device="cuda"))
    lcmoe.backward(shape, x0, L["w_router"], L["bias"], L["w13"], L["w2"], x0, out=out)
    torch.cuda.synchronize()
    assert all(int(torch.count_nonzero(out[k])) == 0 for k in out)
    x = inputs.make_tokens(cfg, "cuda", tokens=2500)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=2500)
    a = run_backward(cfg, L, x, dy)
    b = run_backward(cfg, L, x, dy)
    for k in ("dx", "dw_router", "dw13", "dw2"):
        assert torch.equal(a[k], b[k]), k


def test_backward_staged_events_and_workspace_reuse():
    # the staged entry point gives the same gradients and records every
    # stage; a workspace sized for a larger batch serves a smaller one.
    cfg, L = layer("small")
    x = inputs.make_tokens(cfg, "cuda", tokens=1000)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=1000)
    ref = run_backward(cfg, L, x, dy)
    ws = torch.empty(lcmoe.backward_workspace_bytes(lcmoe.shape_of(cfg), 4096),
                     dtype=torch.uint8, device="cuda")
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    n = len(lcmoe.BWD_STAGES)
    ev = (ctypes.c_void_p * (n + 1))()
    for i in range(n + 1):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        ev[i] = h
    got = run_backward(cfg, L, x, dy, ws=ws, stage_events=ev)
    for k in ("dx", "dw_router", "dw13", "dw2"):
        assert torch.equal(ref[k], got[k]), k
    ms = ctypes.c_float()
    for i in range(n):
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[i], ev[i + 1]) == 0
        assert ms.value >= 0


@pytest.mark.parametrize("name,T", [("tiny", 16), ("tiny", 777), ("small", 300), ("small", 4096)])
def test_training_pair_all_tokens(name, T):
    # lcmoe_forward_train: the same y bit for bit as lcmoe_forward, plus every
    # FFN slot row's u = [W1 x; W3 x] in fp32 (checked against the fp64
    # oracle in the oracle's slot order; fp32 sums of exact bf16 products,
    # bar 1e-4 of each row's largest entry). lcmoe_backward_saved: every
    # gradient against the oracle, within the bar of the recomputing call.
    cfg, L = layer(name)
    shape = lcmoe.shape_of(cfg)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=T)
    u = torch.zeros(lcmoe.u_rows(shape, T), 2 * cfg.inter, dtype=torch.float32, device="cuda")
    ref = lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"])
    got = lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], u_save=u)
    torch.cuda.synchronize()
    for k in ("y", "idx", "gate", "counts"):
        assert torch.equal(ref[k], got[k]), k
    idx = got["idx"].cpu().numpy()
    _, perm, _ = oracle.permutation(idx, cfg.n_ffn)
    xv = bf16_values(x)
    get = expert_getter(L, "bf16", cache={})
    uv = u[: len(perm)].cpu().numpy().astype(np.float64)
    want = np.empty_like(uv)
    for r, slot in enumerate(perm):
        w13, _ = get(int(idx.ravel()[slot]))
        want[r] = w13 @ xv[slot // cfg.k]
    err_u = max_rel_err(uv, want)
    print(f"{name} T={T}: saved u max rel err {err_u:.3e} over {len(perm)} slot rows")
    assert err_u < 1e-4
    res = run_backward(cfg, L, x, dy, u_saved=u)
    check_all(cfg, L, x, dy, res, idx, cache={})


def test_training_pair_longcat_prefill():
    # LongCat prefill batch: the saved-u backward against the recomputing one
    # (same routing; u from the forward's GEMM instead of the backward's) and,
    # on sampled tokens, against the oracle.
    cfg, L = layer("prefill")
    shape = lcmoe.shape_of(cfg)
    x = inputs.make_tokens(cfg, "cuda")
    dy = inputs.make_upstream_grad(cfg, "cuda")
    T = x.shape[0]
    u = torch.empty(lcmoe.u_rows(shape, T), 2 * cfg.inter, dtype=torch.float32, device="cuda")
    lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], u_save=u)
    a = run_backward(cfg, L, x, dy, u_saved=u)
    da = {k: v.clone() for k, v in a.items()}
    del a
    b = run_backward(cfg, L, x, dy)
    err_dx = max_rel_err(da["dx"].cpu().numpy(), b["dx"].cpu().numpy())
    err_r = max_rel_err(da["dw_router"].cpu().numpy(), b["dw_router"].cpu().numpy())
    idx = gpu_selection(cfg, L, x)
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)[: cfg.n_ffn]
    e = int(np.argmax(counts))
    err_w = max(max_rel_err(bf16_values(da["dw13"][e]), bf16_values(b["dw13"][e])),
                max_rel_err(bf16_values(da["dw2"][e]), bf16_values(b["dw2"][e])))
    print(f"saved vs recomputed: dx {err_dx:.3e}, dW_r {err_r:.3e}, dW of expert {e} {err_w:.3e}")
    assert err_dx < TOL and err_r < TOL and err_w < TOL
    del b
    toks = _sample(T, 4)
    ref = oracle_backward(cfg, L, x[torch.as_tensor(toks, device="cuda")],
                          dy[torch.as_tensor(toks, device="cuda")], idx[toks])
    err = max_rel_err(da["dx"][torch.as_tensor(toks, device="cuda")].cpu().numpy(), ref["dx"])
    print(f"saved-u backward dx vs oracle {err:.3e}")
    assert err < TOL

"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: each test uses a closed form,
a brute-force enumeration, a library routine (torch CPU) or a number printed
on the "LongCat-Flash" llm-wiki entity page.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
from mixture_experts_layer_biased_amd import inputs
from tests.helpers import bf16_bits, bf16_values, expert_getter

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    # bf16 = high half of binary32: sign 1, exponent 8 (bias 127), mantissa 7.
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x3FC0, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, 2.0 ** -133, 1.5, 3.140625]
    got = oracle.bf16_bits_to_f64(pats)
    for g, w in zip(got, want):
        assert g == w
    assert np.signbit(got[3])
    # and against torch's bf16 -> fp32 conversion on every finite pattern
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    tv = torch.from_numpy(allp.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ov = oracle.bf16_bits_to_f64(allp)
    fin = np.isfinite(tv)
    assert np.array_equal(tv[fin], ov[fin])
    assert np.array_equal(np.isnan(tv), np.isnan(ov))


def test_e4m3fn_table_matches_torch_all_codes():
    # P-Y4: every code through torch.float8_e4m3fn.
    codes = torch.arange(256, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = oracle.e4m3fn_value_table()
    nan = np.isnan(ov)
    assert np.array_equal(nan, np.isnan(tv))
    assert nan.sum() == 2                     # S.1111.111 for both signs
    assert np.array_equal(ov[~nan], tv[~nan])
    assert ov[0x7E] == 448.0 and ov[0x01] == 2.0 ** -9 and ov[0x08] == 2.0 ** -6


def test_fp8_block_dequant_matches_torch():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(256, 384), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00       # no NaN codes in weights
    scales = rng.uniform(1e-5, 1e-3, size=(2, 3)).astype(np.float32)
    got = oracle.dequant_fp8_blocks(codes, scales)
    q = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    s = torch.from_numpy(scales).repeat_interleave(128, 0).repeat_interleave(128, 1)
    want = (q * s).numpy()
    assert got.dtype == np.float32
    assert np.array_equal(got, want)


def test_fp8_quantizer_round_trip_bound():
    # Inputs: E4M3 has 3 mantissa bits, so |w - fl32(q*s)| <= 2^-4 |w| + tiny.
    g = torch.Generator().manual_seed(7)
    w = torch.randn(256, 256, generator=g) * 0.02
    codes, scales = inputs.quantize_fp8_blocks(w)
    back = oracle.dequant_fp8_blocks(codes.numpy(), scales.numpy())
    err = np.abs(back - w.numpy())
    assert np.all(err <= 2.0 ** -4 * np.abs(w.numpy()) + 2.0 ** -9 * scales.max().item())


# --------------------------------------------------------------------------
# router logits
# --------------------------------------------------------------------------

def test_router_logits_exact_integer_arithmetic():
    # P-R1 inputs: every product is an integer multiple of 2^-13; compare with
    # an integer dot product done in int64.
    x, w, b = inputs.exact_router_inputs(T=8, d=6144, E=24, device="cpu", seed=3)
    xi = (x.float().numpy() * 8).astype(np.int64)
    wi = (w.numpy() * 1024).astype(np.int64)
    z_int = xi @ wi.T                                  # units of 2^-13
    z = oracle.router_logits(bf16_values(x), w.numpy())
    assert np.array_equal(z * 8192.0, z_int.astype(np.float64))
    assert np.all(np.abs(z_int) < 2 ** 24)             # exact in fp32 too
    assert np.array_equal(z.astype(np.float32).astype(np.float64), z)


# --------------------------------------------------------------------------
# top-K selection (P-R4 brute force, P-R5 invariants)
# --------------------------------------------------------------------------

def _outranks(sa, a, sb, b):
    return sa > sb or (sa == sb and a < b)


def _brute_force_topk(s_row, k):
    """The unique K-subset whose every member outranks every non-member."""
    E = len(s_row)
    found = []
    for sub in itertools.combinations(range(E), k):
        inside = set(sub)
        if all(_outranks(s_row[a], a, s_row[b], b)
               for a in inside for b in range(E) if b not in inside):
            found.append(sub)
    assert len(found) == 1
    sub = found[0]
    # selection order: each chosen expert outranks the ones listed after it
    order = sorted(sub, key=lambda i: (-float(s_row[i]), i))
    return list(order)


def test_topk_brute_force_tiny_config():
    cfg = inputs.CONFIGS["tiny"]
    L = inputs.make_layer(cfg, "cpu")
    x = inputs.make_tokens(cfg, "cpu")
    r = oracle.route(bf16_values(x), L["w_router"].numpy(), L["bias"].numpy(), cfg.k)
    s = oracle.selection_scores(r["z32"], L["bias"].numpy())
    for t in range(cfg.tokens):
        assert list(r["idx"][t]) == _brute_force_topk(s[t], cfg.k)


def test_topk_ties_and_signed_zero():
    z = np.array([[1.0, 2.0, 2.0, -0.0, 0.0, 2.0, -1.0, 0.0]], dtype=np.float32)
    b = np.zeros(8, dtype=np.float32)
    # ties at 2.0 resolve by index; -0 == +0 so 3,4,7 tie and resolve by index
    assert list(oracle.select_topk(z, b, 5)[0]) == [1, 2, 5, 0, 3]
    # bias enters in fp32: 1 + 2^-24 rounds to 1 -> tie with expert 0's score
    z2 = np.array([[1.0, 1.0]], dtype=np.float32)
    b2 = np.array([0.0, 2.0 ** -24], dtype=np.float32)
    assert list(oracle.select_topk(z2, b2, 1)[0]) == [0]
    b3 = np.array([0.0, 2.0 ** -23], dtype=np.float32)
    assert list(oracle.select_topk(z2, b3, 1)[0]) == [1]


@settings(max_examples=60, deadline=None)
@given(st.integers(2, 16).flatmap(lambda E: st.tuples(
    st.just(E), st.integers(1, E), st.integers(1, 6),
    st.lists(st.integers(-4, 4), min_size=E * 6, max_size=E * 6))))
def test_topk_brute_force_property(args):
    E, k, T, vals = args
    z = (np.array(vals[: E * T], dtype=np.float32).reshape(T, E)) / 4   # many ties
    b = np.zeros(E, dtype=np.float32)
    idx = oracle.select_topk(z, b, k)
    s = oracle.selection_scores(z, b)
    for t in range(T):
        assert list(idx[t]) == _brute_force_topk(s[t], k)


def test_routing_invariants_small_config():
    cfg = inputs.CONFIGS["small"]
    L = inputs.make_layer(cfg.with_(n_ffn=64), "cpu")
    x = inputs.make_tokens(cfg, "cpu", tokens=512)
    r = oracle.route(bf16_values(x), L["w_router"].numpy(), L["bias"].numpy(), cfg.k)
    idx, g, p = r["idx"], r["g"], r["p"]
    E = cfg.n_experts
    assert idx.min() >= 0 and idx.max() < E
    assert all(len(set(row)) == cfg.k for row in idx)
    assert r["counts"].sum() == cfg.k * 512
    assert np.all(g > 0) and np.all(g <= 1) and np.all(g.sum(1) <= 1 + 1e-12)
    assert np.allclose(p.sum(1), 1.0, rtol=0, atol=1e-12)


def test_permutation_matches_bucket_fill():
    rng = np.random.default_rng(5)
    T, K, N, E = 300, 6, 20, 30
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    offsets, perm, row_of_slot = oracle.permutation(idx, N)
    # independent construction: walk slots in order, append to per-expert buckets
    buckets = [[] for _ in range(N)]
    for j, e in enumerate(idx.ravel()):
        if e < N:
            buckets[e].append(j)
    want = [j for bkt in buckets for j in bkt]
    assert list(perm) == want
    assert list(np.diff(offsets)) == [len(bk) for bk in buckets]
    S = len(want)
    assert sorted(perm) == sorted(j for j in range(T * K) if idx.ravel()[j] < N)
    for r, j in enumerate(perm):
        assert row_of_slot[j] == r
    assert np.all(row_of_slot[idx.ravel() >= N] == -1)
    assert offsets[-1] == S


# --------------------------------------------------------------------------
# gates
# --------------------------------------------------------------------------

def test_softmax_gate_closed_forms():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 30, size=(50, 96))               # large spread, no overflow
    idx = np.argsort(-z, axis=1)[:, :6]
    g, p = oracle.softmax_gates(z, idx)
    assert np.all(np.isfinite(p))
    assert np.allclose(p.sum(1), 1, atol=1e-12)
    # ratio identity p_i / p_j = exp(z_i - z_j) for moderate differences
    zz = rng.normal(0, 1, size=(4, 10))
    _, pp = oracle.softmax_gates(zz, np.zeros((4, 1), np.int64))
    assert np.allclose(pp[:, 3] / pp[:, 7], np.exp(zz[:, 3] - zz[:, 7]), rtol=1e-13)
    # equal logits -> uniform 1/E
    _, pu = oracle.softmax_gates(np.zeros((2, 12)), np.zeros((2, 1), np.int64))
    assert np.allclose(pu, 1 / 12, rtol=1e-15)


# --------------------------------------------------------------------------
# layer output (P-Y1, P-Y2, P-Y3)
# --------------------------------------------------------------------------

def _tiny_layer(**kw):
    cfg = inputs.CONFIGS["tiny"].with_(**kw)
    L = inputs.make_layer(cfg, "cpu")
    return cfg, L


def test_closed_form_all_zero_routing():
    # P-Y1: biases push every FFN expert below every zero expert (K <= Z).
    cfg, L = _tiny_layer()
    x = inputs.make_tokens(cfg, "cpu")
    xv = bf16_values(x)
    b = L["bias"].numpy().copy()
    b[: cfg.n_ffn] = -1e4
    y, r = oracle.forward(xv, L["w_router"].numpy(), b, cfg.k, cfg.n_ffn,
                          expert_getter(L, "bf16"))
    assert np.all(r["idx"] >= cfg.n_ffn)
    assert np.allclose(y, r["g"].sum(1)[:, None] * xv, rtol=1e-14, atol=0)
    # with a zero router every gate is exactly 1/E: y = (K/E) x
    y0, r0 = oracle.forward(xv, np.zeros_like(L["w_router"].numpy()), b, cfg.k,
                            cfg.n_ffn, expert_getter(L, "bf16"))
    assert np.allclose(y0, (cfg.k / cfg.n_experts) * xv, rtol=1e-14, atol=0)
    # mirror: zero experts pushed out -> no identity term at all
    bm = L["bias"].numpy().copy()
    bm[cfg.n_ffn:] = -1e4
    ym, rm = oracle.forward(xv, L["w_router"].numpy(), bm, cfg.k, cfg.n_ffn,
                            expert_getter(L, "bf16"))
    assert np.all(rm["idx"] < cfg.n_ffn)
    get = expert_getter(L, "bf16")
    want = np.zeros_like(xv)
    for t in range(cfg.tokens):
        for k in range(cfg.k):
            w13, w2 = get(int(rm["idx"][t, k]))
            want[t] += rm["g"][t, k] * oracle.expert_ffn(xv[t:t + 1], w13, w2)[0]
    assert np.allclose(ym, want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("name,subset", [("tiny", None), ("small", 256)])
def test_sparse_matches_dense_masked(name, subset):
    # P-Y2: permutation/gather-free evaluation of the same sum.
    cfg = inputs.CONFIGS[name]
    L = inputs.make_layer(cfg, "cpu")
    x = inputs.make_tokens(cfg, "cpu", tokens=subset)
    xv = bf16_values(x)
    get = expert_getter(L, "bf16", cache={})
    y, r = oracle.forward(xv, L["w_router"].numpy(), L["bias"].numpy(), cfg.k,
                          cfg.n_ffn, get)
    pm = np.zeros_like(r["p"])
    np.put_along_axis(pm, r["idx"].astype(np.int64), r["g"], axis=1)
    yd = oracle.dense_masked_forward(xv, pm, cfg.n_ffn, get)
    scale = np.abs(yd).max()
    assert np.abs(y - yd).max() <= 1e-10 * scale


def _torch_ffn(x, w13, w2):
    inter = w2.shape[1]
    u = x @ w13.T
    return (F.silu(u[:, :inter]) * u[:, inter:]) @ w2.T


def test_library_special_cases():
    # P-Y3 (a): one FFN expert, no zero experts, K=1 -> exactly one SwiGLU FFN.
    cfg, L = _tiny_layer(n_ffn=1, n_zero=0, k=1)
    x = inputs.make_tokens(cfg, "cpu")
    xv = bf16_values(x)
    get = expert_getter(L, "bf16")
    y, r = oracle.forward(xv, L["w_router"].numpy(), L["bias"].numpy(), 1, 1, get)
    w13, w2 = get(0)
    want = _torch_ffn(torch.from_numpy(xv), torch.from_numpy(w13), torch.from_numpy(w2)).numpy()
    assert np.allclose(r["g"], 1.0, rtol=0, atol=0)
    assert np.allclose(y, want, rtol=1e-12, atol=1e-14)

    # P-Y3 (b): Z=0 -> plain softmax top-K MoE, no renormalisation (torch ops).
    # A nonzero bias: it must steer the selection and must not reach the gates.
    cfg, L = _tiny_layer(n_zero=0, bias_std=0.3)
    x = inputs.make_tokens(cfg, "cpu")
    xv = bf16_values(x)
    get = expert_getter(L, "bf16")
    y, r = oracle.forward(xv, L["w_router"].numpy(), L["bias"].numpy(), cfg.k, cfg.n_ffn, get)
    unbiased = oracle.select_topk(r["z32"], np.zeros(cfg.n_experts, np.float32), cfg.k)
    assert not np.array_equal(np.sort(unbiased, 1), np.sort(r["idx"], 1))
    xt = torch.from_numpy(xv)
    zt = xt @ L["w_router"].double().T
    pt = torch.softmax(zt, dim=1)
    top = torch.topk(zt.float() + L["bias"], cfg.k, dim=1).indices
    want = torch.zeros_like(xt)
    for e in range(cfg.n_ffn):
        w13, w2 = get(e)
        ye = _torch_ffn(xt, torch.from_numpy(w13), torch.from_numpy(w2))
        sel = (top == e).any(dim=1).double()
        want += (sel * pt[:, e])[:, None] * ye
    assert np.allclose(y, want.numpy(), rtol=1e-12, atol=1e-14)

    # P-Y3 (c): K=E -> the dense softmax mixture over FFN and zero experts.
    cfg, L = _tiny_layer(k=12)
    x = inputs.make_tokens(cfg, "cpu")
    xv = bf16_values(x)
    get = expert_getter(L, "bf16")
    y, r = oracle.forward(xv, L["w_router"].numpy(), L["bias"].numpy(), 12, cfg.n_ffn, get)
    xt = torch.from_numpy(xv)
    pt = torch.softmax(xt @ L["w_router"].double().T, dim=1)
    want = pt[:, cfg.n_ffn:].sum(1, keepdim=True) * xt
    for e in range(cfg.n_ffn):
        w13, w2 = get(e)
        want += pt[:, e:e + 1] * _torch_ffn(xt, torch.from_numpy(w13), torch.from_numpy(w2))
    assert np.allclose(y, want.numpy(), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# bias update (P-B1, P-B2)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,k_e,t_all", [(8, 3, 2.0, 16), (512, 12, 8.0, 16384), (64, 6, 4.0, 4096)])
def test_bias_update_fixed_point_and_signs(N, K, k_e, t_all):
    E = N + N // 2
    rng = np.random.default_rng(N)
    b = rng.normal(0, 0.1, E).astype(np.float32)
    target = k_e * t_all / N
    assert target == int(target)
    counts = np.full(E, 5, dtype=np.int64)
    counts[:N] = int(target)
    nb = oracle.bias_update(b, counts, N, K, 1e-3, k_e, t_all)
    assert np.array_equal(nb.view(np.uint32), b.view(np.uint32))      # exact fixed point
    counts2 = counts.copy()
    counts2[0] += 3
    counts2[1] -= 3
    nb2 = oracle.bias_update(b, counts2, N, K, 0.5, k_e, t_all)
    assert nb2[0] < b[0] and nb2[1] > b[1]                             # over target -> down
    assert np.array_equal(nb2[N:], b[N:])                              # zero experts untouched
    # magnitude against the law as printed: mu*(K_e/K/N - T_i/(K*T_all))
    d0 = 0.5 * (k_e / K / N - counts2[0] / (K * t_all))
    assert math.isclose(float(nb2[0]) - float(b[0]), d0, rel_tol=1e-3, abs_tol=1e-7)


@pytest.mark.parametrize("k_e,mu", [(1.0, 0.3), (2.5, 0.3)])
def test_bias_loop_converges_to_target(k_e, mu):
    # P-B2 on the tiny layer shape, fresh tokens each step (T=4096): after 300
    # steps the mean FFN-expert count per token is within 1% of K_e, as the
    # page reports for the trained model.
    golden = json.load(open(os.path.join(GOLDEN, "longcat_shape.json")))
    tol = golden["bias_controller"]["converged_fluctuation_below"]
    cfg = inputs.CONFIGS["tiny"]
    L = inputs.make_layer(cfg, "cpu")
    wr = L["w_router"].numpy()
    b = np.zeros(cfg.n_experts, dtype=np.float32)
    T = 4096
    hist, loads = [], []
    for j in range(300):
        x = inputs.make_tokens(cfg, "cpu", stream=100 + j, tokens=T)
        r = oracle.route(bf16_values(x), wr, b, cfg.k)
        hist.append(r["counts"][: cfg.n_ffn].sum() / T)
        loads.append(r["counts"][: cfg.n_ffn] / T)
        b = oracle.bias_update(b, r["counts"], cfg.n_ffn, cfg.k, mu, k_e, T)
    tail = np.array(hist[-50:])
    assert abs(tail.mean() - k_e) / k_e < tol
    per_expert = np.array(loads[-50:]).mean(0)
    assert np.allclose(per_expert, k_e / cfg.n_ffn, rtol=0.05)
    assert np.all(b[cfg.n_ffn:] == 0)


# --------------------------------------------------------------------------
# the page's own numbers: layer shape and activated parameters
# --------------------------------------------------------------------------

def test_page_shape_supports_gated_expert_and_k_e_8():
    gd = json.load(open(os.path.join(GOLDEN, "longcat_shape.json")))
    d, I = gd["d_model"], gd["ffn_expert_intermediate"]
    L, K = gd["n_layers_excluding_mtp"], gd["experts_per_token_including_zero"]
    N, Z = gd["n_ffn_experts"], gd["n_zero_experts"]
    act = gd["activated_params_billion"]
    # parameter count of one expert as the oracle evaluates it
    w13 = np.zeros((2 * 4, 3)); w2 = np.zeros((3, 4))
    assert oracle.expert_ffn(np.zeros((1, 3)), w13, w2).shape == (1, 3)
    per_expert = 2 * I * d + d * I                       # gate + up + down
    per_slot_b = per_expert * L / 1e9
    # K slots of FFN experts vs all-zero routing span the activated range
    assert math.isclose(K * per_slot_b, act["max"] - act["min"], rel_tol=0.01)
    # a two-matrix expert would not
    assert not math.isclose(K * 2 * I * d * L / 1e9, act["max"] - act["min"], rel_tol=0.1)
    # mean activation implies ~8 FFN experts per token = K*N/E (symmetric point)
    k_e_mean = (act["mean"] - act["min"]) / per_slot_b
    assert math.isclose(k_e_mean, K * N / (N + Z), rel_tol=0.01)


# ----------------------------------------------------------------------------
# Router-side statistics: device-level balance loss with the zero group, and
# the hidden z-loss ("LongCat-Flash" section 2.1 load-balance control; the
# training-stability section, activation stability).
# ----------------------------------------------------------------------------


def _random_counts(rng, T, K, E):
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    return np.bincount(idx.ravel(), minlength=E)


@pytest.mark.parametrize("N,Z,D", [(8, 4, 2), (8, 4, 8), (64, 32, 8), (16, 0, 4)])
def test_balance_stats_uniform_logits(N, Z, D):
    # z = 0: every expert has probability 1/E, so P_j = |G_j| / E.
    E, K, T = N + Z, 3, 5
    rng = np.random.default_rng(1)
    counts = _random_counts(rng, T, K, E)
    _, _, P = oracle.load_balance_stats(np.zeros((T, E)), counts, N, Z, K, D, 2.0, 1.0)
    want = np.array([N / D / E] * D + [Z / E])
    assert np.allclose(P, want, rtol=0, atol=1e-15)


def test_balance_stats_target_routing_has_unit_f():
    # N=8, Z=4, K=3, K_e=2, D=2, T=4: 12 slots, targets 1/3 per FFN group and
    # 1/3 for the zero group, i.e. 4 slots each -> f = 1 for all three groups,
    # so L_LB = alpha * sum_j P_j = alpha for any logits.
    N, Z, K, D, T = 8, 4, 3, 2, 4
    counts = np.array([1, 1, 2, 0, 0, 3, 1, 0, 2, 0, 1, 1])
    rng = np.random.default_rng(2)
    z = rng.normal(size=(T, N + Z)) * 3
    L, f, P = oracle.load_balance_stats(z, counts, N, Z, K, D, 2.0, 0.25)
    assert np.allclose(f, 1.0, rtol=0, atol=1e-15)
    assert math.isclose(P.sum(), 1.0, rel_tol=1e-14)
    assert math.isclose(L, 0.25, rel_tol=1e-14)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_balance_stats_shares_and_shift_invariance(seed):
    N, Z, K, D, T, k_e = 64, 32, 6, 8, 50, 4.0
    rng = np.random.default_rng(seed)
    z = rng.normal(size=(T, N + Z))
    counts = _random_counts(rng, T, K, N + Z)
    L, f, P = oracle.load_balance_stats(z, counts, N, Z, K, D, k_e, 1.0)
    target = np.array([k_e / (K * D)] * D + [(K - k_e) / K])
    assert math.isclose(float(np.sum(f * target)), 1.0, rel_tol=1e-13)  # shares sum to 1
    # softmax is invariant to a per-token shift of the logits
    L2, f2, P2 = oracle.load_balance_stats(z + rng.normal(size=(T, 1)) * 40, counts, N, Z, K, D,
                                           k_e, 1.0)
    assert np.allclose(P2, P, rtol=1e-12, atol=0) and np.array_equal(f2, f)
    # relabelling experts inside one group changes nothing
    perm = np.arange(N + Z)
    perm[:N // D] = perm[:N // D][::-1]
    L3, _, P3 = oracle.load_balance_stats(z[:, perm], counts[perm], N, Z, K, D, k_e, 1.0)
    assert np.allclose(P3, P, rtol=1e-13) and math.isclose(L3, L, rel_tol=1e-13)


def test_balance_stats_reduce_to_switch_style_loss():
    # One expert per group, no zero experts, K_e = K: f_i = N * c_i / (T K)
    # and P_i = mean softmax probability -- the familiar per-expert auxiliary
    # balance loss, evaluated here with torch's softmax.
    N, K, T = 16, 4, 40
    rng = np.random.default_rng(5)
    z = rng.normal(size=(T, N)) * 2
    counts = _random_counts(rng, T, K, N)
    L, f, P = oracle.load_balance_stats(z, counts, N, 0, K, N, float(K), 0.5)
    Pt = torch.softmax(torch.tensor(z, dtype=torch.float64), dim=1).mean(0).numpy()
    ft = N * counts / (T * K)
    assert np.allclose(P[:N], Pt, rtol=1e-13) and np.allclose(f[:N], ft, rtol=1e-14)
    assert f[N] == 0.0 and P[N] == 0.0
    assert math.isclose(L, 0.5 * float(np.sum(ft * Pt)), rel_tol=1e-13)


def test_hidden_z_loss_closed_forms():
    d, lam = 6144, 1e-3
    assert math.isclose(oracle.hidden_z_loss(np.zeros((3, d)), lam), lam * math.log(d) ** 2,
                        rel_tol=1e-14)
    c = -2.5  # |h| = 2.5 everywhere
    assert math.isclose(oracle.hidden_z_loss(np.full((2, d), c), lam),
                        lam * (2.5 + math.log(d)) ** 2, rel_tol=1e-14)
    # one large entry: lse = 80 + log(1 + (d - 1) e^-80) = 80 to double precision
    h = np.zeros((1, d))
    h[0, 17] = -80.0
    assert math.isclose(oracle.hidden_z_loss(h, 1.0), 80.0 ** 2, rel_tol=1e-15)
    # against torch.logsumexp on random states (sign-symmetric in h)
    rng = np.random.default_rng(3)
    h = rng.normal(size=(7, 333)) * 3
    lse = torch.logsumexp(torch.tensor(np.abs(h)), dim=1).numpy()
    want = 0.3 / 7 * float(np.sum(lse ** 2))
    assert math.isclose(oracle.hidden_z_loss(h, 0.3), want, rel_tol=1e-13)
    assert math.isclose(oracle.hidden_z_loss(-h, 0.3), want, rel_tol=1e-13)
    assert oracle.hidden_z_loss(np.zeros((0, 4)), 1.0) == 0.0


# ----------------------------------------------------------------------------
# fp8 activations (reading R-a8): the E4M3FN encoder, per-row quantization,
# and the expert with quantized input and intermediate rows.
# ----------------------------------------------------------------------------


def test_e4m3fn_encoder_matches_torch():
    vals = oracle.e4m3fn_value_table()
    fin = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))
    mids = (fin[1:] + fin[:-1]) / 2.0                 # exact ties: half-to-even
    rng = np.random.default_rng(0)
    rnd = np.exp(rng.uniform(-16, np.log(448.0), 20000)) * rng.choice([-1, 1], 20000)
    edge = np.array([0.0, -0.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 0.6 * 2.0 ** -9, 448.0, 440.0,
                     2.0 ** -6 * (1 - 2.0 ** -4)])
    v = np.concatenate([fin, -fin, mids, -mids, rnd, edge]).astype(np.float32)
    got = oracle.e4m3fn_encode(v)
    want = torch.tensor(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    # every code decodes back to its value
    assert np.array_equal(oracle.e4m3fn_encode(fin.astype(np.float32)),
                          np.array([np.flatnonzero(vals == f)[0] for f in fin], dtype=np.uint8))


def test_quantize_rows_fp8_round_trip():
    rng = np.random.default_rng(1)
    v = (rng.normal(size=(40, 300)) * np.exp(rng.uniform(-6, 6, (40, 1)))).astype(np.float32)
    v[3] = 0.0
    codes, s = oracle.quantize_rows_fp8(v)
    assert s[3] == 1.0 and not codes[3].any()
    back = oracle.dequant_rows_fp8(codes, s)
    amax = np.abs(v).max(axis=1)
    assert np.allclose(s[amax > 0], (amax[amax > 0] / np.float32(448)).astype(np.float32), rtol=0)
    normal = np.abs(v) >= 2.0 ** -6 * s[:, None]
    err = np.abs(back - v)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(v[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * np.broadcast_to(s[:, None], v.shape)[~normal] * (1 + 1e-6))
    # the row maximum lands on +-448 (or one step below it after rounding)
    top = np.abs(oracle.e4m3fn_value_table()[codes[amax > 0, np.abs(v[amax > 0]).argmax(1)]])
    assert np.all(top >= 416.0)


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(2)
    v = rng.normal(size=5000) * np.exp(rng.uniform(-20, 20, 5000))
    got = oracle.round_to_bf16(v)
    want = torch.tensor(v).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want)


def test_a8_expert_matches_torch_composition():
    # The same expert built from torch primitives: per-row scales, torch's
    # float8_e4m3fn cast, float64 matmuls, torch's bf16 rounding of H.
    rng = np.random.default_rng(3)
    d, inter, m = 256, 128, 9
    x = rng.normal(size=(m, d)).astype(np.float32)
    w13 = (rng.normal(size=(2 * inter, d)) * 0.05).astype(np.float32)
    w2 = (rng.normal(size=(d, inter)) * 0.05).astype(np.float32)

    def tq(a):  # torch per-row quantize-dequantize
        a = torch.tensor(a, dtype=torch.float32)
        amax = a.abs().amax(dim=1)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (a / s[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).double()
        return (q * s.double()[:, None])

    xh = tq(x)
    u = xh @ torch.tensor(w13, dtype=torch.float64).T
    h = (torch.nn.functional.silu(u[:, :inter]) * u[:, inter:]).float().to(torch.bfloat16)
    want = (tq(h.float().numpy()) @ torch.tensor(w2, dtype=torch.float64).T).numpy()
    xq, xs = oracle.quantize_rows_fp8(x)
    got = oracle.expert_ffn_a8(oracle.dequant_rows_fp8(xq, xs), w13, w2)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # and it is a perturbation of the unquantized expert of the expected size
    ref = oracle.expert_ffn(x, w13, w2)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert 1e-4 < rel < 0.1


def test_expert_halves_match_torch():
    # The two halves of the expert against torch primitives: silu gate times
    # up (gate rows first; swapping the halves or transposing W13 changes the
    # result), and the down half on given per-row fp8 codes (torch's
    # float8_e4m3fn decode times the row scale, then W2^T).
    rng = np.random.default_rng(4)
    d, inter, m = 192, 96, 7
    x = rng.normal(size=(m, d))
    w13 = rng.normal(size=(2 * inter, d)) * 0.05
    w2 = rng.normal(size=(d, inter)) * 0.05
    X, W13 = torch.tensor(x), torch.tensor(w13)
    want_h = (torch.nn.functional.silu(X @ W13[:inter].T) * (X @ W13[inter:].T)).numpy()
    got_h = oracle.expert_gate_up(x, w13)
    assert np.allclose(got_h, want_h, rtol=1e-13, atol=1e-13 * np.abs(want_h).max())
    swapped = (torch.nn.functional.silu(X @ W13[inter:].T) * (X @ W13[:inter].T)).numpy()
    assert np.abs(got_h - swapped).max() > 1e-2 * np.abs(want_h).max()
    assert np.allclose(oracle.expert_ffn(x, w13, w2), want_h @ w2.T, rtol=1e-12,
                       atol=1e-12 * np.abs(want_h @ w2.T).max())
    codes = rng.integers(0, 256, size=(m, inter), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11            # no NaN codes
    scales = np.exp(rng.uniform(-8, 2, m)).astype(np.float32)
    q = torch.tensor(codes).view(torch.float8_e4m3fn).double()
    want_y = ((q * torch.tensor(scales).double()[:, None]) @ torch.tensor(w2).T).numpy()
    got_y = oracle.expert_down_fp8_rows(codes, scales, w2)
    assert np.allclose(got_y, want_y, rtol=1e-13, atol=1e-13 * np.abs(want_y).max())


def test_combine_given_expert_outputs_matches_sparse_combine():
    # The MoE sum over given per-slot expert outputs equals the sparse combine
    # that evaluates the experts itself, on the small config's routing (FFN
    # and zero slots mixed, several slots of a token on one expert group).
    cfg = inputs.CONFIGS["small"]
    L = inputs.make_layer(cfg, "cpu")
    x = bf16_values(inputs.make_tokens(cfg, "cpu", tokens=48))
    r = oracle.route(x, L["w_router"].numpy(), L["bias"].numpy(), cfg.k)
    get = expert_getter(L, cfg)
    want = oracle.combine_given_routing(x, r["idx"], r["g"], cfg.n_ffn, get)
    out = np.full((x.shape[0], cfg.k, cfg.d), np.nan)  # zero-expert rows must not be read
    for t in range(x.shape[0]):
        for k in range(cfg.k):
            e = int(r["idx"][t, k])
            if e < cfg.n_ffn:
                w13, w2 = get(e)
                out[t, k] = oracle.expert_ffn(x[t:t + 1], w13, w2)[0]
    assert (r["idx"] >= cfg.n_ffn).any() and (r["idx"] < cfg.n_ffn).any()
    got = oracle.combine_given_expert_outputs(x, r["idx"], r["g"], cfg.n_ffn, out)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_a8_zero_routing_is_exact_identity():
    # FFN experts biased out: y = (sum_k g) x exactly, the identity sees exact x.
    cfg = inputs.CONFIGS["tiny"]
    L = inputs.make_layer(cfg, "cpu")
    x = bf16_values(inputs.make_tokens(cfg, "cpu"))
    b = L["bias"].numpy().copy()
    b[: cfg.n_ffn] = -1e4
    r = oracle.route(x, L["w_router"].numpy(), b, cfg.k)
    assert np.all(r["idx"] >= cfg.n_ffn)
    get = expert_getter(L, cfg)
    y = oracle.combine_given_routing(x, r["idx"], r["g"], cfg.n_ffn, get, a8=True)
    assert np.array_equal(y, r["g"].sum(1)[:, None] * x)


# ----------------------------------------------------------------------------
# Backward of the layer: against torch autograd (float64, CPU) and central
# finite differences.
# ----------------------------------------------------------------------------


def _torch_layer_grads(x, w_router, bias, k, n_ffn, experts, dy, idx=None):
    """The layer in torch with autograd on x, W_r and the expert weights; the
    selection (piecewise constant) is the given one, else the oracle's."""
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    Wr = torch.tensor(np.asarray(w_router, np.float64), requires_grad=True)
    W13 = {e: torch.tensor(np.asarray(a, np.float64), requires_grad=True) for e, (a, _) in experts.items()}
    W2 = {e: torch.tensor(np.asarray(b, np.float64), requires_grad=True) for e, (_, b) in experts.items()}
    if idx is None:
        idx = oracle.route(x, w_router, bias, k)["idx"]
    p = torch.softmax(X @ Wr.T, dim=1)
    y = torch.zeros_like(X)
    for t in range(x.shape[0]):
        for kk in range(k):
            e = int(idx[t, kk])
            if e < n_ffn:
                u = W13[e] @ X[t]
                inter = W2[e].shape[1]
                v = W2[e] @ (F.silu(u[:inter]) * u[inter:])
            else:
                v = X[t]
            y[t] = y[t] + p[t, e] * v
    (y * torch.tensor(dy)).sum().backward()
    def grad(w):
        return np.zeros(tuple(w.shape)) if w.grad is None else w.grad.numpy()

    return X.grad.numpy(), Wr.grad.numpy(), {e: grad(W13[e]) for e in W13}, \
        {e: grad(W2[e]) for e in W2}


@pytest.mark.parametrize("T,seed", [(16, 0), (40, 7)])
def test_layer_backward_matches_torch_autograd(T, seed):
    cfg = inputs.CONFIGS["tiny"]
    L = inputs.make_layer(cfg, "cpu")
    x = bf16_values(inputs.make_tokens(cfg, "cpu", tokens=T))
    wr, b = L["w_router"].numpy(), L["bias"].numpy()
    get = expert_getter(L, cfg)
    experts = {e: get(e) for e in range(cfg.n_ffn)}
    dy = np.random.default_rng(seed).normal(size=x.shape)
    got = oracle.layer_backward(x, wr, b, cfg.k, cfg.n_ffn, get, dy)
    dx, dwr, dw13, dw2 = _torch_layer_grads(x, wr, b, cfg.k, cfg.n_ffn, experts, dy)
    assert np.allclose(got["dx"], dx, rtol=1e-10, atol=1e-12)
    assert np.allclose(got["dw_router"], dwr, rtol=1e-10, atol=1e-12)
    for e in range(cfg.n_ffn):
        if e in got["dw13"]:
            assert np.allclose(got["dw13"][e], dw13[e], rtol=1e-10, atol=1e-12)
            assert np.allclose(got["dw2"][e], dw2[e], rtol=1e-10, atol=1e-12)
        else:  # untouched expert: zero gradient
            assert not dw13[e].any() and not dw2[e].any()


def test_layer_backward_given_selection():
    # an imposed selection (another valid one: K distinct experts per token)
    # gives the autograd gradients of the layer routed that way
    cfg = inputs.CONFIGS["tiny"]
    L = inputs.make_layer(cfg, "cpu")
    T = 12
    x = bf16_values(inputs.make_tokens(cfg, "cpu", tokens=T))
    wr, b = L["w_router"].numpy(), L["bias"].numpy()
    get = expert_getter(L, cfg)
    experts = {e: get(e) for e in range(cfg.n_ffn)}
    dy = np.random.default_rng(11).normal(size=x.shape)
    rng = np.random.default_rng(12)
    idx = np.stack([rng.permutation(cfg.n_experts)[: cfg.k] for _ in range(T)])
    assert not np.array_equal(idx, oracle.route(x, wr, b, cfg.k)["idx"])
    got = oracle.layer_backward(x, wr, b, cfg.k, cfg.n_ffn, get, dy, idx=idx)
    dx, dwr, dw13, dw2 = _torch_layer_grads(x, wr, b, cfg.k, cfg.n_ffn, experts, dy, idx=idx)
    assert np.array_equal(got["routing"]["idx"], idx)
    assert np.allclose(got["dx"], dx, rtol=1e-10, atol=1e-12)
    assert np.allclose(got["dw_router"], dwr, rtol=1e-10, atol=1e-12)
    for e in got["dw13"]:
        assert np.allclose(got["dw13"][e], dw13[e], rtol=1e-10, atol=1e-12)
        assert np.allclose(got["dw2"][e], dw2[e], rtol=1e-10, atol=1e-12)
    # its own selection passed explicitly changes nothing
    own = oracle.route(x, wr, b, cfg.k)["idx"]
    a = oracle.layer_backward(x, wr, b, cfg.k, cfg.n_ffn, get, dy)
    c = oracle.layer_backward(x, wr, b, cfg.k, cfg.n_ffn, get, dy, idx=own)
    assert np.array_equal(a["dx"], c["dx"]) and np.array_equal(a["dw_router"], c["dw_router"])


def test_layer_backward_finite_differences():
    cfg = inputs.CONFIGS["tiny"]
    L = inputs.make_layer(cfg, "cpu")
    x = bf16_values(inputs.make_tokens(cfg, "cpu", tokens=6))
    wr, b = L["w_router"].numpy().astype(np.float64), L["bias"].numpy()
    get = expert_getter(L, cfg)
    dy = np.random.default_rng(3).normal(size=x.shape)
    got = oracle.layer_backward(x, wr, b, cfg.k, cfg.n_ffn, get, dy)
    idx0 = got["routing"]["idx"]

    def loss(xx, ww):
        # the same selection as at x (piecewise-constant selection held fixed)
        r = oracle.route(xx, ww, b, cfg.k)
        assert np.array_equal(r["idx"], idx0)
        y = oracle.combine_given_routing(xx, r["idx"], r["g"], cfg.n_ffn, get)
        return float(np.sum(dy * y))

    eps = 1e-6
    rng = np.random.default_rng(4)
    for _ in range(6):
        t, c = rng.integers(6), rng.integers(cfg.d)
        e1 = np.zeros_like(x); e1[t, c] = eps
        fd = (loss(x + e1, wr) - loss(x - e1, wr)) / (2 * eps)
        assert math.isclose(fd, got["dx"][t, c], rel_tol=1e-5, abs_tol=1e-7)
        i, c2 = rng.integers(cfg.n_experts), rng.integers(cfg.d)
        e2 = np.zeros_like(wr); e2[i, c2] = eps
        fd = (loss(x, wr + e2) - loss(x, wr - e2)) / (2 * eps)
        assert math.isclose(fd, got["dw_router"][i, c2], rel_tol=1e-5, abs_tol=1e-7)


def test_silu_grad_matches_autograd():
    a = torch.linspace(-30, 30, 1001, dtype=torch.float64, requires_grad=True)
    F.silu(a).sum().backward()
    assert np.allclose(oracle.silu_grad(a.detach().numpy()), a.grad.numpy(), rtol=1e-13, atol=1e-15)

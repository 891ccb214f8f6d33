"""GPU parity of the router-side statistics (lcmoe_router_stats) against the
oracle: the device-level load-balance statistic with the zero experts as
group D+1, and the hidden z-loss of the layer input.

The oracle gets the GPU's own exported fp32 logits and counts, so both sides
start from identical inputs. f_j is formed from integer counts with the same
fp64 operations on both sides and must match exactly. P_j, L_LB and L_Z come
from per-token fp32 softmax / log-sum-exp values (a few ulp each) summed in
fp64: relative tolerance 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_biased_amd import inputs, lcmoe
from tests.gpu_common import layer
from tests.helpers import bf16_values

pytestmark = pytest.mark.gpu

RTOL = 1e-5


def run(cfg, L, x, D, k_e, alpha, lam):
    shape = lcmoe.shape_of(cfg)
    r = lcmoe.route(shape, x, L["w_router"], L["bias"], logits=True)
    st = lcmoe.router_stats(shape, x, r["logits"], r["counts"], D, k_e, alpha, lam)
    torch.cuda.synchronize()
    return r, st.cpu().numpy()


def split(st, D):
    return st[0], st[1], st[2:3 + D], st[3 + D:4 + 2 * D]


@pytest.mark.parametrize("name,T,D", [("tiny", 16, 2), ("tiny", 777, 8), ("small", 4096, 8),
                                      ("small", 1000, 64), ("decode", 64, 8),
                                      ("prefill", 8192, 8), ("prefill", 3000, 1)])
def test_router_stats_vs_oracle(name, T, D):
    cfg, L = layer(name)
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    k_e, alpha, lam = cfg.k * cfg.n_ffn / cfg.n_experts, 0.01, 1e-4
    r, st = run(cfg, L, x, D, k_e, alpha, lam)
    L_lb, L_z, f, P = split(st, D)
    z = r["logits"].cpu().numpy().astype(np.float64)
    counts = r["counts"].cpu().numpy()
    L_ref, f_ref, P_ref = oracle.load_balance_stats(z, counts, cfg.n_ffn, cfg.n_zero, cfg.k, D,
                                                    k_e, alpha)
    z_ref = oracle.hidden_z_loss(bf16_values(x), lam)
    print(f"{name} T={T} D={D}: L_LB {L_lb:.6e} (oracle {L_ref:.6e}), L_Z {L_z:.6e} "
          f"(oracle {z_ref:.6e}), max P rel err {np.max(np.abs(P - P_ref) / np.abs(P_ref)):.2e}")
    assert np.array_equal(f, f_ref)
    assert np.allclose(P, P_ref, rtol=RTOL, atol=0)
    assert math.isclose(L_lb, L_ref, rel_tol=RTOL)
    assert math.isclose(L_z, z_ref, rel_tol=RTOL)


def test_router_stats_closed_forms_on_gpu():
    cfg, L = layer("small")
    shape = lcmoe.shape_of(cfg)
    T, D, E = 300, 8, cfg.n_experts
    # uniform logits: P_j = |G_j| / E; zero hidden states: L_Z = lambda (log d)^2
    x = torch.zeros(T, cfg.d, dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(T, E, dtype=torch.float32, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    counts[0] = T * cfg.k
    st = lcmoe.router_stats(shape, x, z, counts, D, 4.0, 1.0, 0.5).cpu().numpy()
    _, L_z, f, P = split(st, D)
    want = np.array([cfg.n_ffn / D / E] * D + [cfg.n_zero / E])
    assert np.allclose(P, want, rtol=1e-6, atol=0)
    assert math.isclose(L_z, 0.5 * math.log(cfg.d) ** 2, rel_tol=1e-6)
    # every slot on expert 0: f_0 = 1 / (K_e/(K D)) = K D / K_e, all others 0
    assert math.isclose(f[0], cfg.k * D / 4.0, rel_tol=1e-15) and not f[1:].any()


def test_router_stats_zero_tokens_and_determinism():
    cfg, L = layer("tiny")
    shape = lcmoe.shape_of(cfg)
    x0 = torch.empty(0, cfg.d, dtype=torch.bfloat16, device="cuda")
    z0 = torch.empty(0, cfg.n_experts, dtype=torch.float32, device="cuda")
    c0 = torch.zeros(cfg.n_experts, dtype=torch.int32, device="cuda")
    st = lcmoe.router_stats(shape, x0, z0, c0, 2, 2.0).cpu().numpy()
    assert not st.any()
    x = inputs.make_tokens(cfg, "cuda", tokens=500)
    _, a = run(cfg, L, x, 4, 2.0, 1.0, 1.0)
    _, b = run(cfg, L, x, 4, 2.0, 1.0, 1.0)
    assert np.array_equal(a, b)

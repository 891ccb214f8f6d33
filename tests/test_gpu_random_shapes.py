"""Seeded random layer shapes through the C ABI, against the oracle.

Thirty-six shapes are drawn (fixed seed) inside the boundary's limits: d and I
multiples of 32 (of 128 with fp8 weights), 1..80 FFN and 0..48 zero experts,
K from 1 to min(E, 16), T from 1 to 600 tokens, router bias of scale 0, 0.1
or 1, with or without the 1% of tokens scaled x20. Every case checks the
forward on every token (and the routing entry point's agreement with it);
cases with bf16 weights also check every backward output. Tolerances are
those of the other parity tests (2e-2 bf16, 5e-2 fp8); with fp8 activations
each stage is checked on the GPU's own inputs to it (codes and scales bit for
bit, H and y within tolerance), at every intermediate size the boundary
accepts.
"""
import numpy as np
import pytest

from mixture_experts_layer_biased_amd import inputs
from tests.test_gpu_backward import check_all, gpu_selection, run_backward
from tests.test_gpu_forward import check_routing_consistent, check_rows, run_forward

SEED = 20261203


def _cases(n=36):
    rng = np.random.default_rng(SEED)
    out = []
    for i in range(n):
        wd = str(rng.choice(["bf16", "bf16", "bf16", "fp8", "fp8a8"]))
        unit = 32 if wd == "bf16" else 128
        d = unit * int(rng.integers(1, 768 // unit + 1))
        inter = unit * int(rng.integers(1, 768 // unit + 1))
        n_ffn = int(rng.integers(1, 81))
        n_zero = int(rng.integers(0, 49))
        k = int(rng.integers(1, min(n_ffn + n_zero, 16) + 1))
        T = int(np.exp(rng.uniform(0.0, np.log(600.0))))
        skew = bool(rng.integers(0, 2))
        out.append(dict(d=d, inter=inter, n_ffn=n_ffn, n_zero=n_zero, k=k, tokens=T,
                        seed=100 + i, wdtype=wd, bias_std=float(rng.choice([0.0, 0.1, 1.0])),
                        skew_frac=0.01 if skew else 0.0, skew_factor=20.0 if skew else 1.0))
    return out


CASES = _cases()


def _id(c):
    return (f"{c['wdtype']}-d{c['d']}-I{c['inter']}-N{c['n_ffn']}-Z{c['n_zero']}-K{c['k']}"
            f"-T{c['tokens']}")


def test_cases_cover_dtypes_and_row_counts():
    # the draw includes every weight type, batches with a few expected rows
    # per expert (at most one 32-row fragment) and batches with several
    # fragments per M-tile
    assert {c["wdtype"] for c in CASES} == {"bf16", "fp8", "fp8a8"}
    assert min(c["inter"] for c in CASES if c["wdtype"] == "fp8a8") < 384
    rows = [c["tokens"] * c["k"] * c["n_ffn"] / (c["n_ffn"] + c["n_zero"]) / c["n_ffn"]
            for c in CASES]
    assert sum(r > 32 for r in rows) >= 2 and sum(r <= 32 for r in rows) >= 2


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape(case):
    cfg = inputs.CONFIGS["tiny"].with_(name="random", **case)
    L = inputs.make_layer(cfg, "cuda")
    x = inputs.make_tokens(cfg, "cuda")
    res = run_forward(cfg, L, x)
    check_routing_consistent(cfg, L, x, res)
    counts = res["counts"].cpu().numpy()[: cfg.n_ffn]
    print(f"{_id(case)}: max rows per FFN expert {counts.max()}")
    check_rows(cfg, L, x, res, np.arange(cfg.tokens), cache={})
    if cfg.wdtype == "bf16":
        dy = inputs.make_upstream_grad(cfg, "cuda")
        resb = run_backward(cfg, L, x, dy)
        check_all(cfg, L, x, dy, resb, gpu_selection(cfg, L, x), cache={})

"""Expert row counts placed on the boundaries of the GEMM kernels, forward
and backward, against the oracle.

Routing is constructed (identity router, top-1, zero bias; see
inputs.counted_routing_inputs) so that each expert receives an exact number
of tokens. The FFN counts sit on either side of every size the kernels
branch on: the 32-row MFMA fragments (a wave multiplies only the fragments
that hold rows; a single row included), the grouped GEMM's M-tile (320
rows, split evenly beyond) and its LDS ring (3 slots up to 168 rows),
the dgrad M tile (256 rows) and its ring (3 slots up to 160 rows), the
weight-gradient k stages (64 slot rows), and an FFN expert with no rows
(zero weight gradients). d = 128 is narrower than one 256-column dgrad
tile; I = 160 makes the gate/up output and the W2^T dy product ragged and
the down product's k an odd multiple of 32. The forward is also checked
with fp8 weights and with fp8 weights and activations (their own kernels and
ring geometry). Tolerances are those of the other parity tests.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_biased_amd import inputs
from tests.test_gpu_backward import check_all, run_backward
from tests.test_gpu_forward import check_rows, run_forward

FFN_COUNTS = [0, 1, 31, 32, 33, 64, 65, 127, 128, 129, 160, 161, 168, 169, 192, 255, 256, 257,
              320, 321, 400]
ZERO_COUNTS = [5, 0, 3, 7]
SEED = 20261204


# fp8 weights need d and I multiples of 128 (the scale blocks); fp8
# activations at the smallest intermediate size the boundary accepts.
INTER = {"bf16": 160, "fp8": 256, "fp8a8": 128}


def _layer(wdtype="bf16"):
    counts = FFN_COUNTS + ZERO_COUNTS
    cfg = inputs.CONFIGS["tiny"].with_(name=f"row_counts_{wdtype}", d=128, inter=INTER[wdtype],
                                       n_ffn=len(FFN_COUNTS), n_zero=len(ZERO_COUNTS), k=1,
                                       tokens=sum(counts), seed=SEED, bias_std=0.0, skew_frac=0.0,
                                       skew_factor=1.0, wdtype=wdtype)
    L = inputs.make_layer(cfg, "cuda")
    x, w_r, bias, choice = inputs.counted_routing_inputs(counts, cfg.d, "cuda", SEED)
    L["w_router"], L["bias"] = w_r, bias
    return cfg, L, x, choice, counts


def test_counts_cover_the_boundaries():
    # host-only: the list straddles every size named above
    c = set(FFN_COUNTS)
    for lo, hi in [(32, 33), (64, 65), (128, 129), (160, 161), (168, 169), (256, 257), (320, 321)]:
        assert lo in c and hi in c
    assert 0 in c and max(c) > 320


def test_counted_routing_inputs_on_cpu():
    # host-only: exact counts, and each token's chosen expert is the unique
    # maximum of its logits x W_r^T (computed exactly here in fp64)
    counts = FFN_COUNTS + ZERO_COUNTS
    x, w_r, bias, choice = inputs.counted_routing_inputs(counts, 128, "cpu", SEED)
    assert np.array_equal(np.bincount(choice.numpy(), minlength=len(counts)), np.array(counts))
    z = x.double() @ w_r.double().T + bias.double()
    top2 = torch.topk(z, 2, dim=1)
    assert torch.equal(top2.indices[:, 0], choice)
    assert bool((top2.values[:, 0] - top2.values[:, 1] > 0.5).all())


@pytest.mark.gpu
@pytest.mark.parametrize("wdtype", ["fp8", "fp8a8"])
def test_forward_fp8_at_row_count_boundaries(wdtype):
    cfg, L, x, choice, counts = _layer(wdtype)
    res = run_forward(cfg, L, x)
    assert torch.equal(res["idx"][:, 0].long(), choice)
    assert np.array_equal(res["counts"].cpu().numpy(), np.array(counts))
    check_rows(cfg, L, x, res, np.arange(cfg.tokens), cache={})


@pytest.mark.gpu
def test_forward_and_backward_at_row_count_boundaries():
    cfg, L, x, choice, counts = _layer()
    res = run_forward(cfg, L, x)
    assert torch.equal(res["idx"][:, 0].long(), choice)
    assert np.array_equal(res["counts"].cpu().numpy(), np.array(counts))
    check_rows(cfg, L, x, res, np.arange(cfg.tokens), cache={})
    dy = inputs.make_upstream_grad(cfg, "cuda")
    resb = run_backward(cfg, L, x, dy)
    check_all(cfg, L, x, dy, resb, res["idx"].cpu().numpy(), cache={})

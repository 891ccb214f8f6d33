"""Host-side logic of bench.py (no GPU): the one-GPU contract, the algorithmic
work the roofline figures are computed from, and the kernel-to-stage maps
used for the rocprofv3 summaries."""
import os
import subprocess
import sys

import numpy as np

import bench
from mixture_experts_layer_biased_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout


def test_forward_work_matches_the_layer_definition():
    # every FFN slot on the large path: gate/up and down flops are 2 S 2I d
    # and 2 S I d; weights of each touched expert are counted once
    cfg = inputs.CONFIGS["prefill"]
    counts = np.zeros(cfg.n_experts, dtype=np.int64)
    counts[: cfg.n_ffn] = 128
    w = bench.kernel_work(cfg, counts)
    S, d, I = 128 * cfg.n_ffn, cfg.d, cfg.inter
    assert w["gateup_large"]["flops"] == 2.0 * S * 2 * I * d
    assert w["down_large"]["flops"] == 2.0 * S * I * d
    assert w["gateup_small"]["rows"] == 0 and w["down_small"]["flops"] == 0
    assert w["gateup_large"]["bytes"] == cfg.n_ffn * 2 * I * d * 2 + S * d * 2 + S * I * 2
    # experts with 1..32 rows go to the small path, untouched experts cost nothing
    counts[:10] = 5
    counts[10:20] = 0
    w = bench.kernel_work(cfg, counts)
    assert w["gateup_small"]["experts"] == 10 and w["gateup_large"]["experts"] == cfg.n_ffn - 20
    lb = bench.layer_bytes(cfg, counts, cfg.tokens)
    assert lb == (cfg.n_ffn - 10) * 3 * I * d * 2 + cfg.n_experts * d * 4 + 2 * cfg.tokens * d * 2


def test_backward_work_counts_every_gradient_written():
    cfg = inputs.CONFIGS["prefill"]
    counts = np.zeros(cfg.n_experts, dtype=np.int64)
    counts[: cfg.n_ffn // 2] = 256      # half the experts touched
    w = bench.backward_work(cfg, counts, cfg.tokens)
    d, I, N = cfg.d, cfg.inter, cfg.n_ffn
    S = 256 * (N // 2)
    # weight gradients are written for every expert, zeros included
    assert w["dw13"]["bytes"] >= N * 2 * I * d * 2
    assert w["dw2"]["bytes"] >= N * d * I * 2
    # dgrad passes read only the touched experts' weights
    assert w["dx_rows"]["bytes"] == (N // 2) * 2 * I * d * 2 + S * (2 * I * 2 + d * 4)
    assert w["u_silu"]["flops"] == 2.0 * S * 2 * I * d
    assert set(w) >= {"u_silu", "w2t_dy", "dx_rows", "dw2", "dw13", "router_grads"}


def test_stage_maps():
    assert bench.stage_of_kernel("void lcmoe::gemm_big_dma_kernel<true, false>(lcmoe::GemmArgs)") \
        == "gateup_large"
    assert bench.stage_of_kernel("void lcmoe::gemm_small_kernel<false, true>(lcmoe::GemmArgs)") \
        == "down_small"
    assert bench.stage_of_kernel("lcmoe::combine_kernel(unsigned short const*)") == "combine"
    assert bench.bwd_stage_of_kernel(
        "void lcmoe::bwd_dgrad_kernel<true, 3>(lcmoe::BwdGemmArgs)") == "dx_rows"
    assert bench.bwd_stage_of_kernel(
        "void lcmoe::bwd_dgrad_kernel<true, 2>(lcmoe::BwdGemmArgs)") == "w2t_dy"
    assert bench.bwd_stage_of_kernel(
        "void lcmoe::bwd_wgrad_f32_kernel<2, 2, 2, 2, 3, 7>(lcmoe::BwdGemmArgs)") == "router_grads"
    assert bench.bwd_stage_of_kernel(
        "void lcmoe::bwd_wgrad_stream_kernel<2, 4, 4, 2, 5>(lcmoe::BwdGemmArgs)") == "dw13"
    assert bench.bwd_stage_of_kernel(
        "void lcmoe::bwd_wgrad_stream_kernel<2, 4, 4, 2, 4>(lcmoe::BwdGemmArgs)") == "dw2"
    assert bench.bwd_stage_of_kernel(
        "void lcmoe::gemm_big_dma_kernel<true, false, true>(lcmoe::GemmArgs)") == "u_silu"
    assert bench.bwd_stage_of_kernel("lcmoe::gather_rows_kernel(unsigned short const*)") \
        == "route_gather"

"""The no-allocation forward (lcmoe_forward_noalloc) against lcmoe_forward.

The entry point runs the forward's kernels with the workspace in a fixed
device array inside the library, shared by every call on the device; its
outputs must be those of lcmoe_forward with a fresh caller workspace, bit for
bit. Two calls in a row, the second with fewer tokens, so the second runs on
an array still holding the first call's contents. A batch whose workspace
exceeds the array is rejected before anything is enqueued.
"""
import ctypes

import pytest
import torch

from mixture_experts_layer_biased_amd import inputs, lcmoe
from tests.gpu_common import layer

pytestmark = pytest.mark.gpu


def _pair(cfg, L, x):
    shape = lcmoe.shape_of(cfg)
    args = (shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], L["w13_scale"], L["w2_scale"])
    ref = lcmoe.forward(*args)
    got = lcmoe.forward_noalloc(*args)
    torch.cuda.synchronize()
    for k in ("y", "idx", "gate", "counts"):
        assert torch.equal(got[k], ref[k]), (cfg.name, x.shape[0], k)
    return got


@pytest.mark.parametrize("name,T1,T2", [("decode", 64, 17), ("small", 900, 300),
                                        ("tiny", 777, 1)])
def test_noalloc_matches_forward_twice(name, T1, T2):
    cfg, L = layer(name)
    print(f"noalloc {name}: T={T1} then T={T2}", flush=True)
    x1 = inputs.make_tokens(cfg, "cuda", tokens=T1)
    x2 = inputs.make_tokens(cfg.with_(seed=cfg.seed + 7), "cuda", tokens=T2)
    _pair(cfg, L, x1)
    _pair(cfg, L, x2)


@pytest.mark.parametrize("wdtype", ["fp8", "fp8a8"])
def test_noalloc_fp8_decode(wdtype):
    cfg, L = layer("small", wdtype=wdtype)
    print(f"noalloc small {wdtype}", flush=True)
    _pair(cfg, L, inputs.make_tokens(cfg, "cuda", tokens=600))
    _pair(cfg, L, inputs.make_tokens(cfg.with_(seed=11), "cuda", tokens=40))


def test_noalloc_rejects_batches_past_the_array():
    cfg, L = layer("decode")
    shape = lcmoe.shape_of(cfg)
    T = 4096  # LongCat shape: about 1 GB of workspace
    assert lcmoe.workspace_bytes(shape, T) > lcmoe.NOALLOC_SCRATCH_BYTES
    x = inputs.make_tokens(cfg, "cuda", tokens=T)
    counts = torch.full((cfg.n_experts,), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(lcmoe.LcmoeError) as e:
        lcmoe.forward_noalloc(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"],
                              out=dict(counts=counts))
    assert e.value.status == lcmoe.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(counts.min()) == 7 and int(counts.max()) == 7  # nothing was enqueued
    # T = 0: counts zeroed, no scratch needed
    x0 = torch.empty(0, cfg.d, dtype=torch.bfloat16, device="cuda")
    lcmoe.forward_noalloc(shape, x0, L["w_router"], L["bias"], L["w13"], L["w2"],
                          out=dict(counts=counts))
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0


def test_noalloc_under_graph_capture():
    # The callers it is for: work captured into a HIP graph. One call captured
    # (no allocation, no memset, kernels only), then replayed on new token
    # values written into the captured input, with eager work between
    # replays; every replay gives the bits of an eager lcmoe_forward call.
    cfg, L = layer("small")
    shape = lcmoe.shape_of(cfg)
    T = 300
    xs = [inputs.make_tokens(cfg.with_(seed=cfg.seed + 5 * j), "cuda", tokens=T) for j in range(3)]
    x_in = xs[0].clone()
    out = dict(y=torch.empty(T, cfg.d, dtype=torch.bfloat16, device="cuda"),
               idx=torch.empty(T, cfg.k, dtype=torch.int32, device="cuda"),
               gate=torch.empty(T, cfg.k, dtype=torch.float32, device="cuda"),
               counts=torch.empty(cfg.n_experts, dtype=torch.int32, device="cuda"))

    def call():
        lcmoe.forward_noalloc(shape, x_in, L["w_router"], L["bias"], L["w13"], L["w2"], out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for j in (1, 2, 0, 2):
        x_in.copy_(xs[j])
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        ref = lcmoe.forward(shape, xs[j], L["w_router"], L["bias"], L["w13"], L["w2"])
        torch.cuda.synchronize()
        for k in ("y", "idx", "gate", "counts"):
            assert torch.equal(got[k], ref[k]), (j, k)

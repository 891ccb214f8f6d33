"""The library keeps no device state of its own: every call works in the
caller's workspace and enqueues on the caller's stream. Calls on two streams
(default priority), each with its own inputs, workspaces and outputs,
enqueued interleaved so that their kernels may overlap, give the bits of the
same calls made one after the other on one stream."""
import pytest
import torch

from mixture_experts_layer_biased_amd import inputs, lcmoe
from tests.gpu_common import layer

pytestmark = pytest.mark.gpu


def _run(shape, L, x, dy):
    f = lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"])
    b = lcmoe.backward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], dy)
    return {**{k: f[k] for k in ("y", "idx", "gate", "counts")}, **b}


@pytest.mark.parametrize("name,T", [("small", 2000), ("tiny", 300)])
def test_two_streams_match_sequential(name, T):
    cfg, L = layer(name)
    shape = lcmoe.shape_of(cfg)
    xs = [inputs.make_tokens(cfg.with_(seed=cfg.seed + 5 * j), "cuda", tokens=T) for j in range(2)]
    dys = [inputs.make_upstream_grad(cfg.with_(seed=cfg.seed + 5 * j), "cuda", tokens=T)
           for j in range(2)]
    seq = [_run(shape, L, xs[j], dys[j]) for j in range(2)]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [None, None]
    for rep in range(2):  # enqueue both streams' work before waiting for either
        for j, s in enumerate(streams):
            with torch.cuda.stream(s):
                got[j] = _run(shape, L, xs[j], dys[j])
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for j in range(2):
        for k, v in seq[j].items():
            assert torch.equal(got[j][k], v), (j, k)

"""The forward (T > 0) enqueues kernels only, on the caller's stream: no
allocation, no memset or copy, no host synchronisation. A caller can capture
it into a HIP graph and replay it. Each replay, on new token values written
into the captured input buffer, must give the bits of an eager call on the
same values; eager work and host synchronisations run between replays, and
the replays reuse one workspace (so nothing may depend on its prior
contents)."""
import pytest
import torch

from mixture_experts_layer_biased_amd import inputs, lcmoe
from tests.gpu_common import layer

pytestmark = pytest.mark.gpu


def _outputs(cfg, T):
    dev = "cuda"
    return dict(y=torch.empty(T, cfg.d, dtype=torch.bfloat16, device=dev),
                idx=torch.empty(T, cfg.k, dtype=torch.int32, device=dev),
                gate=torch.empty(T, cfg.k, dtype=torch.float32, device=dev),
                counts=torch.empty(cfg.n_experts, dtype=torch.int32, device=dev))


@pytest.mark.parametrize("name,T,wdtype", [("small", 4096, "bf16"), ("tiny", 200, "bf16"),
                                           ("small", 300, "fp8"), ("small", 1000, "fp8a8")])
def test_forward_graph_replays_match_eager(name, T, wdtype):
    cfg, L = layer(name, wdtype=wdtype) if wdtype != "bf16" else layer(name)
    shape = lcmoe.shape_of(cfg)
    xs = [inputs.make_tokens(cfg.with_(seed=cfg.seed + 11 * j), "cuda", tokens=T)
          for j in range(3)]
    x_in = xs[0].clone()
    ws = lcmoe.workspace(shape, T)
    out = _outputs(cfg, T)

    def fwd(x, ws_, out_):
        return lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"],
                             L["w13_scale"], L["w2_scale"], ws=ws_, out=out_)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(x_in, ws, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(x_in, ws, out)
    torch.cuda.synchronize()

    ws_eager = lcmoe.workspace(shape, T)
    for j in (0, 1, 2, 1):
        x_in.copy_(xs[j])
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        ref = fwd(xs[j], ws_eager, _outputs(cfg, T))     # eager work between replays
        torch.cuda.synchronize()
        for k in ("y", "idx", "gate", "counts"):
            assert torch.equal(got[k], ref[k]), (j, k)

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


def test_zero_token_calls_graph_replays():
    # With no tokens the forward zeroes the counts and the backward the weight
    # gradients, by kernels (no memset node): captured once, every replay
    # zeroes them again after eager work has filled them in between.
    cfg, L = layer("tiny")
    shape = lcmoe.shape_of(cfg)
    x0 = torch.empty(0, cfg.d, dtype=torch.bfloat16, device="cuda")
    counts = torch.empty(cfg.n_experts, dtype=torch.int32, device="cuda")
    N, I, d, E = cfg.n_ffn, cfg.inter, cfg.d, cfg.n_experts
    grads = dict(dx=torch.empty(0, d, dtype=torch.float32, device="cuda"),
                 dw_router=torch.empty(E, d, dtype=torch.float32, device="cuda"),
                 dw13=torch.empty(N, 2 * I, d, dtype=torch.bfloat16, device="cuda"),
                 dw2=torch.empty(N, d, I, dtype=torch.bfloat16, device="cuda"))
    dy0 = torch.empty(0, d, dtype=torch.bfloat16, device="cuda")
    ws = lcmoe.workspace(shape, 0)

    def calls():
        lcmoe.forward(shape, x0, L["w_router"], L["bias"], L["w13"], L["w2"], ws=ws,
                      out=dict(counts=counts))
        lcmoe.backward(shape, x0, L["w_router"], L["bias"], L["w13"], L["w2"], dy0, ws=ws,
                       out=grads)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for fill in (7, -3):
        counts.fill_(fill)
        for k in ("dw_router", "dw13", "dw2"):
            grads[k].fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(counts.abs().sum()) == 0
        for k in ("dw_router", "dw13", "dw2"):
            assert int(grads[k].abs().sum()) == 0, k


def test_backward_graph_replays_match_eager():
    # The backward forks its weight-gradient GEMMs onto the library's second
    # stream and joins them back with events: captured once, the replays of
    # that fork and join on new x and dy give the bits of eager calls.
    cfg, L = layer("small")
    shape = lcmoe.shape_of(cfg)
    T = 700
    xs = [inputs.make_tokens(cfg.with_(seed=cfg.seed + 3 * j), "cuda", tokens=T) for j in range(3)]
    dys = [inputs.make_upstream_grad(cfg.with_(seed=cfg.seed + 3 * j), "cuda", tokens=T)
           for j in range(3)]
    x_in, dy_in = xs[0].clone(), dys[0].clone()
    N, I, d, E = cfg.n_ffn, cfg.inter, cfg.d, cfg.n_experts

    def grads():
        return dict(dx=torch.empty(T, d, dtype=torch.float32, device="cuda"),
                    dw_router=torch.empty(E, d, dtype=torch.float32, device="cuda"),
                    dw13=torch.empty(N, 2 * I, d, dtype=torch.bfloat16, device="cuda"),
                    dw2=torch.empty(N, d, I, dtype=torch.bfloat16, device="cuda"))

    out = grads()
    ws = torch.empty(lcmoe.backward_workspace_bytes(shape, T), dtype=torch.uint8, device="cuda")

    def bwd(x, dy, ws_, out_):
        return lcmoe.backward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], dy, ws=ws_,
                              out=out_)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bwd(x_in, dy_in, ws, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bwd(x_in, dy_in, ws, out)
    torch.cuda.synchronize()
    ws_eager = torch.empty_like(ws)
    for j in (1, 0, 2, 1):
        x_in.copy_(xs[j])
        dy_in.copy_(dys[j])
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        ref = bwd(xs[j], dys[j], ws_eager, grads())
        torch.cuda.synchronize()
        for k in ("dx", "dw_router", "dw13", "dw2"):
            assert torch.equal(got[k], ref[k]), (j, k)

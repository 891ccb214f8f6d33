"""The Python binding checks every tensor's dtype and shape against the layer
shape before anything reaches the library (which reads and writes through
raw pointers with the sizes the shape implies). Host-only: the checks run
before any workspace is allocated or any device call is made, so CPU tensors
exercise them."""
import pytest
import torch

from mixture_experts_layer_biased_amd import lcmoe

D, N, Z, K, I, T = 128, 8, 4, 3, 256, 5


def _layer(w_dtype="bf16"):
    s = lcmoe.make_shape(D, N, Z, K, I, w_dtype)
    E = N + Z
    wdt = torch.bfloat16 if w_dtype == "bf16" else torch.uint8
    t = dict(x=torch.zeros(T, D, dtype=torch.bfloat16), w_router=torch.zeros(E, D),
             bias=torch.zeros(E), w13=torch.zeros(N, 2 * I, D, dtype=wdt),
             w2=torch.zeros(N, D, I, dtype=wdt), w13_scale=None, w2_scale=None)
    if w_dtype != "bf16":
        t["w13_scale"] = torch.ones(N, 2 * I // 128, D // 128)
        t["w2_scale"] = torch.ones(N, D // 128, I // 128)
    return s, t


def _rejects(fn, name):
    with pytest.raises(lcmoe.LcmoeError) as ei:
        fn()
    assert ei.value.status == lcmoe.ERR_INVALID_ARG
    assert str(ei.value).startswith(name + ":"), str(ei.value)


def _forward(s, t, **over):
    a = dict(t, **over)
    return lambda: lcmoe.forward(s, a["x"], a["w_router"], a["bias"], a["w13"], a["w2"],
                                 a["w13_scale"], a["w2_scale"], out=a.get("out"),
                                 u_save=a.get("u_save"))


@pytest.mark.parametrize("name,bad", [
    ("x", torch.zeros(T, D)),                                   # fp32 tokens
    ("x", torch.zeros(T, D + 32, dtype=torch.bfloat16)),        # wrong width
    ("w_router", torch.zeros(N + Z - 1, D)),                    # one expert short
    ("bias", torch.zeros(N + Z, dtype=torch.float64)),
    ("w13", torch.zeros(N, I, D, dtype=torch.bfloat16)),        # gate rows only
    ("w13", torch.zeros(N, 2 * I, D, dtype=torch.uint8)),       # fp8 codes, bf16 shape
    ("w2", torch.zeros(N, I, D, dtype=torch.bfloat16)),         # transposed
])
def test_forward_rejects_bad_inputs(name, bad):
    s, t = _layer()
    _rejects(_forward(s, t, **{name: bad}), name)


def test_forward_rejects_bad_outputs_and_saved_u():
    s, t = _layer()
    E = N + Z
    _rejects(_forward(s, t, out={"y": torch.zeros(T, D)}), "y")
    _rejects(_forward(s, t, out={"idx": torch.zeros(T, K, dtype=torch.int64)}), "idx")
    _rejects(_forward(s, t, out={"gate": torch.zeros(T, K + 1)}), "gate")
    _rejects(_forward(s, t, out={"counts": torch.zeros(N, dtype=torch.int32)}), "counts")
    rows = lcmoe.u_rows(s, T)
    _rejects(_forward(s, t, u_save=torch.zeros(rows - 1, 2 * I)), "u_save")
    _rejects(_forward(s, t, u_save=torch.zeros(rows, I)), "u_save")
    assert E == s.n_experts


def test_fp8_shapes_need_codes_and_scales():
    s, t = _layer("fp8")
    _rejects(_forward(s, t, w13=torch.zeros(N, 2 * I, D, dtype=torch.bfloat16)), "w13")
    _rejects(_forward(s, t, w13_scale=None), "w13_scale")
    _rejects(_forward(s, t, w2_scale=torch.ones(N, I // 128, D // 128 + 1)), "w2_scale")


def test_other_entry_points_reject_bad_tensors():
    s, t = _layer()
    E = N + Z
    _rejects(lambda: lcmoe.route(s, t["x"], t["w_router"], torch.zeros(E + 1)), "bias")
    _rejects(lambda: lcmoe.permute(s, torch.zeros(T, K + 1, dtype=torch.int32)), "topk_idx")
    _rejects(lambda: lcmoe.bias_update(s, torch.zeros(E, dtype=torch.int64), 1e-3, 2.0,
                                       t["bias"], T), "counts")
    _rejects(lambda: lcmoe.router_stats(s, t["x"], torch.zeros(T, E - 1),
                                        torch.zeros(E, dtype=torch.int32), 1, 2.0), "logits")
    dy = torch.zeros(T, D, dtype=torch.bfloat16)
    bw = lambda **o: (lambda: lcmoe.backward(s, t["x"], t["w_router"], t["bias"], t["w13"],
                                             t["w2"], o.get("dy", dy), out=o.get("out"),
                                             u_saved=o.get("u_saved")))
    _rejects(bw(dy=torch.zeros(T - 1, D, dtype=torch.bfloat16)), "dy")
    _rejects(bw(out={"dx": torch.zeros(T, D, dtype=torch.bfloat16)}), "dx")
    _rejects(bw(out={"dw13": torch.zeros(N, 2 * I, D)}), "dw13")
    _rejects(bw(u_saved=torch.zeros(1, 2 * I)), "u_saved")

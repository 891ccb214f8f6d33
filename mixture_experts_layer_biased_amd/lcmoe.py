"""ctypes binding of liblcmoe.so over torch device tensors.

Argument marshalling only: every step of the layer runs in the HIP library.
Names follow the C ABI (include/lcmoe.h): route, permute, forward,
bias_update, router_stats, workspace_bytes. Work is enqueued on torch's current stream.
If the library is missing, loading fails loudly; there is no fallback.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; LCMOE_LIBRARY names another build of the same library
# (the host-sanitizer build of build_sanitized.py).
LIB_PATH = os.environ.get("LCMOE_LIBRARY") or os.path.join(_PKG, "liblcmoe.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
W_BF16, W_FP8_E4M3_B128, W_FP8_E4M3_B128_A8 = 0, 1, 2

EXPORTS = ("lcmoe_workspace_bytes", "lcmoe_route", "lcmoe_permute", "lcmoe_forward",
           "lcmoe_forward_staged", "lcmoe_forward_inspect", "lcmoe_forward_noalloc",
           "lcmoe_bias_update", "lcmoe_router_stats_workspace_bytes",
           "lcmoe_router_stats", "lcmoe_backward_workspace_bytes", "lcmoe_backward",
           "lcmoe_backward_staged", "lcmoe_forward_train", "lcmoe_backward_saved",
           "lcmoe_status_str")
NUM_STAGES = 6
STAGES = ("router", "topk", "permute", "gateup", "down", "combine")


class LcmoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_ffn", ctypes.c_int32),
                ("n_zero", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_expert", ctypes.c_int32), ("w_dtype", ctypes.c_int32)]

    @property
    def n_experts(self):
        return self.n_ffn + self.n_zero


def make_shape(d_model, n_ffn, n_zero, top_k, d_expert, w_dtype=W_BF16):
    if isinstance(w_dtype, str):
        w_dtype = {"bf16": W_BF16, "fp8": W_FP8_E4M3_B128, "fp8a8": W_FP8_E4M3_B128_A8}[w_dtype]
    return Shape(d_model, n_ffn, n_zero, top_k, d_expert, w_dtype)


def shape_of(cfg):
    """Shape from a LayerConfig (mixture_experts_layer_biased_amd.inputs)."""
    return make_shape(cfg.d, cfg.n_ffn, cfg.n_zero, cfg.k, cfg.inter, cfg.wdtype)


_lib = None
_P = ctypes.c_void_p


def lib():
    """Load liblcmoe.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m mixture_experts_layer_biased_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    S = ctypes.POINTER(Shape)
    i32, sz, st = ctypes.c_int32, ctypes.c_size_t, ctypes.c_int
    L.lcmoe_workspace_bytes.argtypes = [S, i32]
    L.lcmoe_workspace_bytes.restype = sz
    L.lcmoe_route.argtypes = [S, i32, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]
    L.lcmoe_route.restype = st
    L.lcmoe_permute.argtypes = [S, i32, _P, _P, _P, _P, _P, _P, sz, _P]
    L.lcmoe_permute.restype = st
    L.lcmoe_forward.argtypes = [S, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]
    L.lcmoe_forward.restype = st
    L.lcmoe_forward_staged.argtypes = [S, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       sz, _P, _P]
    L.lcmoe_forward_staged.restype = st
    L.lcmoe_forward_inspect.argtypes = [S, i32] + [_P] * 17 + [sz, _P]
    L.lcmoe_forward_inspect.restype = st
    L.lcmoe_forward_noalloc.argtypes = [S, i32] + [_P] * 11 + [_P]
    L.lcmoe_forward_noalloc.restype = st
    L.lcmoe_bias_update.argtypes = [S, i32, _P, ctypes.c_double, ctypes.c_double, _P, _P]
    L.lcmoe_bias_update.restype = st
    L.lcmoe_router_stats_workspace_bytes.argtypes = [S, i32]
    L.lcmoe_router_stats_workspace_bytes.restype = sz
    L.lcmoe_router_stats.argtypes = [S, i32, _P, _P, _P, i32, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_double, _P, _P, sz, _P]
    L.lcmoe_router_stats.restype = st
    L.lcmoe_backward_workspace_bytes.argtypes = [S, i32]
    L.lcmoe_backward_workspace_bytes.restype = sz
    L.lcmoe_backward.argtypes = [S, i32] + [_P] * 11 + [sz, _P]
    L.lcmoe_backward.restype = st
    L.lcmoe_backward_staged.argtypes = [S, i32] + [_P] * 11 + [sz, _P, _P]
    L.lcmoe_backward_staged.restype = st
    L.lcmoe_forward_train.argtypes = [S, i32] + [_P] * 11 + [sz, _P]
    L.lcmoe_forward_train.restype = st
    L.lcmoe_backward_saved.argtypes = [S, i32] + [_P] * 12 + [sz, _P]
    L.lcmoe_backward_saved.restype = st
    L.lcmoe_status_str.argtypes = [st]
    L.lcmoe_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(status):
    return lib().lcmoe_status_str(status).decode()


def _check(status, what):
    if status != OK:
        raise LcmoeError(status, f"{what}: {status_str(status)}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA tensors"


def _expect(name, t, dtype, shape):
    """The library reads and writes through raw pointers with the sizes the
    shape implies, so every tensor's dtype and shape are checked here first."""
    if t is None or t.dtype != dtype or tuple(t.shape) != tuple(int(v) for v in shape):
        got = "None" if t is None else f"{t.dtype} {tuple(t.shape)}"
        raise LcmoeError(ERR_INVALID_ARG,
                         f"{name}: expected {dtype} {tuple(int(v) for v in shape)}, got {got}")


def _expect_layer(shape, T, x, w_router, bias):
    d, E = shape.d_model, shape.n_experts
    _expect("x", x, torch.bfloat16, (T, d))
    _expect("w_router", w_router, torch.float32, (E, d))
    _expect("bias", bias, torch.float32, (E,))


def _expect_experts(shape, w13, w2, w13_scale=None, w2_scale=None):
    d, N, I = shape.d_model, shape.n_ffn, shape.d_expert
    wdt = torch.bfloat16 if shape.w_dtype == W_BF16 else torch.uint8
    _expect("w13", w13, wdt, (N, 2 * I, d))
    _expect("w2", w2, wdt, (N, d, I))
    if shape.w_dtype != W_BF16:
        _expect("w13_scale", w13_scale, torch.float32, (N, 2 * I // 128, d // 128))
        _expect("w2_scale", w2_scale, torch.float32, (N, d // 128, I // 128))


def _expect_routing_out(shape, T, idx, gate, counts):
    K, E = shape.top_k, shape.n_experts
    _expect("idx", idx, torch.int32, (T, K))
    _expect("gate", gate, torch.float32, (T, K))
    _expect("counts", counts, torch.int32, (E,))


def workspace_bytes(shape, max_tokens):
    return int(lib().lcmoe_workspace_bytes(ctypes.byref(shape), int(max_tokens)))


def workspace(shape, max_tokens, device="cuda"):
    n = workspace_bytes(shape, max_tokens)
    if n == 0:
        raise LcmoeError(ERR_INVALID_ARG, "invalid or unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def route(shape, x, w_router, bias, ws=None, logits=False, out=None):
    """Router logits, biased top-K, gates and counts.

    Returns dict(idx int32 [T,K], gate fp32 [T,K], counts int32 [E], logits fp32 [T,E] or None).
    """
    T = x.shape[0]
    dev = x.device
    K, E = shape.top_k, shape.n_experts
    _expect_layer(shape, T, x, w_router, bias)
    o = out or {}
    idx = o.get("idx", torch.empty(T, K, dtype=torch.int32, device=dev))
    gate = o.get("gate", torch.empty(T, K, dtype=torch.float32, device=dev))
    counts = o.get("counts", torch.empty(E, dtype=torch.int32, device=dev))
    _expect_routing_out(shape, T, idx, gate, counts)
    lg = torch.empty(T, E, dtype=torch.float32, device=dev) if logits else None
    if ws is None:
        ws = workspace(shape, T, dev)
    _dev(x, w_router, bias, idx, gate, counts, lg, ws)
    _check(lib().lcmoe_route(ctypes.byref(shape), T, _ptr(x), _ptr(w_router), _ptr(bias),
                             _ptr(idx), _ptr(gate), _ptr(counts), _ptr(lg), _ptr(ws),
                             ws.numel(), _stream()), "lcmoe_route")
    return dict(idx=idx, gate=gate, counts=counts, logits=lg)


def permute(shape, topk_idx, ws=None):
    """Counting-sort permutation of the FFN slots of `topk_idx` [T,K] int32.

    Returns dict(counts [E], offsets [N+1], perm [T*K], row_of_slot [T*K]), int32.
    """
    T = topk_idx.shape[0]
    dev = topk_idx.device
    K, E, N = shape.top_k, shape.n_experts, shape.n_ffn
    _expect("topk_idx", topk_idx, torch.int32, (T, K))
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(N + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * K, dtype=torch.int32, device=dev)
    row_of_slot = torch.empty(T * K, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(shape, T, dev)
    _dev(topk_idx, counts, offsets, perm, row_of_slot, ws)
    _check(lib().lcmoe_permute(ctypes.byref(shape), T, _ptr(topk_idx), _ptr(counts),
                               _ptr(offsets), _ptr(perm), _ptr(row_of_slot), _ptr(ws),
                               ws.numel(), _stream()), "lcmoe_permute")
    return dict(counts=counts, offsets=offsets, perm=perm, row_of_slot=row_of_slot)


def u_rows(shape, T):
    """Rows of the saved pre-activation buffer of a T-token call: T * min(K, N)."""
    return int(T) * min(shape.top_k, shape.n_ffn)


def forward(shape, x, w_router, bias, w13, w2, w13_scale=None, w2_scale=None, ws=None,
            out=None, stage_events=None, u_save=None):
    """The whole layer. Returns dict(y bf16 [T,d], idx, gate, counts).

    stage_events: optional ctypes array of NUM_STAGES + 1 hipEvent_t handles
    recorded at the stage boundaries (lcmoe_forward_staged).
    u_save: optional fp32 [u_rows(shape, T), 2I] tensor; when given, the call
    is lcmoe_forward_train (bf16 weights), which also stores the gate/up
    pre-activations of every FFN slot row for backward(..., u_saved=...)."""
    T = x.shape[0]
    dev = x.device
    K, E, d = shape.top_k, shape.n_experts, shape.d_model
    _expect_layer(shape, T, x, w_router, bias)
    _expect_experts(shape, w13, w2, w13_scale, w2_scale)
    o = out or {}
    y = o.get("y", torch.empty(T, d, dtype=torch.bfloat16, device=dev))
    idx = o.get("idx", torch.empty(T, K, dtype=torch.int32, device=dev))
    gate = o.get("gate", torch.empty(T, K, dtype=torch.float32, device=dev))
    counts = o.get("counts", torch.empty(E, dtype=torch.int32, device=dev))
    _expect("y", y, torch.bfloat16, (T, d))
    _expect_routing_out(shape, T, idx, gate, counts)
    if u_save is not None:
        _expect("u_save", u_save, torch.float32, (u_rows(shape, T), 2 * shape.d_expert))
    if ws is None:
        ws = workspace(shape, T, dev)
    _dev(x, w_router, bias, w13, w2, w13_scale, w2_scale, y, idx, gate, counts, ws)
    if u_save is not None:
        _dev(u_save)
        _check(lib().lcmoe_forward_train(ctypes.byref(shape), T, _ptr(x), _ptr(w_router),
                                         _ptr(bias), _ptr(w13), _ptr(w2), _ptr(y), _ptr(idx),
                                         _ptr(gate), _ptr(counts), _ptr(u_save), _ptr(ws),
                                         ws.numel(), _stream()), "lcmoe_forward_train")
        return dict(y=y, idx=idx, gate=gate, counts=counts, u=u_save)
    args = (ctypes.byref(shape), T, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w13),
            _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(idx), _ptr(gate),
            _ptr(counts), _ptr(ws), ws.numel(), _stream())
    if stage_events is None:
        _check(lib().lcmoe_forward(*args), "lcmoe_forward")
    else:
        _check(lib().lcmoe_forward_staged(*args, stage_events), "lcmoe_forward_staged")
    return dict(y=y, idx=idx, gate=gate, counts=counts)


def forward_inspect(shape, x, w_router, bias, w13, w2, w13_scale, w2_scale, ws=None):
    """lcmoe_forward_inspect (fp8 weights and activations): the forward's
    outputs plus its fp8 activation intermediates. Returns dict(y, idx, gate,
    counts, xq uint8 [T,d], xs fp32 [T], h bf16 [S,I], hq uint8 [S,I],
    hs fp32 [S]) with S = u_rows(shape, T) rows allocated (rows at or past
    the FFN slot count are left unwritten)."""
    T = x.shape[0]
    dev = x.device
    K, E, d, I = shape.top_k, shape.n_experts, shape.d_model, shape.d_expert
    _expect_layer(shape, T, x, w_router, bias)
    _expect_experts(shape, w13, w2, w13_scale, w2_scale)
    S = u_rows(shape, T)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    gate = torch.empty(T, K, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    xq = torch.empty(T, d, dtype=torch.uint8, device=dev)
    xs = torch.empty(T, dtype=torch.float32, device=dev)
    h = torch.empty(S, I, dtype=torch.bfloat16, device=dev)
    hq = torch.empty(S, I, dtype=torch.uint8, device=dev)
    hs = torch.empty(S, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(shape, T, dev)
    _dev(x, w_router, bias, w13, w2, w13_scale, w2_scale, y, idx, gate, counts, xq, xs, h, hq, hs,
         ws)
    _check(lib().lcmoe_forward_inspect(ctypes.byref(shape), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                       _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                       _ptr(y), _ptr(idx), _ptr(gate), _ptr(counts), _ptr(xq),
                                       _ptr(xs), _ptr(h), _ptr(hq), _ptr(hs), _ptr(ws), ws.numel(),
                                       _stream()), "lcmoe_forward_inspect")
    return dict(y=y, idx=idx, gate=gate, counts=counts, xq=xq, xs=xs, h=h, hq=hq, hs=hs)


NOALLOC_SCRATCH_BYTES = 256 << 20


def forward_noalloc(shape, x, w_router, bias, w13, w2, w13_scale=None, w2_scale=None, out=None):
    """lcmoe_forward_noalloc: the forward on the library's fixed per-device
    scratch array (no workspace argument; the call itself allocates
    nothing). Output tensors may be passed in `out` (y, idx, gate, counts).
    Returns dict(y, idx, gate, counts)."""
    T = x.shape[0]
    dev = x.device
    K, E, d = shape.top_k, shape.n_experts, shape.d_model
    _expect_layer(shape, T, x, w_router, bias)
    _expect_experts(shape, w13, w2, w13_scale, w2_scale)
    o = out or {}
    y = o.get("y", torch.empty(T, d, dtype=torch.bfloat16, device=dev))
    idx = o.get("idx", torch.empty(T, K, dtype=torch.int32, device=dev))
    gate = o.get("gate", torch.empty(T, K, dtype=torch.float32, device=dev))
    counts = o.get("counts", torch.empty(E, dtype=torch.int32, device=dev))
    _expect("y", y, torch.bfloat16, (T, d))
    _expect_routing_out(shape, T, idx, gate, counts)
    _dev(x, w_router, bias, w13, w2, w13_scale, w2_scale, y, idx, gate, counts)
    _check(lib().lcmoe_forward_noalloc(ctypes.byref(shape), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                       _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                       _ptr(y), _ptr(idx), _ptr(gate), _ptr(counts), _stream()),
           "lcmoe_forward_noalloc")
    return dict(y=y, idx=idx, gate=gate, counts=counts)


def bias_update(shape, counts, mu, k_e, bias, t_all):
    """In-place bias update of the N FFN experts from `counts` of a T_all-token batch."""
    _expect("counts", counts, torch.int32, (shape.n_experts,))
    _expect("bias", bias, torch.float32, (shape.n_experts,))
    _dev(counts, bias)
    _check(lib().lcmoe_bias_update(ctypes.byref(shape), int(t_all), _ptr(counts),
                                   float(mu), float(k_e), _ptr(bias), _stream()),
           "lcmoe_bias_update")
    return bias


def router_stats_workspace_bytes(shape, n_groups):
    return int(lib().lcmoe_router_stats_workspace_bytes(ctypes.byref(shape), int(n_groups)))


def router_stats(shape, x, logits, counts, n_groups, k_e, alpha=1.0, lam=1.0, ws=None):
    """Device-level load-balance statistic (zero experts as group D+1) and the
    hidden z-loss of x. `logits` [T,E] fp32 and `counts` [E] int32 come from
    the same routing (route(..., logits=True)). Returns a device fp64 tensor
    [2 + 2(D+1)]: L_LB, L_Z, f_1..f_{D+1}, P_1..P_{D+1}."""
    T = x.shape[0]
    dev = x.device
    _expect("x", x, torch.bfloat16, (T, shape.d_model))
    _expect("logits", logits, torch.float32, (T, shape.n_experts))
    _expect("counts", counts, torch.int32, (shape.n_experts,))
    stats = torch.empty(2 + 2 * (int(n_groups) + 1), dtype=torch.float64, device=dev)
    if ws is None:
        n = router_stats_workspace_bytes(shape, n_groups)
        if n == 0:
            raise LcmoeError(ERR_INVALID_ARG, "invalid shape or n_groups")
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    _dev(x, logits, counts, stats, ws)
    _check(lib().lcmoe_router_stats(ctypes.byref(shape), T, _ptr(x), _ptr(logits), _ptr(counts),
                                    int(n_groups), float(k_e), float(alpha), float(lam),
                                    _ptr(stats), _ptr(ws), ws.numel(), _stream()),
           "lcmoe_router_stats")
    return stats


NUM_BWD_STAGES = 9
BWD_STAGES = ("route_gather", "w2t_dy", "u_silu", "dz", "dx_rows", "dw2", "dw13", "router_grads",
              "dx")


def backward_workspace_bytes(shape, max_tokens):
    return int(lib().lcmoe_backward_workspace_bytes(ctypes.byref(shape), int(max_tokens)))


def backward(shape, x, w_router, bias, w13, w2, dy, ws=None, out=None, stage_events=None,
             u_saved=None):
    """Gradients of <dy, y> for y = forward(...). Returns dict(dx fp32 [T,d],
    dw_router fp32 [E,d], dw13 bf16 [N,2I,d], dw2 bf16 [N,d,I]).
    u_saved: the pre-activations a forward(..., u_save=...) stored for the
    same x and parameters (lcmoe_backward_saved: u is not recomputed)."""
    T = x.shape[0]
    dev = x.device
    E, N, I, d = shape.n_experts, shape.n_ffn, shape.d_expert, shape.d_model
    _expect_layer(shape, T, x, w_router, bias)
    _expect_experts(shape, w13, w2)
    _expect("dy", dy, torch.bfloat16, (T, d))
    o = out or {}
    dx = o.get("dx", torch.empty(T, d, dtype=torch.float32, device=dev))
    dwr = o.get("dw_router", torch.empty(E, d, dtype=torch.float32, device=dev))
    dw13 = o.get("dw13", torch.empty(N, 2 * I, d, dtype=torch.bfloat16, device=dev))
    dw2 = o.get("dw2", torch.empty(N, d, I, dtype=torch.bfloat16, device=dev))
    _expect("dx", dx, torch.float32, (T, d))
    _expect("dw_router", dwr, torch.float32, (E, d))
    _expect("dw13", dw13, torch.bfloat16, (N, 2 * I, d))
    _expect("dw2", dw2, torch.bfloat16, (N, d, I))
    if u_saved is not None:
        _expect("u_saved", u_saved, torch.float32, (u_rows(shape, T), 2 * I))
    if ws is None:
        n = backward_workspace_bytes(shape, T)
        if n == 0:
            raise LcmoeError(ERR_INVALID_ARG, "invalid or unsupported shape")
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    _dev(x, w_router, bias, w13, w2, dy, dx, dwr, dw13, dw2, ws)
    if u_saved is not None:
        _dev(u_saved)
        _check(lib().lcmoe_backward_saved(ctypes.byref(shape), T, _ptr(x), _ptr(w_router),
                                          _ptr(bias), _ptr(w13), _ptr(w2), _ptr(dy),
                                          _ptr(u_saved), _ptr(dx), _ptr(dwr), _ptr(dw13),
                                          _ptr(dw2), _ptr(ws), ws.numel(), _stream()),
               "lcmoe_backward_saved")
        return dict(dx=dx, dw_router=dwr, dw13=dw13, dw2=dw2)
    args = (ctypes.byref(shape), T, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w13), _ptr(w2),
            _ptr(dy), _ptr(dx), _ptr(dwr), _ptr(dw13), _ptr(dw2), _ptr(ws), ws.numel(), _stream())
    if stage_events is None:
        _check(lib().lcmoe_backward(*args), "lcmoe_backward")
    else:
        _check(lib().lcmoe_backward_staged(*args, stage_events), "lcmoe_backward_staged")
    return dict(dx=dx, dw_router=dwr, dw13=dw13, dw2=dw2)

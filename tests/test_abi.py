"""C-ABI boundary tests that need no GPU.

The library must load and export every function declared in include/lcmoe.h;
argument validation must return the documented status before any HIP call,
so these run on a CPU-only host (fake, never-dereferenced device pointers).
"""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_biased_amd import lcmoe
from mixture_experts_layer_biased_amd.lcmoe import (ERR_INVALID_ARG, ERR_UNSUPPORTED,
                                                    ERR_WORKSPACE, make_shape)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcmoe.h")

FAKE = 0x10000           # 16-byte aligned, never dereferenced
MIS = 0x10008            # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lcmoe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = lcmoe.lib()
    decl = declared_functions()
    assert set(decl) == set(lcmoe.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name
    # and the shared object's dynamic symbol table agrees
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", lcmoe.LIB_PATH],
                         capture_output=True, text=True).stdout
    syms = set(re.findall(r"\bT (lcmoe_\w+)", out))
    assert set(decl) <= syms


def test_library_has_no_undefined_internal_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", lcmoe.LIB_PATH],
                         capture_output=True, text=True).stdout
    assert "lcmoe" not in out, out


def test_binding_stages_match_the_header():
    # the staged entry points write one event per stage boundary into a
    # caller array of (stage count + 1): the binding's counts and names must
    # be the header's enums, in order
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    fwd = dict((k, int(v)) for k, v in re.findall(r"\b(LCMOE_STAGE_[A-Z_]+|LCMOE_NUM_STAGES)\s*=\s*(\d+)", src))
    assert fwd.pop("LCMOE_NUM_STAGES") == lcmoe.NUM_STAGES == len(lcmoe.STAGES)
    names = [k[len("LCMOE_STAGE_"):].lower() for k, _ in sorted(fwd.items(), key=lambda kv: kv[1])]
    assert sorted(fwd.values()) == list(range(lcmoe.NUM_STAGES))
    assert names == list(lcmoe.STAGES)
    # the backward's staged call documents its event count
    n_bwd = int(re.search(r"recording the caller's (\d+) events", open(HEADER).read()).group(1))
    assert n_bwd == lcmoe.NUM_BWD_STAGES + 1 == len(lcmoe.BWD_STAGES) + 1


def test_status_strings():
    assert lcmoe.status_str(0) == "LCMOE_OK"
    assert lcmoe.status_str(3) == "LCMOE_ERR_WORKSPACE"


def _route(shape, T, x=FAKE, wr=FAKE, b=FAKE, idx=FAKE, g=FAKE, c=FAKE, lg=None, ws=None, wsb=0):
    L = lcmoe.lib()
    return L.lcmoe_route(ctypes.byref(shape), T, x, wr, b, idx, g, c, lg, ws, wsb, None)


def _forward(shape, T, x=FAKE, wr=FAKE, b=FAKE, w13=FAKE, s13=None, w2=FAKE, s2=None, y=FAKE,
             idx=FAKE, g=FAKE, c=FAKE, ws=None, wsb=0):
    L = lcmoe.lib()
    return L.lcmoe_forward(ctypes.byref(shape), T, x, wr, b, w13, s13, w2, s2, y, idx, g, c,
                           ws, wsb, None)


GOOD = dict(d_model=64, n_ffn=8, n_zero=4, top_k=3, d_expert=32)


def shp(**kw):
    a = dict(GOOD)
    a.update(kw)
    return make_shape(a["d_model"], a["n_ffn"], a["n_zero"], a["top_k"], a["d_expert"],
                      a.get("w_dtype", 0))


@pytest.mark.parametrize("kw,status", [
    (dict(n_ffn=0), ERR_INVALID_ARG),
    (dict(n_zero=-1), ERR_INVALID_ARG),
    (dict(top_k=0), ERR_INVALID_ARG),
    (dict(top_k=13), ERR_INVALID_ARG),            # K > N+Z
    (dict(w_dtype=7), ERR_INVALID_ARG),
    (dict(n_ffn=100, top_k=65), ERR_UNSUPPORTED),  # K > 64
    (dict(n_ffn=2000, n_zero=100), ERR_UNSUPPORTED),
    (dict(d_model=48), ERR_UNSUPPORTED),
    (dict(d_expert=40), ERR_UNSUPPORTED),
    (dict(w_dtype=1), ERR_UNSUPPORTED),            # fp8 needs d, I % 128 == 0
    (dict(w_dtype=2), ERR_UNSUPPORTED),            # fp8 activations too
    (dict(w_dtype=3), ERR_INVALID_ARG),
    (dict(d_model=32768, d_expert=32768), ERR_UNSUPPORTED),  # one W13 of 4 GiB
])
def test_invalid_shapes(kw, status):
    assert _route(shp(**kw), 4) == status
    assert _forward(shp(**kw), 4) == status
    assert lcmoe.workspace_bytes(shp(**kw), 4) == 0


def test_invalid_arguments_route():
    s = shp()
    assert _route(s, -1) == ERR_INVALID_ARG
    assert _route(s, 4, x=None) == ERR_INVALID_ARG
    assert _route(s, 4, c=None) == ERR_INVALID_ARG
    assert _route(s, 4, idx=None) == ERR_INVALID_ARG
    assert _route(s, 4, x=MIS) == ERR_UNSUPPORTED
    assert _route(s, 4, ws=None) == ERR_WORKSPACE
    need = lcmoe.workspace_bytes(s, 4)
    assert _route(s, 4, ws=FAKE, wsb=64) == ERR_WORKSPACE
    assert need > 64
    big = 2 ** 31 // 3 + 1
    assert _route(s, big) == ERR_UNSUPPORTED       # T*K >= 2^31


def test_invalid_arguments_forward_and_bias():
    s = shp()
    assert _forward(s, 4, w13=None) == ERR_INVALID_ARG
    assert _forward(s, 4, y=None) == ERR_INVALID_ARG
    assert _forward(s, 4, y=MIS) == ERR_UNSUPPORTED
    assert _forward(s, 4, ws=FAKE, wsb=1024) == ERR_WORKSPACE
    f = make_shape(128, 8, 4, 3, 128, 1)
    assert _forward(f, 4) == ERR_INVALID_ARG        # fp8 without scales
    wide = make_shape(8192, 8, 4, 3, 32)
    assert _forward(wide, 2 ** 18) == ERR_UNSUPPORTED  # x of 4 GiB (32-bit gather offsets)
    L = lcmoe.lib()
    assert L.lcmoe_bias_update(ctypes.byref(s), 0, FAKE, 1e-3, 2.0, FAKE, None) == ERR_INVALID_ARG
    assert L.lcmoe_bias_update(ctypes.byref(s), 16, None, 1e-3, 2.0, FAKE, None) == ERR_INVALID_ARG
    assert L.lcmoe_bias_update(ctypes.byref(s), 16, FAKE, float("nan"), 2.0, FAKE,
                               None) == ERR_INVALID_ARG
    assert L.lcmoe_permute(ctypes.byref(s), 4, None, FAKE, FAKE, FAKE, FAKE, None, 0,
                           None) == ERR_INVALID_ARG
    assert L.lcmoe_permute(ctypes.byref(s), 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                           None) == ERR_WORKSPACE


@pytest.mark.parametrize("dims", [
    (64, 8, 4, 3, 32), (1024, 64, 32, 6, 512), (6144, 512, 256, 12, 2048)])
def test_workspace_monotone(dims):
    s = make_shape(*dims)
    prev = 0
    for T in [0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 129, 1000, 4096, 8192, 16384, 32768]:
        n = lcmoe.workspace_bytes(s, T)
        assert n >= prev, (T, n, prev)
        prev = n
    # large-shape workspace is dominated by the H and Y spills: T*min(K,N)*(I+d)*2
    d, N, Z, K, I = dims
    assert lcmoe.workspace_bytes(s, 8192) >= 8192 * min(K, N) * (I + d) * 2


@pytest.mark.parametrize("dims", [(64, 8, 4, 3, 32), (1024, 64, 32, 6, 512), (512, 100, 28, 4, 64)])
def test_workspace_monotone_past_32k_tokens(dims):
    # With few experts (E <= 128) the router still splits its k range beyond
    # 32768 tokens; the size must stay non-decreasing there, forward and
    # backward, at every run boundary of 256 tokens and around it.
    s = make_shape(*dims)
    Ts = sorted({t for j in range(127, 520, 7) for t in (256 * j - 1, 256 * j, 256 * j + 1)}
                | {32767, 32768, 32769, 65535, 65536, 65537, 131073})
    prev_f = prev_b = 0
    for T in Ts:
        f, b = lcmoe.workspace_bytes(s, T), lcmoe.backward_workspace_bytes(s, T)
        assert f >= prev_f and b >= prev_b, (T, f, prev_f, b, prev_b)
        prev_f, prev_b = f, b


def test_noalloc_validation():
    # lcmoe_forward_noalloc validates like lcmoe_forward and rejects a batch
    # whose workspace exceeds its fixed array, all before any HIP call
    L = lcmoe.lib()

    def fwd(sh, T, **kw):
        a = dict(x=FAKE, wr=FAKE, b=FAKE, w13=FAKE, s13=None, w2=FAKE, s2=None, y=FAKE, idx=FAKE,
                 g=FAKE, c=FAKE)
        a.update(kw)
        return L.lcmoe_forward_noalloc(ctypes.byref(sh), T, a["x"], a["wr"], a["b"], a["w13"],
                                       a["s13"], a["w2"], a["s2"], a["y"], a["idx"], a["g"],
                                       a["c"], None)

    s = shp()
    assert fwd(s, -1) == ERR_INVALID_ARG
    assert fwd(s, 4, c=None) == ERR_INVALID_ARG
    assert fwd(s, 4, w13=None) == ERR_INVALID_ARG
    assert fwd(s, 4, y=MIS) == ERR_UNSUPPORTED
    assert fwd(shp(w_dtype=7), 4) == ERR_INVALID_ARG
    assert fwd(make_shape(128, 8, 4, 3, 128, 1), 4) == ERR_INVALID_ARG   # fp8 without scales
    big = make_shape(6144, 512, 256, 12, 2048)
    assert lcmoe.workspace_bytes(big, 4096) > lcmoe.NOALLOC_SCRATCH_BYTES
    assert fwd(big, 4096) == ERR_WORKSPACE
    assert fwd(big, 2 ** 31 // 12 + 1) == ERR_UNSUPPORTED


def test_zero_tokens_validation():
    # T = 0 still validates its arguments before anything is enqueued
    s = shp()
    assert _route(s, 0, c=None) == ERR_INVALID_ARG
    assert _forward(s, 0, c=None) == ERR_INVALID_ARG
    assert _forward(shp(w_dtype=1), 0) == ERR_UNSUPPORTED
    L = lcmoe.lib()
    assert L.lcmoe_permute(ctypes.byref(s), 0, FAKE, None, FAKE, FAKE, FAKE, None, 0,
                           None) == ERR_INVALID_ARG
    assert _backward(s, 0, dw13=None) == ERR_INVALID_ARG
    assert lcmoe.workspace_bytes(s, 0) > 0


def _stats(shape, T, x=FAKE, lg=FAKE, c=FAKE, D=2, k_e=2.0, alpha=1.0, lam=1.0, st=FAKE, ws=None,
           wsb=0):
    L = lcmoe.lib()
    return L.lcmoe_router_stats(ctypes.byref(shape), T, x, lg, c, D, k_e, alpha, lam, st, ws, wsb,
                                None)


def test_router_stats_validation():
    s = shp()                      # N=8, Z=4, K=3
    assert lcmoe.router_stats_workspace_bytes(s, 2) >= 256 * 4 * 8
    for bad_d in (0, -1, 3, 16):
        assert lcmoe.router_stats_workspace_bytes(s, bad_d) == 0
        assert _stats(s, 4, D=bad_d) == ERR_INVALID_ARG
    assert _stats(s, 4, k_e=0.0) == ERR_INVALID_ARG
    assert _stats(s, 4, k_e=3.5) == ERR_INVALID_ARG      # k_e > K
    assert _stats(s, 4, k_e=float("nan")) == ERR_INVALID_ARG
    assert _stats(s, 4, alpha=float("inf")) == ERR_INVALID_ARG
    assert _stats(s, 4, lam=float("nan")) == ERR_INVALID_ARG
    assert _stats(s, -1) == ERR_INVALID_ARG
    assert _stats(s, 4, st=None) == ERR_INVALID_ARG
    assert _stats(s, 4, c=None) == ERR_INVALID_ARG
    assert _stats(s, 4, x=None) == ERR_INVALID_ARG
    assert _stats(s, 4, lg=None) == ERR_INVALID_ARG
    assert _stats(s, 4, x=MIS) == ERR_UNSUPPORTED
    assert _stats(s, 4, lg=MIS) == ERR_UNSUPPORTED
    assert _stats(s, 4) == ERR_WORKSPACE
    assert _stats(s, 4, ws=FAKE, wsb=64) == ERR_WORKSPACE
    assert _stats(shp(n_ffn=0), 4) == ERR_INVALID_ARG


def _backward(shape, T, x=FAKE, wr=FAKE, b=FAKE, w13=FAKE, w2=FAKE, dy=FAKE, dx=FAKE, dwr=FAKE,
              dw13=FAKE, dw2=FAKE, ws=None, wsb=0):
    return lcmoe.lib().lcmoe_backward(ctypes.byref(shape), T, x, wr, b, w13, w2, dy, dx, dwr,
                                      dw13, dw2, ws, wsb, None)


def test_backward_validation():
    s = shp()
    assert _backward(s, -1) == ERR_INVALID_ARG
    for arg in ("x", "wr", "b", "w13", "w2", "dy", "dx", "dwr", "dw13", "dw2"):
        assert _backward(s, 4, **{arg: None}) == ERR_INVALID_ARG, arg
    for arg in ("x", "dy", "dx", "dwr", "dw13", "dw2"):
        assert _backward(s, 4, **{arg: MIS}) == ERR_UNSUPPORTED, arg
    assert _backward(s, 4) == ERR_WORKSPACE
    need = lcmoe.backward_workspace_bytes(s, 4)
    assert need > 64
    assert _backward(s, 4, ws=FAKE, wsb=64) == ERR_WORKSPACE
    assert _backward(s, 2 ** 31 // 3 + 1) == ERR_UNSUPPORTED   # T*K >= 2^31
    wide = make_shape(8192, 8, 4, 3, 32)
    assert _backward(wide, 2 ** 18) == ERR_UNSUPPORTED  # slot rows of 4 GiB (32-bit offsets)
    # fp8 weights: no backward
    for wd in (1, 2):
        f = make_shape(128, 8, 4, 3, 128, wd)
        assert lcmoe.backward_workspace_bytes(f, 4) == 0
        assert _backward(f, 4) == ERR_UNSUPPORTED
    assert lcmoe.backward_workspace_bytes(s, -1) == 0


@pytest.mark.parametrize("dims", [(64, 8, 4, 3, 32), (6144, 512, 256, 12, 2048)])
def test_backward_workspace(dims):
    s = make_shape(*dims)
    d, N, Z, K, I = dims
    prev = 0
    for T in [0, 1, 2, 63, 64, 65, 1000, 8192]:
        n = lcmoe.backward_workspace_bytes(s, T)
        assert n >= prev, (T, n, prev)
        prev = n
    # per slot row: the gathered x and dy rows, the fp32 Q and dX rows, the
    # bf16 dU and g*h rows
    S = 8192 * min(K, N)
    assert lcmoe.backward_workspace_bytes(s, 8192) >= S * (4 * d + I * 4 + d * 4 + 2 * I * 2
                                                           + I * 2)


def test_training_pair_validation():
    L = lcmoe.lib()
    s = shp()
    fwd = lambda sh, T, u: L.lcmoe_forward_train(ctypes.byref(sh), T, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                  FAKE, FAKE, FAKE, FAKE, u, None, 0, None)
    bwd = lambda sh, T, u: L.lcmoe_backward_saved(ctypes.byref(sh), T, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                   FAKE, u, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert fwd(s, 4, None) == ERR_INVALID_ARG
    assert fwd(s, 4, MIS) == ERR_UNSUPPORTED
    assert fwd(s, 4, FAKE) == ERR_WORKSPACE
    assert bwd(s, 4, None) == ERR_INVALID_ARG
    assert bwd(s, 4, MIS) == ERR_UNSUPPORTED
    assert bwd(s, 4, FAKE) == ERR_WORKSPACE
    for wd in (1, 2):  # fp8 weights: no training pair
        f = make_shape(128, 8, 4, 3, 128, wd)
        assert fwd(f, 4, FAKE) == ERR_UNSUPPORTED
        assert bwd(f, 4, FAKE) == ERR_UNSUPPORTED
    assert lcmoe.u_rows(s, 10) == 10 * min(s.top_k, s.n_ffn)

"""Seeded synthetic inputs for the MoE layer (shared by tests and benchmark).

This module only draws random tensors and stores them in the formats the
layer consumes (bf16 activations and weights, fp8 E4M3FN codes with per-block
scales, fp32 router weights and bias). It performs none of the layer's
arithmetic and imports neither the HIP binding nor the oracle.

Workloads follow the layer shape of "LongCat-Flash" (llm-wiki entity page),
section 1 table: d_model 6144, 512 FFN experts, 256 zero-computation experts,
12 experts per token, expert intermediate size 2048; plus a tiny and a small
layer of the same structure. Every tensor has its own generator stream,
seeded seed*1000 + stream id (x 0, W_r 1, W13 2, W2 3, bias 4, skew subset 5,
bias-loop batch j 100+j, upstream gradient dy 7).
"""

from dataclasses import dataclass, field, replace

import torch

FP8_MAX = 448.0  # largest finite E4M3FN magnitude
FP8_BLOCK = 128


@dataclass(frozen=True)
class LayerConfig:
    name: str
    d: int            # d_model
    n_ffn: int        # N
    n_zero: int       # Z
    k: int            # top-K (zero experts included)
    inter: int        # expert intermediate size I
    tokens: int       # T
    seed: int
    wdtype: str = "bf16"          # "bf16", "fp8" (weights) or "fp8a8" (weights and activations)
    bias_std: float = 0.0         # router bias ~ N(0, bias_std) over all E, 0 -> zeros
    skew_frac: float = 0.0        # fraction of tokens scaled by skew_factor
    skew_factor: float = 1.0
    weight_std: float = 0.02
    extra: dict = field(default_factory=dict)

    @property
    def n_experts(self):
        return self.n_ffn + self.n_zero

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    # Tiny layer: d=64, 8 FFN + 4 zero experts, K=3, I=32, T=16, seed 0.
    "tiny": LayerConfig("tiny", 64, 8, 4, 3, 32, 16, seed=0),
    # Small layer: d=1024, 64 FFN + 32 zero, K=6, I=512, T=4096, bias ~ N(0, 0.1).
    "small": LayerConfig("small", 1024, 64, 32, 6, 512, 4096, seed=2, bias_std=0.1),
    # LongCat shape, decode batch: T=64, bias 0.
    "decode": LayerConfig("decode", 6144, 512, 256, 12, 2048, 64, seed=3),
    # LongCat shape, prefill batch: T=8192, 1% of tokens scaled x20.
    "prefill": LayerConfig("prefill", 6144, 512, 256, 12, 2048, 8192, seed=4,
                           skew_frac=0.01, skew_factor=20.0),
    # LongCat shape, fp8 E4M3 weights with 128x128 block scales, T=16384,
    # followed by 20 bias-update steps (mu=1e-3, K_e=8) on fresh batches.
    "fp8": LayerConfig("fp8", 6144, 512, 256, 12, 2048, 16384, seed=5, wdtype="fp8",
                       extra=dict(bias_steps=20, mu=1e-3, k_e=8.0)),
    # The fp8 configuration's layer and tokens with fp8 activations as well
    # (per-row E4M3FN quantization of expert inputs and intermediates, fp8
    # MFMA); same seed, so the same weights and tokens as "fp8".
    "fp8a8": LayerConfig("fp8a8", 6144, 512, 256, 12, 2048, 16384, seed=5, wdtype="fp8a8"),
    # LongCat shape, bf16, T=32768 (about 512 rows per FFN expert): the batch
    # at which the bf16 grouped GEMM has more MFMA work than weight bytes
    # (512 FLOP/B). An extra measurement point, not one of the five above.
    "prefill32k": LayerConfig("prefill32k", 6144, 512, 256, 12, 2048, 32768, seed=6),
    # One GPU's share of 8-way expert parallelism at the prefill batch: the 64
    # FFN experts of one rank and the 65,536 FFN slot rows it receives when 8
    # ranks route 8192 tokens each (about 1024 rows per local expert). Zero
    # experts never leave a token's home rank, so the shard has none; K = 8
    # FFN slots per token over 64 experts gives the same rows per expert.
    "ep8_shard": LayerConfig("ep8_shard", 6144, 64, 0, 8, 2048, 8192, seed=7),
}


def _gen(device, seed, stream):
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    return g


def make_tokens(cfg, device, stream=0, tokens=None, skew=True):
    """x: bf16 [T, d] ~ N(0, 1); optionally a seeded subset of round(frac*T)
    tokens scaled by skew_factor before the bf16 rounding."""
    T = cfg.tokens if tokens is None else tokens
    g = _gen(device, cfg.seed, stream)
    x = torch.randn(T, cfg.d, generator=g, device=device, dtype=torch.float32)
    if skew and cfg.skew_frac > 0 and T > 0:
        n_skew = int(round(cfg.skew_frac * T))
        gs = _gen(device, cfg.seed, 5)
        sel = torch.randperm(T, generator=gs, device=device)[:n_skew]
        x[sel] *= cfg.skew_factor
    return x.to(torch.bfloat16)


def make_upstream_grad(cfg, device, tokens=None):
    """dy: bf16 [T, d] ~ N(0, 1), the gradient arriving at the layer output
    (its own stream, independent of the tokens)."""
    T = cfg.tokens if tokens is None else tokens
    g = _gen(device, cfg.seed, 7)
    return torch.randn(T, cfg.d, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def quantize_fp8_blocks(w):
    """fp32 [R, C] -> (E4M3FN codes as uint8 [R, C], fp32 scales [R/128, C/128]).

    Per 128x128 block: s = amax / 448 (1 for an all-zero block), q = w / s
    rounded to nearest-even E4M3FN after clamping to +-448.
    """
    R, C = w.shape
    b = FP8_BLOCK
    blocks = w.view(R // b, b, C // b, b)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blocks / scale[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = q.view(R, C).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def make_router(cfg, device):
    """Router weights fp32 [E, d] ~ N(0, weight_std) and bias fp32 [E] (zeros,
    or N(0, bias_std)); the same tensors make_layer returns for `cfg`."""
    E, d = cfg.n_experts, cfg.d
    w_router = torch.randn(E, d, generator=_gen(device, cfg.seed, 1), device=device,
                           dtype=torch.float32) * cfg.weight_std
    if cfg.bias_std > 0:
        bias = torch.randn(E, generator=_gen(device, cfg.seed, 4), device=device,
                           dtype=torch.float32) * cfg.bias_std
    else:
        bias = torch.zeros(E, device=device, dtype=torch.float32)
    return w_router, bias


def make_layer(cfg, device):
    """Router, bias and expert weights for `cfg` on `device`.

    Returns dict with
      w_router fp32 [E, d]    ~ N(0, weight_std)
      bias     fp32 [E]       zeros, or N(0, bias_std)
      w13      bf16 [N, 2I, d]  or uint8 E4M3FN codes (fp8)
      w2       bf16 [N, d, I]   or uint8 codes
      w13_scale fp32 [N, 2I/128, d/128] (fp8 only, else None)
      w2_scale  fp32 [N, d/128, I/128]  (fp8 only, else None)
    Expert weights are drawn one expert at a time (bounded temporary memory).
    """
    E, d, N, I = cfg.n_experts, cfg.d, cfg.n_ffn, cfg.inter
    std = cfg.weight_std
    w_router, bias = make_router(cfg, device)
    g13 = _gen(device, cfg.seed, 2)
    g2 = _gen(device, cfg.seed, 3)
    fp8 = cfg.wdtype in ("fp8", "fp8a8")
    wdt = torch.uint8 if fp8 else torch.bfloat16
    w13 = torch.empty(N, 2 * I, d, device=device, dtype=wdt)
    w2 = torch.empty(N, d, I, device=device, dtype=wdt)
    w13_scale = w2_scale = None
    if fp8:
        w13_scale = torch.empty(N, 2 * I // FP8_BLOCK, d // FP8_BLOCK, device=device)
        w2_scale = torch.empty(N, d // FP8_BLOCK, I // FP8_BLOCK, device=device)
    for e in range(N):
        a = torch.randn(2 * I, d, generator=g13, device=device, dtype=torch.float32) * std
        c = torch.randn(d, I, generator=g2, device=device, dtype=torch.float32) * std
        if fp8:
            w13[e], w13_scale[e] = quantize_fp8_blocks(a)
            w2[e], w2_scale[e] = quantize_fp8_blocks(c)
        else:
            w13[e] = a.to(torch.bfloat16)
            w2[e] = c.to(torch.bfloat16)
    return dict(w_router=w_router, bias=bias, w13=w13, w2=w2,
                w13_scale=w13_scale, w2_scale=w2_scale)


def counted_routing_inputs(counts, d, device, seed):
    """Tokens and a router that send exactly counts[e] tokens to expert e
    (with top-1 selection and zero bias), in a seeded shuffled order.

    W_r is the E x d identity (E <= d), so logit z_e of a token is its x
    coordinate e, exact in fp32. Token t has x[choice_t] = 2 and every other
    coordinate uniform in (-1, 1) rounded to bf16, so its only maximum is its
    chosen expert. Returns x bf16 [T, d], W_r fp32 [E, d], bias fp32 [E] and
    the chosen expert of every token (int64 [T]).
    """
    E = len(counts)
    assert E <= d
    g = _gen(device, seed, 11)
    choice = torch.repeat_interleave(torch.arange(E, device=device),
                                     torch.as_tensor(counts, device=device))
    choice = choice[torch.randperm(choice.numel(), generator=g, device=device)]
    T = choice.numel()
    x = torch.rand(T, d, generator=g, device=device, dtype=torch.float32) * 2 - 1
    x[torch.arange(T, device=device), choice] = 2.0
    w = torch.zeros(E, d, device=device, dtype=torch.float32)
    w[torch.arange(E, device=device), torch.arange(E, device=device)] = 1.0
    return x.to(torch.bfloat16), w, torch.zeros(E, device=device), choice


def exact_router_inputs(T, d, E, device, seed, dup_pairs=0):
    """Inputs on which every fp32 router logit is exact under any summation order.

    x in {-8..8}/8 (bf16-exact), W_r in {-16..16}/1024, bias in Z*2^-13 with
    |b| <= 2. Every product is an integer multiple of 2^-13 and |partial sums|
    stay below 2^24 units for d <= 6144, so z and z+b are exact in fp32.
    dup_pairs > 0 copies router row 2j into row 2j+1 (and its bias) for
    j < dup_pairs, which forces exact score ties.
    """
    g = _gen(device, seed, 0)
    x = torch.randint(-8, 9, (T, d), generator=g, device=device).to(torch.float32) / 8
    w = torch.randint(-16, 17, (E, d), generator=g, device=device).to(torch.float32) / 1024
    b = torch.randint(-(2 ** 14), 2 ** 14 + 1, (E,), generator=g, device=device)
    b = b.to(torch.float32) / 2 ** 13
    for j in range(dup_pairs):
        if 2 * j + 1 < E:
            w[2 * j + 1] = w[2 * j]
            b[2 * j + 1] = b[2 * j]
    return x.to(torch.bfloat16), w, b

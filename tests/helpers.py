"""Test helpers: tensor <-> numpy conversion and expert-weight accessors.

Conversions here only reinterpret storage (bf16 bits, fp8 codes); all value
decoding goes through the oracle.
"""
import numpy as np
import torch

import oracle


def bf16_bits(t):
    """torch bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t):
    """torch bf16 tensor -> fp64 numpy values decoded by the oracle."""
    return oracle.bf16_bits_to_f64(bf16_bits(t))


def expert_getter(layer, wdtype, cache=None):
    """get_expert(e) -> (w13_e, w2_e) as fp64 numpy, decoded by the oracle."""
    w13, w2 = layer["w13"], layer["w2"]
    s13, s2 = layer.get("w13_scale"), layer.get("w2_scale")

    def get(e):
        if cache is not None and e in cache:
            return cache[e]
        if wdtype in ("fp8", "fp8a8"):
            a = oracle.dequant_fp8_blocks(w13[e].cpu().numpy(), s13[e].cpu().numpy())
            b = oracle.dequant_fp8_blocks(w2[e].cpu().numpy(), s2[e].cpu().numpy())
            out = (a.astype(np.float64), b.astype(np.float64))
        else:
            out = (bf16_values(w13[e]), bf16_values(w2[e]))
        if cache is not None:
            cache[e] = out
        return out

    return get

"""Test helpers: tensor <-> numpy conversion and expert-weight accessors.

Conversions here only reinterpret storage (bf16 bits, fp8 codes); all value
decoding goes through the oracle.
"""
import os

import numpy as np
import torch

import oracle


def bf16_bits(t):
    """torch bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t):
    """torch bf16 tensor -> fp64 numpy values decoded by the oracle."""
    return oracle.bf16_bits_to_f64(bf16_bits(t))


def expert_getter(layer, wdtype, cache=None, prefetch=None, ahead=24):
    """get_expert(e) -> (w13_e, w2_e) as fp64 numpy, decoded by the oracle.

    prefetch: optional list of the experts that will be requested, in
    request order; they are then decoded ahead by a thread pool, at most
    `ahead` at a time (each LongCat-shape expert is about 300 MB in fp64)."""
    w13, w2 = layer["w13"], layer["w2"]
    s13, s2 = layer.get("w13_scale"), layer.get("w2_scale")

    def decode(e):
        if wdtype in ("fp8", "fp8a8"):
            a = oracle.dequant_fp8_blocks(w13[e].cpu().numpy(), s13[e].cpu().numpy())
            b = oracle.dequant_fp8_blocks(w2[e].cpu().numpy(), s2[e].cpu().numpy())
            return (a.astype(np.float64), b.astype(np.float64))
        return (bf16_values(w13[e]), bf16_values(w2[e]))

    pending = {}
    order = [int(e) for e in prefetch] if prefetch is not None else []
    pool = None
    if order:
        from concurrent.futures import ThreadPoolExecutor
        pool = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
        for e in order[:ahead]:
            pending[e] = pool.submit(decode, e)
    nxt = [min(ahead, len(order))]

    def get(e):
        e = int(e)
        if cache is not None and e in cache:
            return cache[e]
        if e in pending:
            out = pending.pop(e).result()
            if nxt[0] < len(order):
                pending[order[nxt[0]]] = pool.submit(decode, order[nxt[0]])
                nxt[0] += 1
        else:
            out = decode(e)
        if not pending and pool is not None and nxt[0] >= len(order):
            pool.shutdown(wait=False)
        if cache is not None:
            cache[e] = out
        return out

    return get

"""Plain reference for the paged KV-cache write that precedes a decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU
library imports this module.

Source: aclnnMlaPrologV3WeightNz — "Parameters": kvCacheRef and krCacheRef
are updated in place at the positions cacheIndexOptional names; with
CacheMode "PA_BSND" the cache is (BlockNum, BlockSize, Nkv, D) and every
index is a slot in [0, BlockNum * BlockSize), one per token.  The write is
a copy: the stored bits of each source row land unchanged in the cache row
of slot s = cacheIndex[t], i.e. block s // BlockSize, position s % BlockSize.

Readings (also in the design notes): a slot outside [0, BlockNum *
BlockSize) is skipped (the page states the range but not what happens
outside it); the head-major pool (BlockNum, Nkv, BlockSize, D) takes the same
slot numbering; a write may cover channels col_offset .. col_offset + D - 1
of a wider cached row, which is how one row [latent 512 | rope 64] receives
kvCache and krCache.
"""

from __future__ import annotations

import torch


def cache_write(cache: torch.Tensor, layout: str, src: torch.Tensor, slot_index, col_offset: int = 0) -> torch.Tensor:
    """Return a copy of ``cache`` after the write (the input is left alone).

    cache: "paged_bsh" (BlockNum, BlockSize, Nkv, W) or "paged" (BlockNum,
    Nkv, BlockSize, W), any dtype; src: (T, Nkv, D) of the cache's dtype with
    col_offset + D <= W; slot_index: T integers.  Pure-Python loop over
    tokens and heads, a plain element copy per row.
    """
    out = cache.detach().to("cpu").clone()
    s = src.detach().to("cpu")
    if layout == "paged_bsh":
        n_blocks, block_size, n_kv, _ = out.shape
    elif layout == "paged":
        n_blocks, n_kv, block_size, _ = out.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    T, n_kv_src, D = s.shape
    if n_kv_src != n_kv:
        raise ValueError("source and cache disagree on the KV heads")
    idx = [int(x) for x in torch.as_tensor(slot_index).to("cpu").tolist()]
    for t in range(T):
        slot = idx[t]
        if slot < 0 or slot >= n_blocks * block_size:
            continue  # outside the pool: skipped
        blk, pos = slot // block_size, slot % block_size
        for g in range(n_kv):
            if layout == "paged_bsh":
                out[blk, pos, g, col_offset:col_offset + D] = s[t, g]
            else:
                out[blk, g, pos, col_offset:col_offset + D] = s[t, g]
    return out

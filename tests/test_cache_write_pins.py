"""Pins for the oracle's paged KV-cache write (aclnnMlaPrologV3WeightNz
"Parameters": kvCacheRef / krCacheRef updated in place at cacheIndexOptional,
CacheMode PA_BSND, slots in [0, BlockNum * BlockSize)).

The write is tied to the decode's gather, which is pinned separately: tokens
written at the slots a block table assigns must read back, through that
table, as exactly the rows that were written."""

import numpy as np
import pytest
import torch

import oracle


def _pool(layout, n_blocks, bs, n_kv, w, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    shape = (n_blocks, bs, n_kv, w) if layout == "paged_bsh" else (n_blocks, n_kv, bs, w)
    x = torch.randn(shape, generator=g)
    return (torch.round(x * 30).clamp(-128, 127) if dtype == torch.int8 else x).to(dtype)


@pytest.mark.parametrize("layout", ["paged", "paged_bsh"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int8])
def test_written_tokens_read_back_through_the_block_table(layout, dtype):
    bs, n_kv, D = 16, 2, 8
    lengths = [0, 1, 15, 16, 17, 40]
    nb = [(L + bs - 1) // bs for L in lengths]
    n_blocks = sum(nb) + 3
    rng = np.random.default_rng(4)
    perm = rng.permutation(n_blocks)
    table = np.full((len(lengths), max(nb)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[k:k + n]
        k += n
    cache = _pool(layout, n_blocks, bs, n_kv, D, dtype, 1)
    src, slots = [], []
    g = torch.Generator().manual_seed(2)
    for b, L in enumerate(lengths):
        for j in range(L):
            slots.append(int(table[b, j // bs]) * bs + j % bs)
    T = len(slots)
    src = _pool("paged_bsh", T, 1, n_kv, D, dtype, 3).reshape(T, n_kv, D)
    out = oracle.cache_write(cache, layout, src, slots)
    t = 0
    for b, L in enumerate(lengths):
        for gh in range(n_kv):
            rows = oracle.gather_kv(out, layout, b, gh, L, table, bs)
            np.testing.assert_array_equal(rows, oracle.as_f64(src[t:t + L, gh]))
        t += L
    # every slot no token names keeps its bits
    named = torch.zeros(n_blocks * bs, dtype=torch.bool)
    named[torch.tensor(slots, dtype=torch.long)] = True
    view = (lambda c: c.reshape(n_blocks * bs, n_kv, D)) if layout == "paged_bsh" else \
        (lambda c: c.permute(0, 2, 1, 3).reshape(n_blocks * bs, n_kv, D))
    assert torch.equal(view(out)[~named].view(torch.uint8), view(cache)[~named].view(torch.uint8))


def test_slots_outside_the_pool_are_skipped():
    cache = _pool("paged_bsh", 3, 16, 1, 8, torch.float32, 5)
    src = torch.ones((3, 1, 8))
    out = oracle.cache_write(cache, "paged_bsh", src, [-1, 48, 47])
    assert torch.equal(out[:2], cache[:2]) and torch.equal(out[2, :15], cache[2, :15])
    assert torch.all(out[2, 15, 0] == 1)


def test_latent_and_rope_parts_fill_one_row():
    """aclnnMlaPrologV3WeightNz: kvCache (latent, 512 wide) and krCache (rope,
    64 wide) of one token; written into one cached row [latent | rope] at
    offsets 0 and 512 they equal one write of the concatenated row."""
    cache = _pool("paged_bsh", 4, 16, 1, 576, torch.bfloat16, 6)
    lat = _pool("paged_bsh", 5, 1, 1, 512, torch.bfloat16, 7).reshape(5, 1, 512)
    rope = _pool("paged_bsh", 5, 1, 1, 64, torch.bfloat16, 8).reshape(5, 1, 64)
    slots = [3, 17, 18, 40, 63]
    two = oracle.cache_write(oracle.cache_write(cache, "paged_bsh", lat, slots), "paged_bsh", rope, slots, col_offset=512)
    one = oracle.cache_write(cache, "paged_bsh", torch.cat([lat, rope], dim=2), slots)
    assert torch.equal(two.view(torch.int16), one.view(torch.int16))

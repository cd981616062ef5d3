"""GPU parity of the paged KV-cache write (ifa_kv_cache_write) against the
oracle's copy: bit-exact over the whole pool, for every dtype and both pool
layouts, then a decode step over the tokens just written."""

import numpy as np
import pytest
import torch

import attention_ifa_decode_amd as ifa
import oracle
from synth import make_workload

from test_gpu_decode import _announce, _full_check

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    return (torch.round(x * 30).clamp(-128, 127) if dtype == torch.int8 else x).to(dtype)


@pytest.mark.parametrize("layout", ["paged", "paged_bsh"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16", "i8"])
@pytest.mark.parametrize("d", [64, 128])
def test_cache_write_bit_exact(layout, dt, d):
    dtype = DT[dt]
    nb, bs, n_kv, T = 9, 32, 4, 50
    shape = (nb, bs, n_kv, d) if layout == "paged_bsh" else (nb, n_kv, bs, d)
    cache = _rand(shape, dtype, 1)
    src = _rand((T, n_kv, d), dtype, 2)
    rng = np.random.default_rng(3)
    slots = rng.permutation(nb * bs)[:T].tolist()
    slots[5], slots[17] = -1, nb * bs  # outside the pool: skipped
    _announce(f"cache write {layout} {dt} d={d}")
    idx = torch.tensor(slots, dtype=torch.int64)
    ref = oracle.cache_write(cache, layout, src, idx)
    got = ifa.kv_cache_write(src.cuda(), idx.cuda(), cache.cuda(), layout)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu().view(torch.uint8), ref.view(torch.uint8))


def test_cache_write_latent_and_rope_into_one_row():
    """The MLA row [latent 512 | rope 64]: two writes at offsets 0 and 512."""
    cache = _rand((6, 64, 1, 576), torch.bfloat16, 4)
    lat, rope = _rand((40, 1, 512), torch.bfloat16, 5), _rand((40, 1, 64), torch.bfloat16, 6)
    idx = torch.tensor(np.random.default_rng(7).permutation(6 * 64)[:40], dtype=torch.int64)
    ref = oracle.cache_write(oracle.cache_write(cache, "paged_bsh", lat, idx), "paged_bsh", rope, idx, col_offset=512)
    c = cache.cuda()
    ifa.kv_cache_write(lat.cuda(), idx.cuda(), c, "paged_bsh")
    ifa.kv_cache_write(rope.cuda(), idx.cuda(), c, "paged_bsh", col_offset=512)
    torch.cuda.synchronize()
    assert torch.equal(c.cpu().view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("layout", ["paged", "paged_bsh"])
def test_write_then_decode(layout):
    """A decode step as a server runs it: each sequence's new K/V row is
    written at position L_b (slot block_table[b][L_b / bs] * bs + L_b % bs),
    then the decode reads L_b + 1 tokens."""
    lens = [0, 15, 16, 63, 64, 200]
    bs = 16
    w = make_workload(batch=len(lens), n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", layout=layout, block_size=bs,
                      lengths=[L + 1 for L in lens], seed=91, extra_blocks=2)
    # the new rows, and the slots they go to
    new_k = _rand((len(lens), 2, 128), torch.bfloat16, 8)
    new_v = _rand((len(lens), 2, 128), torch.bfloat16, 9)
    bt = w.block_table.long()
    idx = torch.tensor([int(bt[b, L // bs]) * bs + L % bs for b, L in enumerate(lens)], dtype=torch.int64)
    k_ref = oracle.cache_write(w.k_cache, layout, new_k, idx)
    v_ref = oracle.cache_write(w.v_cache, layout, new_v, idx)
    wg = w.to("cuda")
    ifa.kv_cache_write(new_k.cuda(), idx.cuda(), wg.k_cache, layout)
    ifa.kv_cache_write(new_v.cuda(), idx.cuda(), wg.v_cache, layout)
    torch.cuda.synchronize()
    assert torch.equal(wg.k_cache.cpu().view(torch.int16), k_ref.view(torch.int16))
    assert torch.equal(wg.v_cache.cpu().view(torch.int16), v_ref.view(torch.int16))
    # the decode over the caches as written (bit-equal to the oracle's)
    w.k_cache, w.v_cache = k_ref, v_ref
    _full_check(w, 2)

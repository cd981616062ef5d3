"""Checks of the seeded input generators (no attention arithmetic here)."""

import math

import torch

from synth import config_workload, make_workload, paged_block_table, blocks_needed, CONFIGS


def test_block_table_is_bijection_onto_used_blocks():
    g = torch.Generator().manual_seed(3)
    lens = [0, 1, 127, 128, 129, 1000]
    table, pool = paged_block_table(lens, 128, 16, g, extra_blocks=5)
    assert pool == blocks_needed(lens, 128) + 5
    used = []
    for b, L in enumerate(lens):
        nb = (L + 127) // 128
        assert (table[b, nb:] == -1).all()
        used += table[b, :nb].tolist()
    assert len(used) == len(set(used)) == blocks_needed(lens, 128)
    assert all(0 <= u < pool for u in used)


def test_seeded_and_device_independent_structure():
    a = config_workload(3, batch=4, lengths=("uniform", 512, 8192))
    b = config_workload(3, batch=4, lengths=("uniform", 512, 8192))
    assert torch.equal(a.block_table, b.block_table)
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))  # NaN poison compares by bytes
    assert all(512 <= L <= 8192 for L in a.lengths())


def test_poisoning_marks_only_unread_slots():
    w = make_workload(batch=3, n_q=2, n_kv=1, qk_dim=8, kv_dtype="f16", layout="paged",
                      block_size=16, lengths=[5, 16, 20], seed=1, extra_blocks=2)
    bt = w.block_table.long()
    for b, L in enumerate(w.lengths()):
        for j in range(L):
            assert not torch.isnan(w.k_cache[bt[b, j // 16], 0, j % 16]).any()
        if L % 16:
            assert torch.isnan(w.k_cache[bt[b, (L - 1) // 16], 0, L % 16:]).all()
    wb = make_workload(batch=2, n_q=2, n_kv=1, qk_dim=8, kv_dtype="f32", layout="bnsd",
                       lengths=[3, 7], s_cap=10, seed=1)
    assert torch.isnan(wb.k_cache[0, :, 3:]).all() and not torch.isnan(wb.k_cache[0, :, :3]).any()


def test_int8_values_and_antiquant_ranges():
    w = make_workload(batch=1, n_q=8, n_kv=2, qk_dim=128, kv_dtype="i8", layout="paged",
                      block_size=32, lengths=[64], seed=2, sink=True)
    assert w.k_cache.dtype == torch.int8 and w.q.dtype == torch.bfloat16
    assert w.antiquant_scale.shape == (2, 2, 128)
    assert (w.antiquant_scale >= 0.02).all() and (w.antiquant_scale <= 0.04).all()
    assert (w.antiquant_offset >= -1).all() and (w.antiquant_offset <= 1).all()
    assert w.sink.shape == (8,) and w.sink.dtype == torch.float32


def test_config_shapes():
    assert CONFIGS[5]["qk_dim"] == 576 and CONFIGS[5]["v_dim"] == 512
    w = config_workload(5, batch=2, lengths=[100, 300], max_blocks_per_seq=4)
    assert w.v_aliases_k and w.k_cache.shape[1:] == (1, 128, 576)
    assert abs(w.scale - 1 / math.sqrt(192)) < 1e-15


def test_value_seed_keeps_structure_and_changes_values():
    """Timing copies of one workload (same seed, another value seed) share the
    lengths, block table, pool size and poisoned slots, so every copy is the
    same workload; only the values differ."""
    for layout in ("paged", "bnsd"):
        kw = dict(batch=3, n_q=4, n_kv=2, qk_dim=8, kv_dtype="bf16", layout=layout, block_size=16,
                  lengths=("uniform", 1, 60), s_cap=64 if layout == "bnsd" else None, seed=5)
        a = make_workload(**kw)
        b = make_workload(value_seed=99, **kw)
        assert a.lengths() == b.lengths()
        assert a.k_cache.shape == b.k_cache.shape
        if layout == "paged":
            assert torch.equal(a.block_table, b.block_table)
        assert torch.equal(torch.isnan(a.k_cache), torch.isnan(b.k_cache))
        assert torch.equal(torch.isnan(a.v_cache), torch.isnan(b.v_cache))
        valid = ~torch.isnan(a.k_cache)
        assert not torch.equal(a.k_cache[valid], b.k_cache[valid])
        assert not torch.equal(a.q, b.q)

"""Host-side tests of the binding's argument checks (no GPU, nothing queued).

Every tensor of a decode call must agree with the sizes the call passes to the
C ABI (which sees pointers only): cache heads and head dims against
num_key_value_heads and the query, the block table and lengths against the
batch, the sink against num_heads, antiquant parameters against (2, N_kv, D)
or (2), the tree mask against (B, S_q, S_q), and caller-supplied outputs
against (B, N_q, v_dim) / (B, N_q) in their dtype.  A mismatch raises
ValueError before any launch.
"""

import pytest
import torch

from attention_ifa_decode_amd._checks import check_decode, check_update


def _gqa(B=3, nq=8, nkv=2, d=128, bs=16, nblk=10, mb=4, dtype=torch.bfloat16, layout="paged"):
    q = torch.zeros(B, nq, d, dtype=dtype)
    if layout == "paged":
        k = torch.zeros(nblk, nkv, bs, d, dtype=dtype)
    elif layout == "paged_bsh":
        k = torch.zeros(nblk, bs, nkv * d, dtype=dtype)
    elif layout == "bnsd":
        k = torch.zeros(B, nkv, 64, d, dtype=dtype)
    else:
        k = torch.zeros(B, 64, nkv, d, dtype=dtype)
    v = torch.zeros_like(k)
    bt = torch.zeros(B, mb, dtype=torch.int32) if layout in ("paged", "paged_bsh") else None
    lens = torch.zeros(B, dtype=torch.int64)
    return dict(q=q, k_cache=k, v_cache=v, block_table=bt, actual_seq_lengths=lens, num_heads=nq,
                num_key_value_heads=nkv, kv_layout=layout)


def check(**kw):
    kw.setdefault("device_check", False)
    return check_decode(**kw)


@pytest.mark.parametrize("layout", ["paged", "paged_bsh", "bnsd", "bsnd"])
def test_valid_calls_give_their_sizes(layout):
    sh = check(**_gqa(layout=layout))
    assert (sh.batch, sh.n_q, sh.n_kv, sh.qk_dim, sh.v_dim) == (3, 8, 2, 128, 128)
    if layout.startswith("paged"):
        assert (sh.num_blocks, sh.block_size, sh.max_blocks, sh.s_cap) == (10, 16, 4, 0)
    else:
        assert (sh.num_blocks, sh.s_cap) == (0, 64)
    assert sh.out_dtype == torch.bfloat16 and sh.antiquant_mode == ""


def test_mla_alias_and_zero_kv_heads():
    q = torch.zeros(2, 128, 576, dtype=torch.bfloat16)
    kv = torch.zeros(5, 1, 128, 576, dtype=torch.bfloat16)
    sh = check(q=q, k_cache=kv, v_cache=kv, block_table=torch.zeros(2, 3, dtype=torch.int32),
               actual_seq_lengths=torch.zeros(2, dtype=torch.int64), num_heads=128, num_key_value_heads=1, v_dim=512)
    assert sh.alias and sh.v_dim == 512
    a = _gqa(nq=4, nkv=4, layout="bnsd")
    a["num_key_value_heads"] = 0
    assert check(**a).n_kv == 4


@pytest.mark.parametrize("mutate,match", [
    (lambda a: a.update(k_cache=torch.zeros(10, 4, 16, 128, dtype=torch.bfloat16)), "KV heads"),
    (lambda a: a.update(k_cache=torch.zeros(10, 2, 16, 64, dtype=torch.bfloat16)), "channels"),
    (lambda a: a.update(v_cache=torch.zeros(11, 2, 16, 128, dtype=torch.bfloat16)), "disagree"),
    (lambda a: a.update(v_cache=torch.zeros(10, 2, 16, 128, dtype=torch.float16)), "must be"),
    (lambda a: a.update(block_table=torch.zeros(2, 4, dtype=torch.int32)), "block_table"),
    (lambda a: a.update(block_table=torch.zeros(3, 4, dtype=torch.int64)), "int32"),
    (lambda a: a.update(block_table=None), "block_table"),
    (lambda a: a.update(actual_seq_lengths=torch.zeros(4, dtype=torch.int64)), "actual_seq_lengths"),
    (lambda a: a.update(actual_seq_lengths=torch.zeros(3, dtype=torch.int32)), "int64"),
    (lambda a: a.update(num_heads=16), "num_heads"),
    (lambda a: a.update(num_key_value_heads=3), "multiple"),
    (lambda a: a.update(learnable_sink=torch.zeros(7)), "learnable_sink"),
    (lambda a: a.update(learnable_sink=torch.zeros(8, dtype=torch.float64)), "float32"),
    (lambda a: a.update(antiquant_scale=torch.zeros(2), antiquant_offset=torch.zeros(2)), "int8"),
    (lambda a: a.update(kv_layout="bnsd"), "block_table"),
    (lambda a: a.update(kv_layout="nope"), "kv_layout"),
    (lambda a: a.update(out=torch.zeros(3, 8, 64, dtype=torch.bfloat16)), "out"),
    (lambda a: a.update(out=torch.zeros(3, 8, 128, dtype=torch.float32), out_dtype=torch.bfloat16), "out"),
    (lambda a: a.update(lse=torch.zeros(3, 7)), "lse"),
    (lambda a: a.update(lse=torch.zeros(3, 8, dtype=torch.float16)), "float32"),
    (lambda a: a.update(q=torch.zeros(3, 8, 128, dtype=torch.float16)), "query dtype"),
    (lambda a: a.update(q=torch.zeros(3, 128, 8, dtype=torch.bfloat16).transpose(1, 2)), "contiguous"),
    (lambda a: a.update(sparse_mode=9), "tree_mask"),
    (lambda a: a.update(sparse_mode=5), "sparse_mode"),
])
def test_mismatches_raise(mutate, match):
    a = _gqa()
    mutate(a)
    with pytest.raises(ValueError, match=match):
        check(**a)


def test_out_dtype_follows_a_supplied_out():
    """An fp32 out with no out_dtype is written as fp32, not in the query dtype."""
    a = _gqa()
    a["out"] = torch.zeros(3, 8, 128, dtype=torch.float32)
    assert check(**a).out_dtype == torch.float32


def test_contiguous_layouts_check_the_batch():
    a = _gqa(layout="bnsd")
    a["k_cache"] = a["v_cache"] = None
    a["k_cache"] = torch.zeros(4, 2, 64, 128, dtype=torch.bfloat16)
    a["v_cache"] = torch.zeros(4, 2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="sequences"):
        check(**a)
    b = _gqa(layout="bsnd")
    b["k_cache"] = torch.zeros(3, 64, 3 * 128, dtype=torch.bfloat16)
    b["v_cache"] = torch.zeros(3, 64, 3 * 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="N_kv"):
        check(**b)


def test_int8_antiquant_shapes():
    a = _gqa()
    a["k_cache"] = torch.zeros(10, 2, 16, 128, dtype=torch.int8)
    a["v_cache"] = torch.zeros(10, 2, 16, 128, dtype=torch.int8)
    with pytest.raises(ValueError, match="needs antiquant"):
        check(**a)
    for shp, mode in (((2,), "tensor"), ((2, 2, 128), "channel")):
        a["antiquant_scale"], a["antiquant_offset"] = torch.zeros(shp), torch.zeros(shp)
        assert check(**a).antiquant_mode == mode
    a["antiquant_scale"], a["antiquant_offset"] = torch.zeros(2, 2, 64), torch.zeros(2, 2, 64)
    with pytest.raises(ValueError, match="antiquant parameters"):
        check(**a)
    a["antiquant_scale"], a["antiquant_offset"] = torch.zeros(2), torch.zeros(2, 2, 128)
    with pytest.raises(ValueError, match="shape of antiquant_scale"):
        check(**a)


def test_multi_token_query_and_tree_mask():
    a = _gqa()
    a["q"] = torch.zeros(3, 4, 8, 128, dtype=torch.bfloat16)
    a["sparse_mode"] = 9
    a["tree_mask"] = torch.zeros(3, 4, 4, dtype=torch.uint8)
    sh = check(**a)
    assert sh.q_seq == 4 and sh.lead == (3, 4)
    a["out"] = torch.zeros(3, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        check(**a)
    del a["out"]
    a["tree_mask"] = torch.zeros(3, 4, 3, dtype=torch.uint8)
    with pytest.raises(ValueError, match="tree_mask"):
        check(**a)


def test_host_tensors_rejected_with_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        check_decode(**_gqa())


def test_update_operands():
    o = torch.zeros(5, 64)
    m = torch.zeros(5)
    assert check_update(o, m, m, o, m, m, device_check=False) == (5, 64, 1)
    m1 = torch.zeros(5, 1)
    assert check_update(o, m1, m1, o, m1, m1, device_check=False) == (5, 64, 1)
    m8 = torch.zeros(5, 8)
    assert check_update(o, m8, m8, o, m8, m8, device_check=False) == (5, 64, 8)
    with pytest.raises(ValueError, match="cur_out"):
        check_update(o, m, m, torch.zeros(5, 32), m, m, device_check=False)
    with pytest.raises(ValueError, match="cur_max"):
        check_update(o, m, m, o, torch.zeros(4), m, device_check=False)
    with pytest.raises(ValueError, match="statistics"):
        check_update(o, torch.zeros(5, 3), torch.zeros(5, 3), o, torch.zeros(5, 3), torch.zeros(5, 3),
                     device_check=False)
    with pytest.raises(ValueError, match="out"):
        check_update(o, m, m, o, m, m, out=torch.zeros(5, 64, dtype=torch.float16), device_check=False)
    with pytest.raises(ValueError, match="sum_out"):
        check_update(o, m, m, o, m, m, sum_out=torch.zeros(6), device_check=False)


def test_per_token_antiquant_shapes():
    """Per-token parameters (2, B, S) and (2, B, N_kv, S) over the logical
    capacity S (max_blocks_per_seq * block_size paged, S_cap contiguous);
    where (2, B, S) coincides with (2, N_kv, D) the mode must be named."""
    a = _gqa()  # B 3, N_kv 2, block 16, 4 blocks per sequence: S = 64
    a["k_cache"] = torch.zeros(10, 2, 16, 128, dtype=torch.int8)
    a["v_cache"] = torch.zeros(10, 2, 16, 128, dtype=torch.int8)
    for shp, mode in (((2, 3, 64), "token"), ((2, 3, 2, 64), "token_head")):
        a["antiquant_scale"], a["antiquant_offset"] = torch.zeros(shp), torch.zeros(shp)
        assert check(**a).antiquant_mode == mode
        assert check(antiquant_mode=mode, **a).antiquant_mode == mode
    a["antiquant_scale"], a["antiquant_offset"] = torch.zeros(2, 3, 63), torch.zeros(2, 3, 63)
    with pytest.raises(ValueError, match="antiquant parameters"):
        check(**a)
    a["antiquant_scale"], a["antiquant_offset"] = torch.zeros(2, 3, 64), torch.zeros(2, 3, 64)
    with pytest.raises(ValueError, match="needs parameters of shape"):
        check(antiquant_mode="channel", **a)
    # (2, B, S) == (2, N_kv, D): per channel unless named
    b = _gqa(B=2, nkv=2, mb=8)  # S = 128 = D
    b["k_cache"] = torch.zeros(10, 2, 16, 128, dtype=torch.int8)
    b["v_cache"] = torch.zeros(10, 2, 16, 128, dtype=torch.int8)
    b["antiquant_scale"], b["antiquant_offset"] = torch.zeros(2, 2, 128), torch.zeros(2, 2, 128)
    assert check(**b).antiquant_mode == "channel"
    assert check(antiquant_mode="token", **b).antiquant_mode == "token"
    c = _gqa(d=64)
    c["k_cache"] = torch.zeros(10, 2, 16, 64, dtype=torch.int8)
    c["v_cache"] = torch.zeros(10, 2, 16, 64, dtype=torch.int8)
    c["antiquant_scale"], c["antiquant_offset"] = torch.zeros(2, 3, 64), torch.zeros(2, 3, 64)
    with pytest.raises(ValueError, match="head dim 128"):
        check(antiquant_mode="token", **c)

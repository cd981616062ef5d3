"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library loads, exports every function include/ifa_decode.h declares, sizes
workspaces, and rejects bad arguments with the pages' status codes
(aclnnIncreFlashAttentionV3 "Return Value": 161001 null pointer, 161002
invalid parameter; 561002 for an unusable workspace) before queueing any work.
"""

import ctypes
import os
import re

import pytest

import attention_ifa_decode_amd as ifa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ifa_decode.h")
FAKE = 0x1000  # a non-NULL placeholder; never dereferenced on the host


def lib():
    if not os.path.exists(ifa.LIB_PATH):
        pytest.fail("library not built: run __graft_entry__.build() first")
    return ifa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(ifa.EXPORTED), names
    L = lib()
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    # the symbols are plain C (unmangled) in the dynamic symbol table
    out = os.popen(f"nm -D --defined-only {ifa.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), n


def base_args(**kw):
    a = ifa.DecodeArgs()
    a.query = a.key_cache = FAKE
    a.value_cache = FAKE + 0x100
    a.block_table = FAKE + 0x200
    a.actual_seq_lengths = FAKE + 0x300
    a.attention_out = FAKE + 0x400
    a.batch, a.num_heads, a.num_key_value_heads = 64, 32, 8
    a.qk_dim = a.v_dim = 128
    a.block_size, a.max_blocks_per_seq, a.num_blocks = 128, 64, 2300
    a.scale_value = 128 ** -0.5
    a.q_dtype = a.kv_dtype = a.out_dtype = ifa.IFA_BF16
    a.kv_layout = ifa.IFA_KV_PAGED
    a.num_splits = 4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def ws_size(a):
    sz = ctypes.c_size_t(0)
    st = lib().ifa_decode_workspace_size(ctypes.byref(a), ctypes.byref(sz))
    return st, sz.value


def test_workspace_size_formula():
    st, sz = ws_size(base_args())
    assert st == ifa.IFA_OK, ifa.last_error()
    rows = 64 * 32 * 4
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert sz == al(rows * 128 * 4) + 2 * al(rows * 4) + al(64 * 8)  # + the longest-first plan (B = 64)
    n = ctypes.c_int32()
    assert lib().ifa_decode_num_splits(ctypes.byref(base_args()), ctypes.byref(n)) == 0 and n.value == 4


def test_auto_splits_are_positive_and_deterministic():
    a = base_args(num_splits=0)
    n1, n2 = ctypes.c_int32(), ctypes.c_int32()
    assert lib().ifa_decode_num_splits(ctypes.byref(a), ctypes.byref(n1)) == 0
    assert lib().ifa_decode_num_splits(ctypes.byref(a), ctypes.byref(n2)) == 0
    assert 1 <= n1.value <= 256 and n1.value == n2.value


def test_batch_zero_needs_no_workspace():
    st, sz = ws_size(base_args(batch=0))
    assert st == 0 and sz == 0
    # and the launch with batch 0 is a no-op that queues nothing
    a = base_args(batch=0)
    assert lib().ifa_decode(ctypes.byref(a), None, 0, None) == 0


@pytest.mark.parametrize("field,value,code", [
    ("query", 0, ifa.IFA_ERR_PARAM_NULLPTR),
    ("key_cache", 0, ifa.IFA_ERR_PARAM_NULLPTR),
    ("actual_seq_lengths", 0, ifa.IFA_ERR_PARAM_NULLPTR),
    ("attention_out", 0, ifa.IFA_ERR_PARAM_NULLPTR),
    ("block_table", 0, ifa.IFA_ERR_PARAM_NULLPTR),
    ("num_heads", 257, ifa.IFA_ERR_PARAM_INVALID),
    ("num_heads", 0, ifa.IFA_ERR_PARAM_INVALID),
    ("num_key_value_heads", 5, ifa.IFA_ERR_PARAM_INVALID),   # 32 % 5 != 0
    ("batch", 65537, ifa.IFA_ERR_PARAM_INVALID),
    ("block_size", 120, ifa.IFA_ERR_PARAM_INVALID),           # not 16-aligned
    ("block_size", 2048, ifa.IFA_ERR_PARAM_INVALID),
    ("qk_dim", 96, ifa.IFA_ERR_PARAM_INVALID),
    ("v_dim", 64, ifa.IFA_ERR_PARAM_INVALID),
    ("q_dtype", ifa.IFA_I8, ifa.IFA_ERR_PARAM_INVALID),
    ("kv_dtype", ifa.IFA_F16, ifa.IFA_ERR_PARAM_INVALID),      # float KV must match q
    ("out_dtype", 7, ifa.IFA_ERR_PARAM_INVALID),
    ("kv_layout", 5, ifa.IFA_ERR_PARAM_INVALID),
    ("num_splits", -1, ifa.IFA_ERR_PARAM_INVALID),
    ("num_splits", 300, ifa.IFA_ERR_PARAM_INVALID),
    ("antiquant_mode", 1, ifa.IFA_ERR_PARAM_INVALID),          # set for a bf16 cache
    ("q_seq_len", 17, ifa.IFA_ERR_PARAM_INVALID),
    ("q_seq_len", -1, ifa.IFA_ERR_PARAM_INVALID),
    ("sparse_mode", 5, ifa.IFA_ERR_PARAM_INVALID),
    ("sparse_mode", ifa.IFA_MASK_TREE, ifa.IFA_ERR_PARAM_NULLPTR),  # no tree_mask
    ("reserved", 1, ifa.IFA_ERR_PARAM_INVALID),
    ("scale_value", float("nan"), ifa.IFA_ERR_PARAM_INVALID),
    ("max_blocks_per_seq", 0, ifa.IFA_ERR_PARAM_INVALID),
])
def test_invalid_arguments_are_rejected(field, value, code):
    a = base_args(**{field: value})
    st, _ = ws_size(a)
    assert st == code, (st, ifa.last_error())
    assert ifa.last_error()
    # phase 2 rejects the same arguments before touching the GPU
    assert lib().ifa_decode(ctypes.byref(a), FAKE, 1 << 30, None) == code


def test_int8_rules():
    a = base_args(kv_dtype=ifa.IFA_I8)
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_NULLPTR  # antiquant parameters missing
    a = base_args(kv_dtype=ifa.IFA_I8, antiquant_scale=FAKE, antiquant_offset=FAKE)
    assert ws_size(a)[0] == ifa.IFA_OK
    a = base_args(kv_dtype=ifa.IFA_I8, antiquant_scale=FAKE, antiquant_offset=FAKE,
                  antiquant_mode=ifa.IFA_ANTIQUANT_PER_TENSOR)
    assert ws_size(a)[0] == ifa.IFA_OK
    a = base_args(kv_dtype=ifa.IFA_I8, antiquant_scale=FAKE, antiquant_offset=FAKE, antiquant_mode=5)
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_INVALID


@pytest.mark.parametrize("layout", [ifa.IFA_KV_PAGED_BSH, ifa.IFA_KV_BSND])
def test_token_major_layouts_plan_like_head_major(layout):
    """The token-major layouts take the same arguments as their head-major
    twins (paged: block table, block size, pool; contiguous: s_cap) and give
    the same workspace."""
    twin = ifa.IFA_KV_PAGED if layout == ifa.IFA_KV_PAGED_BSH else ifa.IFA_KV_BNSD
    extra = {} if twin == ifa.IFA_KV_PAGED else dict(block_table=0, s_cap=4096)
    a, b = base_args(kv_layout=layout, **extra), base_args(kv_layout=twin, **extra)
    sa, sb = ws_size(a), ws_size(b)
    assert sa[0] == ifa.IFA_OK and sa == sb, (sa, sb, ifa.last_error())
    if twin == ifa.IFA_KV_PAGED:
        assert ws_size(base_args(kv_layout=layout, block_table=0))[0] == ifa.IFA_ERR_PARAM_NULLPTR
    a = base_args(kv_dtype=ifa.IFA_I8, antiquant_scale=FAKE, antiquant_offset=FAKE, block_size=48)
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_INVALID  # int8 needs 32-aligned blocks
    a = base_args(antiquant_scale=FAKE, antiquant_offset=FAKE)
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_INVALID  # antiquant with float KV


def test_mla_shape_rules():
    mla = dict(num_heads=128, num_key_value_heads=1, qk_dim=576, v_dim=512, max_blocks_per_seq=256)
    a = base_args(**mla)
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_INVALID  # V must alias K
    a = base_args(value_cache=FAKE, **mla)
    assert ws_size(a)[0] == ifa.IFA_OK, ifa.last_error()
    a = base_args(value_cache=FAKE, **dict(mla, num_key_value_heads=2))
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_INVALID
    # the MFMA path takes query heads in groups of 32
    a = base_args(value_cache=FAKE, **dict(mla, num_heads=48))
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_INVALID
    a = base_args(value_cache=FAKE, **dict(mla, num_heads=96))
    assert ws_size(a)[0] == ifa.IFA_OK, ifa.last_error()
    # one split may touch at most 1022 cache blocks (its block-table slice sits in LDS)
    long_seq = dict(mla, block_size=16, max_blocks_per_seq=4096, num_blocks=1 << 20)
    a = base_args(value_cache=FAKE, **dict(long_seq, num_splits=1))
    assert ws_size(a)[0] == ifa.IFA_ERR_PARAM_INVALID
    a = base_args(value_cache=FAKE, **dict(long_seq, num_splits=0))
    n = ctypes.c_int32()
    assert lib().ifa_decode_num_splits(ctypes.byref(a), ctypes.byref(n)) == ifa.IFA_OK, ifa.last_error()
    assert (4096 * 16 + n.value - 1) // n.value <= 1022 * 16


def test_workspace_too_small_or_misaligned():
    a = base_args()
    st, sz = ws_size(a)
    assert lib().ifa_decode(ctypes.byref(a), FAKE, sz - 1, None) == ifa.IFA_ERR_PLAN
    assert lib().ifa_decode_splitkv(ctypes.byref(a), FAKE, sz - 1, None) == ifa.IFA_ERR_PLAN
    assert lib().ifa_decode_combine(ctypes.byref(a), FAKE, sz - 1, None) == ifa.IFA_ERR_PLAN
    assert lib().ifa_decode(ctypes.byref(a), FAKE + 8, sz, None) == ifa.IFA_ERR_PARAM_INVALID
    assert lib().ifa_decode(ctypes.byref(a), None, sz, None) == ifa.IFA_ERR_PARAM_NULLPTR


def test_timed_splitkv_checks_before_launching():
    """The timed variant validates like ifa_decode_splitkv and requires both
    events; every case here is rejected on the host, before any launch."""
    a = base_args()
    st, sz = ws_size(a)
    L = lib()
    assert L.ifa_decode_splitkv_timed(ctypes.byref(a), FAKE, sz, None, None, FAKE) == ifa.IFA_ERR_PARAM_NULLPTR
    assert L.ifa_decode_splitkv_timed(ctypes.byref(a), FAKE, sz, None, FAKE, None) == ifa.IFA_ERR_PARAM_NULLPTR
    assert L.ifa_decode_splitkv_timed(ctypes.byref(a), FAKE, sz - 1, None, FAKE, FAKE) == ifa.IFA_ERR_PLAN
    bad = base_args(num_splits=-1)
    assert L.ifa_decode_splitkv_timed(ctypes.byref(bad), FAKE, sz, None, FAKE, FAKE) == ifa.IFA_ERR_PARAM_INVALID


def test_null_args_and_outputs():
    L = lib()
    sz = ctypes.c_size_t()
    assert L.ifa_decode_workspace_size(None, ctypes.byref(sz)) == ifa.IFA_ERR_PARAM_NULLPTR
    assert L.ifa_decode_workspace_size(ctypes.byref(base_args()), None) == ifa.IFA_ERR_PARAM_NULLPTR


def test_attn_update_argument_checks():
    L = lib()
    p = [FAKE] * 9
    assert L.attn_update(*p, 4, 64, ifa.IFA_BF16, 3, None) == ifa.IFA_ERR_PARAM_INVALID  # stride
    assert L.attn_update(*p, 4, 64, ifa.IFA_I8, 1, None) == ifa.IFA_ERR_PARAM_INVALID   # dtype
    assert L.attn_update(*p, -1, 64, ifa.IFA_F16, 1, None) == ifa.IFA_ERR_PARAM_INVALID
    assert L.attn_update(*p, 4, 0, ifa.IFA_F16, 1, None) == ifa.IFA_ERR_PARAM_INVALID
    q = list(p)
    q[4] = None
    assert L.attn_update(*q, 4, 64, ifa.IFA_F32, 8, None) == ifa.IFA_ERR_PARAM_NULLPTR
    assert L.attn_update(*p, 0, 64, ifa.IFA_F32, 8, None) == ifa.IFA_OK  # rows == 0: no-op


def test_block_count_worked_example():
    """aclnnMlaPrologV3WeightNz Constraints, BlockNum row: lengths
    [47, 104, 110, 161] at block size 128 occupy 5 blocks."""
    import json

    g = json.load(open(os.path.join(ROOT, "tests", "golden", "mla_blocknum_example.json")))
    assert ifa.paged_block_count(g["expected_lengths"], g["block_size"]) == g["expected_block_num"]
    assert ifa.paged_block_count([], 128) == 0
    with pytest.raises(ValueError):
        ifa.paged_block_count([-1], 128)


@pytest.mark.parametrize("kw,code", [
    (dict(tokens=-1), ifa.IFA_ERR_PARAM_INVALID),
    (dict(n_kv=0), ifa.IFA_ERR_PARAM_INVALID),
    (dict(d=100), ifa.IFA_ERR_PARAM_INVALID),            # 200 bytes: not a multiple of 16
    (dict(col_offset=8), ifa.IFA_ERR_PARAM_INVALID),     # 16 bytes, fine, but col_offset + d > row_elems
    (dict(layout=ifa.IFA_KV_BNSD), ifa.IFA_ERR_PARAM_INVALID),
    (dict(dtype=9), ifa.IFA_ERR_PARAM_INVALID),
    (dict(block_size=0), ifa.IFA_ERR_PARAM_INVALID),
    (dict(src=0), ifa.IFA_ERR_PARAM_NULLPTR),
    (dict(src=FAKE + 8), ifa.IFA_ERR_PARAM_INVALID),     # not 16-byte aligned
    (dict(tokens=0, src=0), ifa.IFA_OK),                 # empty: no-op before any pointer check
])
def test_cache_write_checks_before_launching(kw, code):
    a = dict(src=FAKE, slot_index=FAKE + 0x1000, cache=FAKE + 0x2000, tokens=64, n_kv=8, d=128, row_elems=128,
             col_offset=0, num_blocks=100, block_size=128, layout=ifa.IFA_KV_PAGED_BSH, dtype=ifa.IFA_BF16)
    a.update(kw)
    st = lib().ifa_kv_cache_write(a["src"], a["slot_index"], a["cache"], a["tokens"], a["n_kv"], a["d"],
                                  a["row_elems"], a["col_offset"], a["num_blocks"], a["block_size"], a["layout"],
                                  a["dtype"], None)
    assert st == code, (st, ifa.last_error())


def test_multi_token_decode_plans_rows_per_query_token():
    """S_q query tokens per sequence: the workspace holds S_q times the rows;
    the MLA shape takes one query token and no mask."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    st, sz = ws_size(base_args(q_seq_len=4, sparse_mode=ifa.IFA_MASK_CAUSAL, batch=64))
    assert st == ifa.IFA_OK, ifa.last_error()
    rows = 64 * 4 * 32 * 4
    assert sz == al(rows * 128 * 4) + 2 * al(rows * 4) + al(64 * 8)
    mla = dict(qk_dim=576, v_dim=512, num_heads=128, num_key_value_heads=1, value_cache=FAKE, num_splits=16)
    assert ws_size(base_args(**mla))[0] == ifa.IFA_OK, ifa.last_error()
    assert ws_size(base_args(q_seq_len=2, **mla))[0] == ifa.IFA_ERR_PARAM_INVALID
    assert ws_size(base_args(sparse_mode=ifa.IFA_MASK_CAUSAL, **mla))[0] == ifa.IFA_ERR_PARAM_INVALID


def split_mode(a):
    m = ctypes.c_int32(-1)
    st = lib().ifa_decode_split_mode(ctypes.byref(a), ctypes.byref(m))
    assert st == ifa.IFA_OK, ifa.last_error()
    return m.value


def test_mla_balanced_split_plan():
    """The MLA shape's automatic split is balanced (runs of the whole batch's
    tiles) for batch <= 256: n = 256 * 128 / N_q runs (at most 256), n + B
    partial slots, and the (first slot, count) pairs in the plan region.
    Explicit split counts, bigger batches and GQA split per sequence."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    mla = dict(qk_dim=576, v_dim=512, num_heads=128, num_key_value_heads=1, value_cache=FAKE, batch=32,
               max_blocks_per_seq=256)
    a = base_args(num_splits=0, **mla)
    assert split_mode(a) == 1
    n = ctypes.c_int32()
    assert lib().ifa_decode_num_splits(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == 256
    st, sz = ws_size(a)
    assert st == ifa.IFA_OK, ifa.last_error()
    rows = (256 + 32) * 128
    # attn_out partials in fp16 on the MLA shape, max and sum in fp32
    assert sz == al(rows * 512 * 2) + 2 * al(rows * 4) + al(32 * 8)
    # per-sequence split: the same element sizes
    st, sz = ws_size(base_args(num_splits=16, **mla))
    rows = 32 * 128 * 16
    assert st == ifa.IFA_OK and sz == al(rows * 512 * 2) + 2 * al(rows * 4) + al(32 * 8)
    for nq, runs in ((256, 128), (64, 256), (32, 256), (96, 256), (224, 146)):
        a = base_args(num_splits=0, **dict(mla, num_heads=nq))
        assert split_mode(a) == 1
        assert lib().ifa_decode_num_splits(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == runs, nq
    assert split_mode(base_args(num_splits=16, **mla)) == 0
    assert split_mode(base_args(num_splits=0, **dict(mla, batch=257))) == 0
    assert split_mode(base_args(num_splits=0, q_dtype=ifa.IFA_F32, kv_dtype=ifa.IFA_F32)) == 0  # GQA on VALU
    # a run longer than 1022 blocks of 16 tokens falls back to the per-sequence split
    big = dict(mla, batch=256, block_size=16, max_blocks_per_seq=1 << 14)
    assert split_mode(base_args(num_splits=0, **big)) == 0


def test_gqa_balanced_split_plan():
    """The automatic split of the GQA shapes on the matrix cores (head dim 128,
    16-bit or int8 K/V) is balanced for batch <= 256: one round of resident
    one-wave workgroups (1024 for 16-bit K/V, 2048 for int8),
    n = that / (N_kv * row groups) runs, fewer when the batch's
    units at full length (B (max_len / 32 + 8)) give a run less than 32 of
    them; partials in n + B slots of S_q * N_q rows.  int8 K/V with more than
    16 query rows per KV head, explicit split counts, batches over 256 and
    the VALU shapes split per sequence."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    n = ctypes.c_int32()

    def runs(a):
        assert lib().ifa_decode_num_splits(ctypes.byref(a), ctypes.byref(n)) == 0, ifa.last_error()
        return n.value

    # paged bf16, B 64, 8192 tokens at most, 4 rows per KV head: 1024 / 8 runs
    a = base_args(num_splits=0)
    assert split_mode(a) == 1 and runs(a) == 128
    st, sz = ws_size(a)
    assert st == ifa.IFA_OK, ifa.last_error()
    rows = (128 + 64) * 32
    assert sz == al(rows * 128 * 4) + 2 * al(rows * 4) + al(64 * 8)
    # the padded fp16 shape (B 16, s_cap 4096): one round, 1024 / 8 runs
    c2 = dict(num_splits=0, batch=16, kv_layout=ifa.IFA_KV_BNSD, s_cap=4096, q_dtype=ifa.IFA_F16,
              kv_dtype=ifa.IFA_F16, out_dtype=ifa.IFA_F16)
    assert split_mode(base_args(**c2)) == 1 and runs(base_args(**c2)) == 128
    # one sequence of at most one block (128 tokens): 4 tiles + 8 start units,
    # one run per unit
    assert runs(base_args(num_splits=0, batch=1, max_blocks_per_seq=1)) == 12
    # multi-token decode: 4 tokens x 4 heads = 16 rows per KV head, S_q N_q rows per slot
    mt = base_args(num_splits=0, q_seq_len=4, sparse_mode=ifa.IFA_MASK_CAUSAL)
    assert split_mode(mt) == 1 and runs(mt) == 128
    rows = (128 + 64) * 4 * 32
    assert ws_size(mt)[1] == al(rows * 128 * 4) + 2 * al(rows * 4) + al(64 * 8)
    # 64 rows per KV head: 2 row groups of 32 columns -> 1024 / 16 runs
    assert runs(base_args(num_splits=0, q_seq_len=16)) == 64
    # int8 K/V: balanced with at most 16 rows per KV head, per sequence above
    i8 = dict(num_splits=0, kv_dtype=ifa.IFA_I8, antiquant_scale=FAKE, antiquant_offset=FAKE,
              antiquant_mode=ifa.IFA_ANTIQUANT_PER_CHANNEL, num_heads=64)
    assert split_mode(base_args(**i8)) == 1 and runs(base_args(**i8)) == 256  # 2048 / 8
    assert split_mode(base_args(q_seq_len=4, **i8)) == 0
    assert split_mode(base_args(num_splits=4)) == 0
    assert split_mode(base_args(num_splits=0, batch=257, num_blocks=9000)) == 0
    assert split_mode(base_args(num_splits=0, qk_dim=64, v_dim=64)) == 0


def test_noalloc_rejects_oversize_calls_on_the_host():
    """ifa_decode_noalloc refuses, before touching any device, a call whose
    partials exceed its fixed array (IFA_NOALLOC_SCRATCH_BYTES, 128 MiB): the
    MLA shape with 256 splits of 40 sequences needs 40*128*256*514*4 bytes."""
    a = base_args(batch=40, num_heads=128, num_key_value_heads=1, qk_dim=576, v_dim=512, max_blocks_per_seq=1,
                  num_blocks=64, num_splits=256)
    a.value_cache = a.key_cache
    st, sz = ws_size(a)
    assert st == ifa.IFA_OK and sz > (128 << 20)
    assert lib().ifa_decode_noalloc(ctypes.byref(a), None) == ifa.IFA_ERR_PLAN
    assert "scratch" in ifa.last_error()
    bad = base_args(num_heads=0)
    assert lib().ifa_decode_noalloc(ctypes.byref(bad), None) == ifa.IFA_ERR_PARAM_INVALID


def test_per_token_antiquant_modes_on_the_host():
    """Per-token (2) and per-token-per-head (3) antiquant modes are accepted
    for int8 K/V with head dim 128 and rejected elsewhere; other codes are
    invalid."""
    i8 = dict(kv_dtype=ifa.IFA_I8, antiquant_scale=FAKE + 0x500, antiquant_offset=FAKE + 0x600)
    for mode in (ifa.IFA_ANTIQUANT_PER_TOKEN, ifa.IFA_ANTIQUANT_PER_TOKEN_HEAD):
        assert ws_size(base_args(antiquant_mode=mode, **i8))[0] == ifa.IFA_OK, ifa.last_error()
        st, _ = ws_size(base_args(antiquant_mode=mode, qk_dim=64, v_dim=64, **i8))
        assert st == ifa.IFA_ERR_PARAM_INVALID and "128" in ifa.last_error()
    assert ws_size(base_args(antiquant_mode=4, **i8))[0] == ifa.IFA_ERR_PARAM_INVALID
    assert ws_size(base_args(antiquant_mode=ifa.IFA_ANTIQUANT_PER_TOKEN))[0] == ifa.IFA_ERR_PARAM_INVALID


def test_check_inputs_argument_errors_on_the_host():
    """ifa_decode_check_inputs validates like the workspace query and needs a
    flags pointer; nothing is queued on an error."""
    assert lib().ifa_decode_check_inputs(ctypes.byref(base_args()), None, None) == ifa.IFA_ERR_PARAM_NULLPTR
    assert lib().ifa_decode_check_inputs(ctypes.byref(base_args(num_heads=0)), FAKE, None) == ifa.IFA_ERR_PARAM_INVALID
    assert lib().ifa_decode_check_inputs(ctypes.byref(base_args(block_table=0)), FAKE, None) == \
        ifa.IFA_ERR_PARAM_NULLPTR

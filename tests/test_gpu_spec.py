"""GPU parity of the multi-token decode (speculative verification) against
the oracle: S_q query tokens per sequence, the last S_q of its length, under
no mask, rightDownCausal, or a tree mask (B, S_q, S_q) with 1 = removed.
Tolerances as for one query token."""

import numpy as np
import pytest
import torch

import attention_ifa_decode_amd as ifa
import oracle
from synth import make_workload

from test_gpu_decode import TOL_F32, TOL_LOWP, TOL_LSE, _announce, half_ulp

pytestmark = pytest.mark.gpu

MODES = {"none": ifa.IFA_MASK_NONE, "causal": ifa.IFA_MASK_CAUSAL, "tree": ifa.IFA_MASK_TREE}


def _query(B, q_seq, n_q, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, q_seq, n_q, d), generator=g).to(dtype)


def _tree(B, q_seq, seed):
    rng = np.random.default_rng(seed)
    tm = (rng.random((B, q_seq, q_seq)) < 0.5).astype(np.uint8)
    for b in range(B):
        np.fill_diagonal(tm[b], 0)
    return torch.from_numpy(tm)


def _check(w, q, mode, tm, splits):
    _announce(f"spec decode B={w.batch} S_q={q.shape[1]} nq={w.n_q} nkv={w.n_kv} d={w.qk_dim} kv={w.kv_dtype} "
              f"layout={w.layout} mode={mode} lens={w.lengths()[:8]} splits={splits}")
    wg = w.to("cuda")
    out, lse = ifa.decode(q.cuda(), wg.k_cache, wg.v_cache, wg.block_table, wg.seq_lens, w.n_q, w.n_kv, w.scale,
                          learnable_sink=wg.sink, antiquant_scale=wg.antiquant_scale,
                          antiquant_offset=wg.antiquant_offset, num_splits=splits, v_dim=w.v_dim,
                          out_dtype=w.out_dtype, kv_layout=w.layout, sparse_mode=MODES[mode],
                          tree_mask=None if tm is None else tm.cuda(), antiquant_mode=w.antiquant_mode)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    ref_o, ref_l = oracle.decode_multi(q, w.k_cache, w.v_cache, w.layout, w.seq_lens, w.n_kv, w.scale,
                                       sparse_mode=MODES[mode], tree_mask=tm, block_table=w.block_table,
                                       block_size=w.block_size, sink=w.sink, antiquant_scale=w.antiquant_scale,
                                       antiquant_offset=w.antiquant_offset, v_dim=w.v_dim,
                                       antiquant_mode=w.antiquant_mode)
    assert out.shape == ref_o.shape and not np.isnan(out).any()
    tol = TOL_F32 if w.kv_dtype == torch.float32 else TOL_LOWP
    excess = np.abs(out - ref_o) - half_ulp(np.maximum(np.abs(out), np.abs(ref_o)), w.out_dtype)
    assert float(np.max(excess)) <= tol, float(np.max(excess))
    fin = np.isfinite(ref_l)
    np.testing.assert_array_equal(lse[~fin], ref_l[~fin])
    if fin.any():
        assert np.max(np.abs(lse[fin] - ref_l[fin])) <= TOL_LSE


@pytest.mark.parametrize("mode", ["none", "causal", "tree"])
@pytest.mark.parametrize("kv", ["f32", "f16", "bf16", "i8"])
def test_multi_token_every_dtype(mode, kv):
    """S_q 4 with group 4: sixteen query rows per KV head; lengths include
    L < S_q (queries that see nothing under the causal mask)."""
    q_seq, lens = 4, [1, 4, 5, 17, 130, 333]
    w = make_workload(batch=len(lens), n_q=8, n_kv=2, qk_dim=128, kv_dtype=kv, layout="paged", block_size=32,
                      lengths=lens, seed=101, sink=(kv == "i8"), extra_blocks=1)
    q = _query(len(lens), q_seq, 8, 128, w.q.dtype, 102)
    _check(w, q, mode, _tree(len(lens), q_seq, 103) if mode == "tree" else None, 3)


@pytest.mark.parametrize("mode", ["causal", "tree"])
@pytest.mark.parametrize("aq", ["token", "token_head"])
def test_multi_token_per_token_antiquant(mode, aq):
    """S_q 4 over an int8 cache with per-token antiquant pairs: the pairs
    follow the cached token positions, whatever the query token."""
    q_seq, lens = 4, [2, 5, 33, 300]
    w = make_workload(batch=len(lens), n_q=16, n_kv=4, qk_dim=128, kv_dtype="i8", layout="paged", block_size=32,
                      lengths=lens, seed=140, sink=True, antiquant_mode=aq, extra_blocks=1)
    q = _query(len(lens), q_seq, 16, 128, torch.bfloat16, 141)
    _check(w, q, mode, _tree(len(lens), q_seq, 142) if mode == "tree" else None, 2)


@pytest.mark.parametrize("mode", ["none", "causal", "tree"])
@pytest.mark.parametrize("aq", ["channel", "token", "token_head"])
def test_multi_token_int8_32_rows(mode, aq):
    """int8 with 32 query rows per KV head (S_q 4 x group 8): the 32-column
    MFMA kernel, whose V^T operands come through the byte-transposing read
    with offsets of their own for each 16-token k-step; lengths leave a
    ragged last tile and one tile-aligned sequence."""
    q_seq, lens = 4, [1, 4, 37, 300, 1030, 96]
    w = make_workload(batch=len(lens), n_q=16, n_kv=2, qk_dim=128, kv_dtype="i8", layout="paged", block_size=32,
                      lengths=lens, seed=150, sink=True, antiquant=True, antiquant_mode=aq, extra_blocks=1)
    q = _query(len(lens), q_seq, 16, 128, torch.bfloat16, 151)
    _check(w, q, mode, _tree(len(lens), q_seq, 152) if mode == "tree" else None, 3)


@pytest.mark.parametrize("q_seq,n_q,n_kv,d", [(2, 32, 8, 128), (3, 64, 8, 128), (7, 4, 4, 64), (16, 8, 8, 64),
                                             (5, 16, 2, 128)])
@pytest.mark.parametrize("mode", ["causal", "tree"])
def test_multi_token_shapes(q_seq, n_q, n_kv, d, mode):
    """Query tokens and groups that make workgroups span several query tokens
    (group 1 and 2), split a KV head's rows over several workgroups (3 x 8
    rows), and use the largest S_q."""
    lens = [q_seq, 40, 200, 1000]
    w = make_workload(batch=len(lens), n_q=n_q, n_kv=n_kv, qk_dim=d, kv_dtype="bf16", layout="paged",
                      block_size=64, lengths=lens, seed=110 + q_seq)
    q = _query(len(lens), q_seq, n_q, d, torch.bfloat16, 111)
    _check(w, q, mode, _tree(len(lens), q_seq, 112) if mode == "tree" else None, 4)


@pytest.mark.parametrize("layout", ["bnsd", "paged_bsh"])
def test_multi_token_layouts(layout):
    kw = dict(s_cap=512) if layout == "bnsd" else dict(block_size=16)
    w = make_workload(batch=3, n_q=16, n_kv=4, qk_dim=128, kv_dtype="f16", layout=layout, lengths=[6, 90, 500],
                      seed=120, **kw)
    q = _query(3, 6, 16, 128, torch.float16, 121)
    _check(w, q, "tree", _tree(3, 6, 122), 2)


def test_one_token_with_causal_mask_equals_plain_decode():
    w = make_workload(batch=4, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", layout="paged", block_size=32,
                      lengths=[1, 31, 32, 300], seed=130)
    wg = w.to("cuda")
    a = ifa.decode_workload(wg)
    q4 = wg.q[:, None]
    b = ifa.decode(q4, wg.k_cache, wg.v_cache, wg.block_table, wg.seq_lens, 8, 2, w.scale,
                   sparse_mode=ifa.IFA_MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0][:, 0]) and torch.equal(a[1], b[1][:, 0])

"""Pins for the oracle's multi-token decode (FusedInferAttentionScore blog:
sparseMode 3 rightDownCausal, 9 treeMask (B, Q_S, Q_S), 1 = removed).

Each mask is pinned through the single-query decode, which is pinned on its
own: a causal query equals the decode of a shorter sequence, and a tree
query equals the decode of a cache from which its removed draft tokens have
been physically dropped."""

import numpy as np
import pytest
import torch

import oracle
from oracle import spec_ref
from synth import make_workload

Q_S = 4


def _work(seed, lengths=(4, 5, 9, 40), layout="paged"):
    w = make_workload(batch=len(lengths), n_q=4, n_kv=2, qk_dim=16, kv_dtype="f32", layout=layout,
                      block_size=16, lengths=list(lengths), seed=seed, sink=True)
    g = torch.Generator().manual_seed(seed + 5)
    q = torch.randn((len(lengths), Q_S, 4, 16), generator=g)
    return w, q


def _kw(w):
    return dict(block_table=w.block_table, block_size=w.block_size, sink=w.sink)


def test_one_query_is_the_single_query_decode():
    w, q = _work(1)
    q1 = q[:, :1]
    ref_o, ref_l = oracle.decode(q1[:, 0], w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale, **_kw(w))
    for mode, tm in ((oracle.MASK_NONE, None), (oracle.MASK_CAUSAL, None),
                     (oracle.MASK_TREE, torch.zeros((4, 1, 1), dtype=torch.uint8))):
        o, l = oracle.decode_multi(q1, w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale, sparse_mode=mode,
                                   tree_mask=tm, **_kw(w))
        np.testing.assert_array_equal(o[:, 0], ref_o)
        np.testing.assert_array_equal(l[:, 0], ref_l)


def test_causal_query_is_a_shorter_sequence():
    """rightDownCausal: query i of Q_S sits at position L - Q_S + i, so it is
    the single-query decode of the first L - Q_S + i + 1 tokens."""
    w, q = _work(2)
    o, l = oracle.decode_multi(q, w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale,
                               sparse_mode=oracle.MASK_CAUSAL, **_kw(w))
    for i in range(Q_S):
        lens = w.seq_lens - (Q_S - 1 - i)
        ro, rl = oracle.decode(q[:, i], w.k_cache, w.v_cache, w.layout, lens, 2, w.scale, **_kw(w))
        np.testing.assert_allclose(o[:, i], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[:, i], rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_tree_query_is_a_cache_without_its_removed_drafts(seed):
    """treeMask: for each (b, i), copy the tokens the query keeps (all but the
    removed drafts) into a fresh contiguous cache and decode the query alone
    over it."""
    w, q = _work(seed)
    rng = np.random.default_rng(seed)
    tm = (rng.random((4, Q_S, Q_S)) < 0.5).astype(np.uint8)
    for b in range(4):
        np.fill_diagonal(tm[b], 0)
    o, l = oracle.decode_multi(q, w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale,
                               sparse_mode=oracle.MASK_TREE, tree_mask=torch.from_numpy(tm), **_kw(w))
    bt = w.block_table.long()
    for b, L in enumerate(w.lengths()):
        for i in range(Q_S):
            keep = [j for j in range(L) if j < L - Q_S or tm[b, i, j - (L - Q_S)] == 0]
            kc = torch.zeros((1, 2, max(1, len(keep)), 16))
            vc = torch.zeros((1, 2, max(1, len(keep)), 16))
            for n, j in enumerate(keep):
                kc[0, :, n] = w.k_cache[bt[b, j // 16], :, j % 16]
                vc[0, :, n] = w.v_cache[bt[b, j // 16], :, j % 16]
            ro, rl = oracle.decode(q[b:b + 1, i], kc, vc, "bnsd", torch.tensor([len(keep)]), 2, w.scale, sink=w.sink)
            np.testing.assert_allclose(o[b, i], ro[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(l[b, i], rl[0], rtol=0, atol=1e-12)


def test_causal_is_the_chain_tree_and_zero_tree_is_no_mask():
    w, q = _work(6)
    chain = torch.triu(torch.ones((Q_S, Q_S), dtype=torch.uint8), diagonal=1).expand(4, Q_S, Q_S).contiguous()
    a = oracle.decode_multi(q, w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale,
                            sparse_mode=oracle.MASK_CAUSAL, **_kw(w))
    b = oracle.decode_multi(q, w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale,
                            sparse_mode=oracle.MASK_TREE, tree_mask=chain, **_kw(w))
    np.testing.assert_array_equal(a[0], b[0])
    zero = torch.zeros((4, Q_S, Q_S), dtype=torch.uint8)
    c = oracle.decode_multi(q, w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale,
                            sparse_mode=oracle.MASK_TREE, tree_mask=zero, **_kw(w))
    d = oracle.decode_multi(q, w.k_cache, w.v_cache, w.layout, w.seq_lens, 2, w.scale, **_kw(w))
    np.testing.assert_array_equal(c[0], d[0])


def test_planted_off_by_one_is_caught(monkeypatch):
    orig = spec_ref.visible_tokens

    def strict(L, q_seq, i, mode, tree_row=None):
        j = orig(L, q_seq, i, mode, tree_row)
        return j[j < L - q_seq + i] if mode == oracle.MASK_CAUSAL else j

    monkeypatch.setattr(spec_ref, "visible_tokens", strict)
    with pytest.raises(AssertionError):
        test_causal_query_is_a_shorter_sequence()

"""Multi-token decode (speculative verification) with the masks of the
FusedInferAttentionScore pages.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU
library imports this module.

Source: FusedInferAttentionScore blog (lpqz.cn), the mask's sparseMode
values: 0 defaultMask (no masking when no mask is passed), 3 rightDownCausal,
9 treeMask, the tree-shaped attention mask of speculative decoding with shape
(B, Q_S, Q_S).  A mask entry of 1 removes a position, 0 keeps it (the pages'
optimised causal matrix is a lower triangle whose diagonal is all 0).

Readings where the pages are silent (also in the design notes):
* the Q_S queries of a sequence of actual length L are its last Q_S tokens,
  query i sitting at position L - Q_S + i;
* rightDownCausal: query i attends to token j iff j <= L - Q_S + i;
* treeMask: every query attends to all tokens before the last Q_S, and to
  the last-Q_S token k (position L - Q_S + k) iff tree_mask[b][i][k] == 0.
A query that attends to no token gives out 0 and lse -inf (reading R6).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attn_ref import _as_int, _kv_rows, as_f64, attention_row

MASK_NONE, MASK_CAUSAL, MASK_TREE = 0, 3, 9


def visible_tokens(L: int, q_seq: int, i: int, mode: int, tree_row=None) -> np.ndarray:
    """Indices j in [0, L) that query i of q_seq attends to."""
    j = np.arange(L, dtype=np.int64)
    if mode == MASK_NONE:
        return j
    base = L - q_seq  # position of query 0
    if mode == MASK_CAUSAL:
        return j[j <= base + i]
    if mode == MASK_TREE:
        k = j - base
        keep = k < 0
        inside = ~keep
        keep[inside] = np.asarray(tree_row)[k[inside]] == 0
        return j[keep]
    raise ValueError(f"unknown sparse mode {mode}")


def decode_multi(q, k_cache, v_cache, layout: str, seq_lens, n_kv: int, scale: float,
                 sparse_mode: int = MASK_NONE, tree_mask=None, block_table=None, block_size: int = 0,
                 sink=None, antiquant_scale=None, antiquant_offset=None, v_dim: Optional[int] = None,
                 v_from_k: bool = False, antiquant_mode: Optional[str] = None):
    """q (B, Q_S, N_q, qk_dim) -> (out (B, Q_S, N_q, v_dim), lse (B, Q_S, N_q)):
    each (query token, head) row is the decode attention of that row over
    the tokens the mask leaves it."""
    qf = as_f64(q)
    B, q_seq, n_q, qk_dim = qf.shape
    v_dim = qk_dim if v_dim is None else v_dim
    n_kv_e = n_q if n_kv == 0 else n_kv
    G = n_q // n_kv_e
    lens = _as_int(seq_lens)
    sinkf = as_f64(sink)
    aq_s, aq_o = as_f64(antiquant_scale), as_f64(antiquant_offset)
    tm = None if tree_mask is None else _as_int(tree_mask)
    out = np.zeros((B, q_seq, n_q, v_dim))
    lse = np.zeros((B, q_seq, n_q))
    for b in range(B):
        L = int(lens[b])
        for g in range(n_kv_e):
            K, V = _kv_rows(k_cache, v_cache, layout, b, g, L, block_table, block_size, qk_dim, v_dim, v_from_k,
                            aq_s, aq_o, antiquant_mode)
            for i in range(q_seq):
                idx = visible_tokens(L, q_seq, i, sparse_mode, None if tm is None else tm[b, i])
                for h in range(g * G, (g + 1) * G):
                    out[b, i, h], lse[b, i, h] = attention_row(qf[b, i, h], K[idx], V[idx], scale,
                                                               None if sinkf is None else float(sinkf[h]))
    return out, lse

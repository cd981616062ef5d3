"""Plain float64 reference for decode attention, its split partials and merge.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU
library imports this module.

Sources, by page title and section:

[IFA]   aclnnIncreFlashAttentionV3 — "Function": Attention(Q,K,V) =
        Softmax(Q K^T / sqrt(d)) V, query S fixed to 1, per-batch actual KV
        lengths; "Parameters": numHeads, numKeyValueHeads (0 means equal to
        numHeads), scaleValue, antiquantScale/antiquantOffset (index 0 is K,
        1 is V; per channel, or per tensor with shape (2)); "Constraints":
        page attention scenario (KV cache layouts (blocknum, KV_N,
        blocksize, D) and (blocknum, blocksize, H)), antiquant modes.
[RAU]   aclnnRingAttentionUpdate — "功能说明" (function) formula for updating
        an attention output from two (out, softmax_max, softmax_sum) results.
[SINK]  aclnnFlashAttentionScoreV4 — "计算公式" (formula): learnable sink.
[MLA]   aclnnMlaPrologV3WeightNz — "Constraints": BlockNum worked example;
        query/key split into a 512-wide latent part and a 64-wide rope part.
[FIA]   FusedInferAttentionScore blog (lpqz.cn) — empty-tensor semantics and
        the softmaxLse output that exists for splitting the S axis outside.

Readings where the pages are silent or garbled (each one is also listed with
its reason in the design notes):

R1  merge: the printed update omits cur_softmax_sum and the sum weights of the
    two outputs.  The oracle uses the weighted form
        M = max(pm, cm);  w_p = ps e^(pm-M);  w_c = cs e^(cm-M)
        sum = w_p + w_c;  out = (w_p po + w_c co) / sum
    which reduces to the printed formula when both sums are 1 (outputs in
    log-sum-exp form) and is the form under which merging the attention of
    any split of the KV axis gives the attention over the whole axis.
R2  antiquant: x_hat = (x + offset) * scale per (kv head, channel).  The sign
    convention of the offset is parity unpinned.
R24 per-token antiquant ([FIA] antiquantMode list: 1 per-token, 3 per-token
    with per-head; no shape is printed): fp32 parameters (2, B, S) with one
    (scale, offset) pair per logical token position j < S of sequence b,
    applied to every channel (and every KV head) of that token, or
    (2, B, KV_N, S) with one pair per token and KV head; the R2 form
    x_hat = (x + offset) * scale; index 0 is K, 1 is V.
R3  GQA: query head h reads KV head h // (N_q / N_kv) (contiguous groups).
    Parity unpinned as to convention.
R4  the sink is a logit in the units of the scaled score scale * q.k.
R5  lse = m + ln(den), natural log, over scaled logits, sink term included.
R6  an empty sequence gives out = 0 and lse = -inf without a sink (the
    neutral element of the merge); with a sink it gives out = 0, lse = sink.
R17 MLA: V is the first v_dim channels of the cached key row.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")


# ----------------------------------------------------------------------------
# conversions and storage access
# ----------------------------------------------------------------------------

def as_f64(x) -> np.ndarray:
    """Exact conversion of a stored tensor (fp32/fp16/bf16/int8/int32/int64,
    torch or NumPy) to a float64 NumPy array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor; bf16 has no NumPy type
        import torch

        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _as_int(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def gather_kv(cache, layout: str, b: int, g: int, length: int,
              block_table=None, block_size: int = 0, dim: Optional[int] = None) -> np.ndarray:
    """Rows of tokens j = 0 .. length-1 of batch b, KV head g, as float64.

    [IFA] "Constraints", page attention scenario: key/value sit in one
    contiguous block pool; token j of batch b lives in block
    blockTable[b][j // blockSize] at slot j % blockSize.  Layouts:
      "paged"    : (blocknum, KV_N, blocksize, D)   (the page's recommended one)
      "paged_bsh": (blocknum, blocksize, H), H = KV_N * D, held as the 4-D
                   (blocknum, blocksize, KV_N, D) with the same memory order
      "bnsd"     : (B, KV_N, S, D) padded contiguous
      "bsnd"     : (B, S, KV_N, D) padded contiguous ([IFA] "Parameters",
                   the BSND / BSH key and value layouts)
    Only the first ``dim`` channels are returned when ``dim`` is given.
    """
    j = np.arange(length, dtype=np.int64)
    if layout == "bnsd":
        rows = cache[b, g, :length]
    elif layout == "bsnd":
        rows = cache[b, :length, g]
    elif layout in ("paged", "paged_bsh"):
        bt = _as_int(block_table)
        blk = bt[b, j // block_size] if length else np.zeros(0, np.int64)
        slot = j % block_size
        if hasattr(cache, "detach"):
            import torch

            blk, slot = torch.from_numpy(blk), torch.from_numpy(slot)
        rows = cache[blk, g, slot] if layout == "paged" else cache[blk, slot, g]
    else:
        raise ValueError(f"unknown layout {layout!r}")
    rows = as_f64(rows)
    if dim is not None:
        rows = rows[:, :dim]
    return rows


def dequant(x: np.ndarray, scale_c, offset_c) -> np.ndarray:
    """[IFA] antiquantScale / antiquantOffset; reading R2: x_hat = (x +
    offset) * scale for every token row x.  Per-channel mode: scale_c and
    offset_c are vectors over the channels; per-tensor mode: scalars."""
    # NumPy broadcasting: a vector applies along the channel axis of every row
    return (x + np.asarray(offset_c, dtype=np.float64)) * np.asarray(scale_c, dtype=np.float64)


# ----------------------------------------------------------------------------
# attention over one query row
# ----------------------------------------------------------------------------

def softmax_weights(s: np.ndarray, sink: Optional[float] = None):
    """Softmax over the scaled scores s, with the optional learnable sink as one
    extra logit that takes weight but carries no value ([SINK] formula,
    m = max(sink, max S)).

    Returns (p, p_sink, m, den): p[j] = e^(s_j - m) / den, p_sink =
    e^(sink - m) / den, den = sum_j e^(s_j - m) + e^(sink - m).  With no terms
    at all (empty s, no sink) it returns den = 0 and m = -inf.
    """
    smax = float(np.max(s)) if s.size else NEG_INF
    m = max(smax, sink) if sink is not None else smax
    if m == NEG_INF:
        return np.zeros_like(s), 0.0, NEG_INF, 0.0
    w = np.exp(s - m)
    ws = math.exp(sink - m) if sink is not None else 0.0
    den = float(np.sum(w)) + ws
    return w / den, ws / den, m, den


def attention_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                  sink: Optional[float] = None) -> Tuple[np.ndarray, float]:
    """One query row: out = Softmax(scale * K q) V  ([IFA] Function formula),
    with the sink term in the denominator ([SINK]).  Returns (out, lse) with
    lse = m + ln(den) (R5); an empty row gives (0, -inf) or (0, sink) (R6)."""
    s = scale * (K @ q)
    p, _, m, den = softmax_weights(s, sink)
    if den == 0.0:
        return np.zeros(V.shape[1]), NEG_INF
    out = p @ V
    return out, m + math.log(den)


def partial_triple(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """The (attn_out, softmax_max, softmax_sum) triple of attention restricted
    to the given token rows, the quantities [RAU] merges: attn_out is the
    softmax-normalised output over these tokens, softmax_max = max_j s_j and
    softmax_sum = sum_j e^(s_j - softmax_max).  No tokens: (0, -inf, 0)."""
    s = scale * (K @ q)
    if s.size == 0:
        return np.zeros(V.shape[1]), NEG_INF, 0.0
    m = float(np.max(s))
    w = np.exp(s - m)
    l = float(np.sum(w))
    return (w @ V) / l, m, l


def merge(po, pm, ps, co, cm, cs):
    """[RAU] update of two partial results, weighted form (reading R1).

    Works elementwise on scalars or on rows: po/co are (..., D), pm/ps/cm/cs
    are (...).  A partial with max -inf has weight 0.
    """
    po, co = np.asarray(po, np.float64), np.asarray(co, np.float64)
    pm, ps = np.asarray(pm, np.float64), np.asarray(ps, np.float64)
    cm, cs = np.asarray(cm, np.float64), np.asarray(cs, np.float64)
    M = np.maximum(pm, cm)
    with np.errstate(invalid="ignore"):
        wp = np.where(pm == NEG_INF, 0.0, ps * np.exp(pm - M))
        wc = np.where(cm == NEG_INF, 0.0, cs * np.exp(cm - M))
    tot = wp + wc
    safe = np.where(tot > 0, tot, 1.0)
    out = (wp[..., None] * po + wc[..., None] * co) / safe[..., None]
    out = np.where((tot > 0)[..., None], out, 0.0)
    return out, M, tot


def merge_many(triples: Iterable):
    """Left fold of ``merge`` over (out, max, sum) triples, in the given order."""
    it = iter(triples)
    o, m, l = next(it)
    for (o2, m2, l2) in it:
        o, m, l = merge(o, m, l, o2, m2, l2)
    return o, m, l


def attn_update(prev_out, prev_max, prev_sum, cur_out, cur_max, cur_sum):
    """[RAU] over rows: (rows, D) outputs and (rows,) max/sum; returns the
    updated (attn_out, softmax_max, softmax_sum)."""
    return merge(as_f64(prev_out), as_f64(prev_max), as_f64(prev_sum),
                 as_f64(cur_out), as_f64(cur_max), as_f64(cur_sum))


# ----------------------------------------------------------------------------
# the whole decode call
# ----------------------------------------------------------------------------

def antiquant_mode_of(aq_scale, mode: Optional[str] = None) -> Optional[str]:
    """The antiquant mode of a parameter array: "tensor" for shape (2),
    "channel" for (2, KV_N, D), "token_head" for (2, B, KV_N, S); a 3-D array
    is per channel unless ``mode`` says "token" ((2, B, S))."""
    if aq_scale is None:
        return None
    if mode:
        return mode
    return {1: "tensor", 3: "channel", 4: "token_head"}[np.ndim(aq_scale)]


def _kv_rows(k_cache, v_cache, layout, b, g, L, block_table, block_size,
             qk_dim, v_dim, v_from_k, aq_scale, aq_offset, aq_mode=None):
    K = gather_kv(k_cache, layout, b, g, L, block_table, block_size, dim=qk_dim)
    if v_from_k:
        V = K[:, :v_dim]  # R17: V is the first v_dim channels of the key row
    else:
        V = gather_kv(v_cache, layout, b, g, L, block_table, block_size, dim=v_dim)
    mode = antiquant_mode_of(aq_scale, aq_mode)
    if mode == "tensor":  # shape (2): [K, V]
        K = dequant(K, aq_scale[0], aq_offset[0])
        V = dequant(V, aq_scale[1], aq_offset[1])
    elif mode == "channel":  # (2, KV_N, D)
        K = dequant(K, aq_scale[0, g, :qk_dim], aq_offset[0, g, :qk_dim])
        V = dequant(V, aq_scale[1, g, :v_dim], aq_offset[1, g, :v_dim])
    elif mode == "token":  # (2, B, S): one pair per logical token of sequence b, every channel and head
        K = dequant(K, aq_scale[0, b, :L, None], aq_offset[0, b, :L, None])
        V = dequant(V, aq_scale[1, b, :L, None], aq_offset[1, b, :L, None])
    elif mode == "token_head":  # (2, B, KV_N, S): one pair per logical token and KV head
        K = dequant(K, aq_scale[0, b, g, :L, None], aq_offset[0, b, g, :L, None])
        V = dequant(V, aq_scale[1, b, g, :L, None], aq_offset[1, b, g, :L, None])
    elif mode is not None:
        raise ValueError(f"unknown antiquant mode {mode!r}")
    return K, V


def decode_rows(q, k_cache, v_cache, layout: str, seq_lens, n_kv: int, scale: float,
                rows: Sequence[Tuple[int, int]], block_table=None, block_size: int = 0,
                sink=None, antiquant_scale=None, antiquant_offset=None,
                v_dim: Optional[int] = None, v_from_k: bool = False, antiquant_mode: Optional[str] = None):
    """Decode attention for the listed (batch, query head) rows only.

    q is (B, N_q, qk_dim); query head h reads KV head h // (N_q / N_kv)
    (reading R3; numKeyValueHeads = 0 means N_kv = N_q, [IFA] Parameters).
    Returns (out (len(rows), v_dim), lse (len(rows),)).
    """
    qf = as_f64(q)
    B, n_q, qk_dim = qf.shape
    n_kv = n_q if n_kv == 0 else n_kv
    if n_q % n_kv:
        raise ValueError("numHeads must be a multiple of numKeyValueHeads")
    G = n_q // n_kv
    v_dim = qk_dim if v_dim is None else v_dim
    lens = _as_int(seq_lens)
    sinkf = as_f64(sink)
    aq_s = as_f64(antiquant_scale)
    aq_o = as_f64(antiquant_offset)
    out = np.zeros((len(rows), v_dim))
    lse = np.zeros(len(rows))
    cache = {}
    for i, (b, h) in enumerate(rows):
        g = h // G
        if (b, g) not in cache:
            cache[(b, g)] = _kv_rows(k_cache, v_cache, layout, b, g, int(lens[b]), block_table,
                                     block_size, qk_dim, v_dim, v_from_k, aq_s, aq_o, antiquant_mode)
        K, V = cache[(b, g)]
        out[i], lse[i] = attention_row(qf[b, h], K, V, scale,
                                       None if sinkf is None else float(sinkf[h]))
    return out, lse


def decode(q, k_cache, v_cache, layout: str, seq_lens, n_kv: int, scale: float,
           block_table=None, block_size: int = 0, sink=None, antiquant_scale=None,
           antiquant_offset=None, v_dim: Optional[int] = None, v_from_k: bool = False,
           antiquant_mode: Optional[str] = None):
    """Decode attention for every (batch, query head): (out (B, N_q, v_dim),
    lse (B, N_q)).  Loops batch by batch and KV head by KV head."""
    qf = as_f64(q)
    B, n_q, qk_dim = qf.shape
    v_dim = qk_dim if v_dim is None else v_dim
    n_kv_e = n_q if n_kv == 0 else n_kv
    G = n_q // n_kv_e
    lens = _as_int(seq_lens)
    sinkf = as_f64(sink)
    aq_s = as_f64(antiquant_scale)
    aq_o = as_f64(antiquant_offset)
    out = np.zeros((B, n_q, v_dim))
    lse = np.zeros((B, n_q))
    for b in range(B):
        for g in range(n_kv_e):
            K, V = _kv_rows(k_cache, v_cache, layout, b, g, int(lens[b]), block_table, block_size,
                            qk_dim, v_dim, v_from_k, aq_s, aq_o, antiquant_mode)
            for h in range(g * G, (g + 1) * G):
                out[b, h], lse[b, h] = attention_row(qf[b, h], K, V, scale,
                                                     None if sinkf is None else float(sinkf[h]))
    return out, lse


def decode_workload(w, rows=None):
    """Convenience: run ``decode`` (or ``decode_rows``) on a synthetic workload
    object carrying the decode arguments as attributes."""
    kw = dict(block_table=w.block_table, block_size=w.block_size, sink=w.sink,
              antiquant_scale=w.antiquant_scale, antiquant_offset=w.antiquant_offset,
              v_dim=w.v_dim, v_from_k=w.v_aliases_k, antiquant_mode=getattr(w, "antiquant_mode", None))
    if rows is None:
        return decode(w.q, w.k_cache, w.v_cache, w.layout, w.seq_lens, w.n_kv, w.scale, **kw)
    return decode_rows(w.q, w.k_cache, w.v_cache, w.layout, w.seq_lens, w.n_kv, w.scale, rows, **kw)


# ----------------------------------------------------------------------------
# pool sizing
# ----------------------------------------------------------------------------

def lengths_from_prefix_sums(prefix: Sequence[int]) -> list:
    """[MLA] Constraints, BlockNum row: actualSeqLen given as prefix sums."""
    out, prev = [], 0
    for v in prefix:
        out.append(int(v) - prev)
        prev = int(v)
    return out


def block_count(lengths: Sequence[int], block_size: int) -> int:
    """[MLA] Constraints, BlockNum row: BlockNum >= sum_b ceil(S_b / BlockSize)."""
    return sum(-(-int(L) // int(block_size)) for L in lengths)

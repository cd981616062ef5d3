"""Pins for the float64 oracle: checks against what the pages and the
mathematics fix, never against the oracle's own formulas retyped.

Each test names the page passage it rests on.  Together they are chosen so
that a plausible slip anywhere in the oracle (dropped scale, wrong sign,
transposed operand, wrong head or block index, missing sum weight, sink on the
wrong side) fails at least one of them; ``test_planted_mistakes_are_caught``
plants such slips in copies of the oracle and checks exactly that.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attn_ref
from synth import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL = 1e-12


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _bruteforce_row(q, K, V, scale, sink=None):
    """Literal formula of the aclnnIncreFlashAttentionV3 "Function" section
    (and the sink denominator of aclnnFlashAttentionScoreV4): no max
    subtraction, pure-Python loops, math.fsum.  Tiny inputs only."""
    L, D = len(K), len(q)
    e = [math.exp(scale * math.fsum(q[d] * K[j][d] for d in range(D))) for j in range(L)]
    den = math.fsum(e) + (math.exp(sink) if sink is not None else 0.0)
    out = [math.fsum(e[j] * V[j][c] for j in range(L)) / den for c in range(len(V[0]))] if L else [0.0] * len(V[0])
    return out, math.log(den)


# ---------------------------------------------------------------- P1
def test_softmax_rows_sum_to_one():
    """aclnnIncreFlashAttentionV3 Function: each row is normalised by softmax;
    aclnnFlashAttentionScoreV4 formula: the sink weight is part of the sum."""
    rng = np.random.default_rng(1)
    for L in (1, 2, 17, 300):
        s = _rand(rng, L) * 5
        p, ps, m, den = oracle.softmax_weights(s)
        assert ps == 0.0 and abs(p.sum() - 1.0) < RTOL
        for sink in (-3.0, 0.0, 9.0):
            p, ps, m, den = oracle.softmax_weights(s, sink)
            assert abs(p.sum() + ps - 1.0) < RTOL
            assert m == max(s.max(), sink)
            assert np.all(p >= 0) and ps > 0


# ---------------------------------------------------------------- P2
@pytest.mark.parametrize("seed", range(6))
def test_split_invariance_merge_equals_full(seed):
    """aclnnRingAttentionUpdate formula (weighted reading R1): merging the
    partial results of any split of the KV axis, in any order, reproduces the
    attention over the whole axis."""
    rng = np.random.default_rng(100 + seed)
    L, D, Dv = int(rng.integers(1, 200)), 16, 12
    q, K, V = _rand(rng, D), _rand(rng, L, D), _rand(rng, L, Dv)
    scale = 1 / math.sqrt(D)
    full, lse = oracle.attention_row(q, K, V, scale)
    nparts = int(rng.integers(2, 17))
    cuts = np.sort(rng.integers(0, L + 1, size=nparts - 1))
    bounds = [0, *cuts.tolist(), L]
    parts = [oracle.partial_triple(q, K[a:b], V[a:b], scale) for a, b in zip(bounds[:-1], bounds[1:])]
    order = rng.permutation(len(parts))
    o, m, l = oracle.merge_many([parts[i] for i in order])
    np.testing.assert_allclose(o, full, rtol=0, atol=1e-12)
    assert abs((m + math.log(l)) - lse) < 1e-12


def test_split_invariance_two_halves_of_64():
    """The tiny fp32 workload is checked as the merge of its two 64-token halves."""
    rng = np.random.default_rng(7)
    D = 64
    q, K, V = _rand(rng, D), _rand(rng, 128, D), _rand(rng, 128, D)
    full, lse = oracle.attention_row(q, K, V, 1 / 8)
    a = oracle.partial_triple(q, K[:64], V[:64], 1 / 8)
    b = oracle.partial_triple(q, K[64:], V[64:], 1 / 8)
    o, m, l = oracle.merge(*a, *b)
    np.testing.assert_allclose(o, full, atol=1e-13)
    assert abs(m + math.log(l) - lse) < 1e-12


def test_merge_empty_partial_is_neutral():
    """An empty partial (max -inf, sum 0) leaves the other one unchanged, on
    either side; two empty partials stay empty (no NaN from -inf - -inf)."""
    rng = np.random.default_rng(3)
    o = _rand(rng, 8)
    for args in [(o, 1.5, 2.0, np.zeros(8), -np.inf, 0.0), (np.zeros(8), -np.inf, 0.0, o, 1.5, 2.0)]:
        r, m, l = oracle.merge(*args)
        np.testing.assert_array_equal(r, o)
        assert m == 1.5 and l == 2.0
    r, m, l = oracle.merge(np.zeros(8), -np.inf, 0.0, np.zeros(8), -np.inf, 0.0)
    assert np.all(r == 0) and m == -np.inf and l == 0.0


# ---------------------------------------------------------------- P3
def test_printed_update_formula_in_lse_form():
    """aclnnRingAttentionUpdate prints sum = ps e^(pm-M) + e^(cm-M) and
    out = po e^(pm-M)/sum + co e^(cm-M)/sum.  With the partials in
    log-sum-exp form (max = lse, sum = 1) the printed formula and the weighted
    reading agree exactly; with sums != 1 only the weighted reading matches
    full attention."""
    rng = np.random.default_rng(11)
    D = 8
    q, K, V = _rand(rng, D), _rand(rng, 40, D), _rand(rng, 40, D)
    full, lse = oracle.attention_row(q, K, V, 0.3)
    po, pm, ps = oracle.partial_triple(q, K[:15], V[:15], 0.3)
    co, cm, cs = oracle.partial_triple(q, K[15:], V[15:], 0.3)
    plse, clse = pm + math.log(ps), cm + math.log(cs)

    def printed(po, pm, ps, co, cm):
        M = max(pm, cm)
        s = ps * math.exp(pm - M) + math.exp(cm - M)
        return po * math.exp(pm - M) / s + co * math.exp(cm - M) / s, M, s

    o1, M1, s1 = printed(po, plse, 1.0, co, clse)
    o2, M2, s2 = oracle.merge(po, plse, 1.0, co, clse, 1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(o1, full, atol=1e-12)
    # (m, l) form gives the same merged output and the same lse
    o3, M3, s3 = oracle.merge(po, pm, ps, co, cm, cs)
    np.testing.assert_allclose(o3, full, atol=1e-12)
    assert abs(M3 + math.log(s3) - lse) < 1e-12
    # the printed formula applied literally to (m, l) triples is not attention
    o4, _, _ = printed(po, pm, ps, co, cm)
    assert np.max(np.abs(o4 - full)) > 1e-3


# ---------------------------------------------------------------- P4 / P13
@pytest.mark.parametrize("bs,lengths", [(16, [1, 15, 16, 17, 40]), (32, [0, 31, 32, 33, 100]), (128, [5, 127, 128, 129, 300])])
def test_paged_equals_contiguous(bs, lengths):
    """aclnnIncreFlashAttentionV3 Constraints, page attention scenario: the
    paged layout (blocknum, KV_N, blocksize, D) addressed through blockTable
    gives the same attention as the contiguous layout holding the same tokens;
    the block permutation is seeded and random; lengths straddle block
    boundaries (bs-1, bs, bs+1) and include 0."""
    B, Nq, Nkv, D = len(lengths), 4, 2, 8
    w = make_workload(batch=B, n_q=Nq, n_kv=Nkv, qk_dim=D, kv_dtype="f32", layout="paged",
                      block_size=bs, lengths=lengths, seed=5, sink=False, extra_blocks=3)
    smax = max(lengths) + 3
    kc = torch.full((B, Nkv, smax, D), float("nan"))
    vc = torch.full((B, Nkv, smax, D), float("nan"))
    bt = w.block_table.long()
    for b, L in enumerate(lengths):
        for j in range(L):
            kc[b, :, j] = w.k_cache[bt[b, j // bs], :, j % bs]
            vc[b, :, j] = w.v_cache[bt[b, j // bs], :, j % bs]
    o_p, l_p = oracle.decode_workload(w)
    o_c, l_c = oracle.decode(w.q, kc, vc, "bnsd", w.seq_lens, Nkv, w.scale)
    np.testing.assert_array_equal(o_p, o_c)
    np.testing.assert_array_equal(l_p, l_c)
    assert not np.isnan(o_p).any()
    # identity block table over a pool laid out in batch order
    nb = [(L + bs - 1) // bs for L in lengths]
    pool = sum(nb)
    kp = torch.zeros((pool, Nkv, bs, D))
    vp = torch.zeros((pool, Nkv, bs, D))
    tab = torch.full((B, max(nb) or 1), -1, dtype=torch.int32)
    off = 0
    for b, L in enumerate(lengths):
        for i in range(nb[b]):
            tab[b, i] = off + i
            n = min(bs, L - i * bs)
            kp[off + i, :, :n] = kc[b, :, i * bs:i * bs + n]
            vp[off + i, :, :n] = vc[b, :, i * bs:i * bs + n]
        off += nb[b]
    o_i, l_i = oracle.decode(w.q, kp, vp, "paged", w.seq_lens, Nkv, w.scale, block_table=tab, block_size=bs)
    np.testing.assert_array_equal(o_i, o_c)
    np.testing.assert_array_equal(l_i, l_c)


# ---------------------------------------------------------------- P5
@pytest.mark.parametrize("bs,lengths", [(16, [0, 1, 15, 16, 17, 40]), (32, [31, 32, 33, 100])])
def test_token_major_layouts_equal_logical_kv(bs, lengths):
    """aclnnIncreFlashAttentionV3 Constraints, page attention scenario (the
    KV cache layouts (blocknum, blocksize, H) and (blocknum, KV_N,
    blocksize, D)) and Parameters (BSND key/value): each token-major layout,
    filled here element by element from one logical K/V[b][g][j][d] (reading
    H = KV_N x D with head g in columns g D .. g D + D - 1), gives exactly
    the attention of that logical K/V taken row by row in brute force."""
    rng = np.random.default_rng(bs)
    B, Nq, Nkv, D = len(lengths), 4, 2, 4
    S = max(lengths) + 2
    Kl, Vl = _rand(rng, B, Nkv, S, D), _rand(rng, B, Nkv, S, D)
    q = _rand(rng, B, Nq, D)
    scale = 0.5
    # block pool (pool, bs, H) with a seeded permutation of blocks
    nb = [(L + bs - 1) // bs for L in lengths]
    pool = sum(nb) + 2
    perm = rng.permutation(pool)
    tab = np.full((B, max(max(nb), 1)), -1, dtype=np.int32)
    kp, vp = np.full((pool, bs, Nkv * D), np.nan), np.full((pool, bs, Nkv * D), np.nan)
    kc, vc = np.full((B, S, Nkv * D), np.nan), np.full((B, S, Nkv * D), np.nan)
    used = 0
    for b, L in enumerate(lengths):
        for i in range(nb[b]):
            tab[b, i] = perm[used]
            used += 1
        for j in range(L):
            for g in range(Nkv):
                for d in range(D):
                    kp[tab[b, j // bs], j % bs, g * D + d] = Kl[b, g, j, d]
                    vp[tab[b, j // bs], j % bs, g * D + d] = Vl[b, g, j, d]
                    kc[b, j, g * D + d] = Kl[b, g, j, d]
                    vc[b, j, g * D + d] = Vl[b, g, j, d]
    lens = np.array(lengths)
    o_p, l_p = oracle.decode(q, kp.reshape(pool, bs, Nkv, D), vp.reshape(pool, bs, Nkv, D), "paged_bsh", lens,
                             Nkv, scale, block_table=tab, block_size=bs)
    o_c, l_c = oracle.decode(q, kc.reshape(B, S, Nkv, D), vc.reshape(B, S, Nkv, D), "bsnd", lens, Nkv, scale)
    for b, L in enumerate(lengths):
        for h in range(Nq):
            g = h // (Nq // Nkv)
            for o, l in ((o_p, l_p), (o_c, l_c)):
                if L:
                    ref, ref_lse = _bruteforce_row(q[b, h], Kl[b, g, :L].tolist(), Vl[b, g, :L].tolist(), scale)
                    np.testing.assert_allclose(o[b, h], ref, rtol=0, atol=1e-12)
                    assert abs(l[b, h] - ref_lse) < 1e-12
                else:  # empty sequence: zero output, lse -inf
                    assert np.all(o[b, h] == 0) and l[b, h] == -np.inf


def test_per_tensor_antiquant_is_per_channel_with_constant_vectors():
    """aclnnIncreFlashAttentionV3 Constraints on antiquantScale and
    antiquantOffset: per-tensor mode has shape (2), entry 0 for K and entry 1
    for V, the per-channel mode (2, N, D) otherwise.  A per-tensor pair
    (s_K, o_K), (s_V, o_V) equals the per-channel parameters that repeat
    them over every head and channel, and with the V entries set to the
    identity it changes the output only through K (distinct K and V values,
    so a swapped index fails)."""
    w = make_workload(batch=2, n_q=4, n_kv=2, qk_dim=16, kv_dtype="i8", layout="paged",
                      block_size=32, lengths=[40, 70], seed=19, antiquant_mode="tensor")
    assert tuple(w.antiquant_scale.shape) == (2,)
    kw = dict(block_table=w.block_table, block_size=32)
    sc, off = w.antiquant_scale, w.antiquant_offset
    full_s = torch.empty((2, 2, 16)); full_o = torch.empty((2, 2, 16))
    for i in range(2):
        full_s[i] = float(sc[i]); full_o[i] = float(off[i])
    o_t, l_t = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale,
                             antiquant_scale=sc, antiquant_offset=off, **kw)
    o_c, l_c = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale,
                             antiquant_scale=full_s, antiquant_offset=full_o, **kw)
    np.testing.assert_allclose(o_t, o_c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_t, l_c, rtol=0, atol=1e-12)
    # V side identity: out is the attention of dequantised K over the raw V bytes
    sv = sc.clone(); sv[1] = 1.0
    ov = off.clone(); ov[1] = 0.0
    o_k, _ = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale,
                           antiquant_scale=sv, antiquant_offset=ov, **kw)
    np.testing.assert_allclose(o_t, float(sc[1]) * (o_k + float(off[1])), rtol=0, atol=1e-10)


def test_token_permutation_invariance():
    """Attention is a sum over KV tokens: permuting (K_j, V_j) jointly changes nothing."""
    rng = np.random.default_rng(21)
    q, K, V = _rand(rng, 16), _rand(rng, 77, 16), _rand(rng, 77, 10)
    o, l = oracle.attention_row(q, K, V, 0.25, sink=0.7)
    p = rng.permutation(77)
    o2, l2 = oracle.attention_row(q, K[p], V[p], 0.25, sink=0.7)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    assert abs(l2 - l) < 1e-12


# ---------------------------------------------------------------- P6
@pytest.mark.parametrize("sink", [-5.0, 0.0, 8.0, 30.0])
def test_sink_closed_form(sink):
    """aclnnFlashAttentionScoreV4 formula: the sink adds e^(sink-m) to the
    denominator only.  Hence out_sink = out / (1 + e^(sink - lse)),
    lse_sink = logaddexp(lse, sink), and it equals merging in a pseudo
    partial with out 0, max sink, sum 1."""
    rng = np.random.default_rng(31)
    q, K, V = _rand(rng, 16), _rand(rng, 50, 16), _rand(rng, 50, 16)
    o0, l0 = oracle.attention_row(q, K, V, 0.25)
    o1, l1 = oracle.attention_row(q, K, V, 0.25, sink=sink)
    np.testing.assert_allclose(o1, o0 / (1 + math.exp(sink - l0)), atol=1e-13, rtol=1e-12)
    assert abs(l1 - np.logaddexp(l0, sink)) < 1e-12
    part = oracle.partial_triple(q, K, V, 0.25)
    om, mm, lm = oracle.merge(*part, np.zeros(16), sink, 1.0)
    np.testing.assert_allclose(om, o1, atol=1e-13)
    assert abs(mm + math.log(lm) - l1) < 1e-12


def test_sink_to_minus_infinity_recovers_plain_attention():
    rng = np.random.default_rng(32)
    q, K, V = _rand(rng, 8), _rand(rng, 20, 8), _rand(rng, 20, 8)
    o0, l0 = oracle.attention_row(q, K, V, 0.5)
    for s in (-np.inf, -1e4):
        o1, l1 = oracle.attention_row(q, K, V, 0.5, sink=s)
        np.testing.assert_allclose(o1, o0, atol=1e-15)
        assert abs(l1 - l0) < 1e-12


# ---------------------------------------------------------------- P7
def test_ifa_v3_example_all_ones():
    """Golden: the aclnnIncreFlashAttentionV3 sample (all-ones inputs) gives 1.0."""
    g = json.load(open(os.path.join(GOLDEN, "ifa_v3_example_all_ones.json")))
    B, N, D, S = g["batch"], g["num_heads"], g["head_dim"], g["kv_len"]
    assert g["scale_value"] == 1 / math.sqrt(D)
    q = np.ones((B, N, D))
    k = np.ones((B, g["num_key_value_heads"], S, D))
    out, lse = oracle.decode(q, k, k.copy(), "bnsd", [S] * B, g["num_key_value_heads"], g["scale_value"])
    np.testing.assert_array_equal(out, np.full((B, N, D), g["expected_out"]))
    # every score equals scale * D, so lse = scale*D + ln S
    np.testing.assert_allclose(lse, g["scale_value"] * D + math.log(S), atol=1e-12)


def test_special_cases():
    """V constant -> output constant; K = 0 -> uniform weights (mean of V,
    lse = ln L); one token -> its own value row and lse = its score."""
    rng = np.random.default_rng(41)
    q = _rand(rng, 12)
    K = _rand(rng, 33, 12)
    o, _ = oracle.attention_row(q, K, np.full((33, 5), -2.5), 0.3)
    np.testing.assert_allclose(o, -2.5, atol=1e-14)
    V = _rand(rng, 33, 5)
    o, l = oracle.attention_row(q, np.zeros((33, 12)), V, 0.3)
    np.testing.assert_allclose(o, V.mean(0), atol=1e-14)
    assert abs(l - math.log(33)) < 1e-14
    o, l = oracle.attention_row(q, K[:1], V[:1], 0.3)
    np.testing.assert_allclose(o, V[0], atol=1e-15)
    assert abs(l - 0.3 * float(K[0] @ q)) < 1e-13


def test_empty_sequence():
    """FusedInferAttentionScore blog, empty-tensor semantics: empty KV gives
    an all-zero output; the lse of an empty row is -inf (reading R6), and
    with a sink the row is the sink alone (out 0, lse = sink)."""
    o, l = oracle.attention_row(np.ones(4), np.zeros((0, 4)), np.zeros((0, 3)), 0.5)
    assert np.all(o == 0) and l == -np.inf
    o, l = oracle.attention_row(np.ones(4), np.zeros((0, 4)), np.zeros((0, 3)), 0.5, sink=1.25)
    assert np.all(o == 0) and l == 1.25
    o, m, s = oracle.partial_triple(np.ones(4), np.zeros((0, 4)), np.zeros((0, 3)), 0.5)
    assert np.all(o == 0) and m == -np.inf and s == 0.0


# ---------------------------------------------------------------- P8
@pytest.mark.parametrize("seed", range(5))
def test_bruteforce_tiny(seed):
    """Whole decode vs a separate pure-Python evaluation of the literal
    formula (no max subtraction) on tiny shapes, with GQA, paging, sink."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 3))
    Nkv = int(rng.choice([1, 2]))
    Nq = Nkv * int(rng.choice([1, 2]))
    D = int(rng.choice([4, 8]))
    lengths = [int(x) for x in rng.integers(0, 17, size=B)]
    use_sink = bool(seed % 2)
    w = make_workload(batch=B, n_q=Nq, n_kv=Nkv, qk_dim=D, kv_dtype="f32", layout="paged",
                      block_size=16, lengths=lengths, seed=seed, sink=use_sink)
    out, lse = oracle.decode_workload(w)
    qf = w.q.double().numpy()
    bt = w.block_table.long().numpy()
    G = Nq // Nkv
    for b in range(B):
        L = lengths[b]
        for h in range(Nq):
            g = h // G
            K = [[float(w.k_cache[bt[b, j // 16], g, j % 16, d]) for d in range(D)] for j in range(L)]
            V = [[float(w.v_cache[bt[b, j // 16], g, j % 16, d]) for d in range(D)] for j in range(L)]
            sk = float(w.sink[h]) if use_sink else None
            if L == 0 and sk is None:
                assert np.all(out[b, h] == 0) and lse[b, h] == -np.inf
                continue
            ob, lb = _bruteforce_row(qf[b, h].tolist(), K, V if L else [[0.0] * D], w.scale, sk)
            np.testing.assert_allclose(out[b, h], ob, rtol=1e-12, atol=1e-14)
            assert abs(lse[b, h] - lb) < 1e-12


# ---------------------------------------------------------------- P9
def test_gqa_equals_mha_with_repeated_kv():
    """aclnnIncreFlashAttentionV3: numHeads is a multiple of
    numKeyValueHeads; with contiguous head groups (reading R3) GQA equals
    MHA over KV heads repeated G times.  numKeyValueHeads = 0 means N_kv = N_q."""
    rng = np.random.default_rng(61)
    B, Nkv, G, S, D = 2, 3, 4, 20, 8
    q = _rand(rng, B, Nkv * G, D)
    k = _rand(rng, B, Nkv, S, D)
    v = _rand(rng, B, Nkv, S, D)
    lens = [20, 13]
    o1, l1 = oracle.decode(q, k, v, "bnsd", lens, Nkv, 0.35)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o2, l2 = oracle.decode(q, kr, vr, "bnsd", lens, Nkv * G, 0.35)
    np.testing.assert_array_equal(o1, o2)
    o3, l3 = oracle.decode(q, kr, vr, "bnsd", lens, 0, 0.35)
    np.testing.assert_array_equal(o3, o2)
    np.testing.assert_array_equal(l3, l2)


# ---------------------------------------------------------------- P10
def test_int8_antiquant_identity_and_affine():
    """aclnnIncreFlashAttentionV3 antiquantScale/antiquantOffset (per channel,
    index 0 = K, 1 = V), reading R2 x_hat = (x + offset) * scale.  Pins:
    scale 1, offset 0 is attention over the integer values; the V offset and
    scale act affinely on the output; the K offset shifts every score of a
    head by one constant, so the output is unchanged and the lse moves."""
    w = make_workload(batch=2, n_q=4, n_kv=2, qk_dim=16, kv_dtype="i8", layout="paged",
                      block_size=32, lengths=[40, 70], seed=9)
    kw = dict(block_table=w.block_table, block_size=32)
    ones, zeros = torch.ones_like(w.antiquant_scale), torch.zeros_like(w.antiquant_offset)
    o_q, l_q = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale,
                             antiquant_scale=ones, antiquant_offset=zeros, **kw)
    o_f, l_f = oracle.decode(w.q, w.k_cache.float(), w.v_cache.float(), "paged", w.seq_lens, 2, w.scale, **kw)
    np.testing.assert_array_equal(o_q, o_f)
    np.testing.assert_array_equal(l_q, l_f)

    sc, off = w.antiquant_scale.double().numpy(), w.antiquant_offset.double().numpy()
    # V side only: out = sc_v * (out_int + off_v)
    s_v = ones.clone(); s_v[1] = w.antiquant_scale[1]
    o_v_off = zeros.clone(); o_v_off[1] = w.antiquant_offset[1]
    o_a, l_a = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale,
                             antiquant_scale=s_v, antiquant_offset=o_v_off, **kw)
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(o_a[:, h], sc[1, g] * (o_f[:, h] + off[1, g]), atol=1e-12)
    np.testing.assert_allclose(l_a, l_f, atol=1e-12)
    # K side: offset shifts the scores by scale * sum_d q_d sc_d off_d
    s_k = ones.clone(); s_k[0] = w.antiquant_scale[0]
    o_k0, l_k0 = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale,
                               antiquant_scale=s_k, antiquant_offset=zeros, **kw)
    o_k_off = zeros.clone(); o_k_off[0] = w.antiquant_offset[0]
    o_k1, l_k1 = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale,
                               antiquant_scale=s_k, antiquant_offset=o_k_off, **kw)
    np.testing.assert_allclose(o_k1, o_k0, atol=1e-12)
    qf = w.q.double().numpy()
    for b in range(2):
        for h in range(4):
            g = h // 2
            c = w.scale * float(np.sum(qf[b, h] * sc[0, g] * off[0, g]))
            assert abs(l_k1[b, h] - (l_k0[b, h] + c)) < 1e-10


# ---------------------------------------------------------------- P11
def test_mla_equals_mqa_with_value_prefix():
    """MLA decode (aclnnMlaPrologV3WeightNz shapes: 512 latent + 64 rope,
    Nkv = 1): one cache row serves as K (all 576 channels) and, through its
    first 512 channels, as V.  It equals MQA with a separate V cache holding
    those channels."""
    w = make_workload(batch=2, n_q=8, n_kv=1, qk_dim=576, v_dim=512, kv_dtype="bf16", layout="paged",
                      block_size=16, lengths=[20, 33], seed=4, scale=1 / math.sqrt(192), v_aliases_k=True)
    o1, l1 = oracle.decode_workload(w)
    vsep = w.k_cache[..., :512].clone()
    o2, l2 = oracle.decode(w.q, w.k_cache, vsep, "paged", w.seq_lens, 1, w.scale,
                           block_table=w.block_table, block_size=16, v_dim=512)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    assert o1.shape == (2, 8, 512)


# ---------------------------------------------------------------- P12
def test_blocknum_worked_example():
    """Golden: aclnnMlaPrologV3WeightNz Constraints, BlockNum row."""
    g = json.load(open(os.path.join(GOLDEN, "mla_blocknum_example.json")))
    lens = oracle.lengths_from_prefix_sums(g["actual_seq_len_prefix_sums"])
    assert lens == g["expected_lengths"]
    assert oracle.block_count(lens, g["block_size"]) == g["expected_block_num"]


# ---------------------------------------------------------------- P19
@pytest.mark.parametrize("layout,mode", [("paged", "token"), ("paged_bsh", "token"), ("bnsd", "token_head"),
                                         ("paged", "token_head")])
def test_per_token_antiquant_bruteforce(layout, mode):
    """Per-token antiquant (FusedInferAttentionScore blog, antiquantMode 1
    per-token and 3 per-token with per-head; reading R24: fp32 (2, B, S) or
    (2, B, N_kv, S), one (scale, offset) pair per logical token position,
    x_hat = (x + offset) * scale).  The whole decode against the literal
    formula evaluated in pure Python, each K and V element dequantised from
    its stored byte with the pair of its sequence, token (and head); the
    paged pool is a random block permutation, so the pair must follow the
    logical position, not the storage slot."""
    B, nq, nkv, d, bs = 2, 4, 2, 8, 4
    lengths = [11, 6]
    w = make_workload(batch=B, n_q=nq, n_kv=nkv, qk_dim=d, kv_dtype="i8", layout=layout, block_size=bs,
                      lengths=lengths, s_cap=12, seed=33, sink=True, antiquant_mode=mode, extra_blocks=1)
    assert w.antiquant_mode == mode
    out, lse = oracle.decode_workload(w)
    kc, vc = w.k_cache.double().numpy(), w.v_cache.double().numpy()
    bt = w.block_table.long().tolist() if w.block_table is not None else None
    sc, off = w.antiquant_scale.double().numpy(), w.antiquant_offset.double().numpy()
    qf = w.q.double().numpy()
    G = nq // nkv
    for b in range(B):
        L = lengths[b]
        for h in range(nq):
            g = h // G

            def pair(i, j):
                return (sc[i, b, j], off[i, b, j]) if mode == "token" else (sc[i, b, g, j], off[i, b, g, j])

            K = [[(float(_stored(kc, layout, bt, bs, b, g, j)[c]) + pair(0, j)[1]) * pair(0, j)[0] for c in range(d)]
                 for j in range(L)]
            V = [[(float(_stored(vc, layout, bt, bs, b, g, j)[c]) + pair(1, j)[1]) * pair(1, j)[0] for c in range(d)]
                 for j in range(L)]
            ob, lb = _bruteforce_row(qf[b, h].tolist(), K, V, w.scale, float(w.sink[h]))
            np.testing.assert_allclose(out[b, h], ob, rtol=1e-11, atol=1e-13)
            assert abs(lse[b, h] - lb) < 1e-11


def test_per_token_antiquant_special_cases():
    """Reading R24 reduces to the other modes where it must: a per-token pair
    constant over tokens and sequences is the per-tensor pair (aclnnIncre-
    FlashAttentionV3 "Constraints": per-tensor shape (2)); per-token-per-head
    pairs equal over heads are the per-token pairs; and K scales all equal
    to c with zero K offsets are a change of the softmax scale from scale to
    scale * c over the raw K bytes (aclnnIncreFlashAttentionV3 "Function",
    the scale multiplies every logit)."""
    w = make_workload(batch=2, n_q=4, n_kv=2, qk_dim=16, kv_dtype="i8", layout="paged", block_size=16,
                      lengths=[37, 20], seed=34, antiquant_mode="token")
    kw = dict(block_table=w.block_table, block_size=16)
    S = w.antiquant_scale.shape[2]
    ts, to = torch.tensor([0.031, 0.022]), torch.tensor([0.4, -0.7])
    tok_s = ts[:, None, None].expand(2, 2, S).contiguous()
    tok_o = to[:, None, None].expand(2, 2, S).contiguous()
    o1, l1 = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale, antiquant_scale=tok_s,
                           antiquant_offset=tok_o, antiquant_mode="token", **kw)
    o2, l2 = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale, antiquant_scale=ts,
                           antiquant_offset=to, **kw)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    # per token and head, equal over heads
    sth = w.antiquant_scale[:, :, None, :].expand(2, 2, 2, S).contiguous()
    oth = w.antiquant_offset[:, :, None, :].expand(2, 2, 2, S).contiguous()
    o3, l3 = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale, antiquant_scale=sth,
                           antiquant_offset=oth, **kw)
    o4, l4 = oracle.decode_workload(w)
    np.testing.assert_array_equal(o3, o4)
    np.testing.assert_array_equal(l3, l4)
    # K side: all scales c, offsets 0 -> softmax scale * c over the raw bytes; V side identity
    c = float(torch.tensor(0.037, dtype=torch.float32))  # the value the fp32 parameter holds
    ks = torch.ones_like(w.antiquant_scale); ks[0] = c
    ko = torch.zeros_like(w.antiquant_offset)
    o5, l5 = oracle.decode(w.q, w.k_cache, w.v_cache, "paged", w.seq_lens, 2, w.scale, antiquant_scale=ks,
                           antiquant_offset=ko, antiquant_mode="token", **kw)
    o6, l6 = oracle.decode(w.q, w.k_cache.double(), w.v_cache.double(), "paged", w.seq_lens, 2, w.scale * c, **kw)
    np.testing.assert_allclose(o5, o6, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l5, l6, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P18
_ROWS_CASES = [
    # (layout, kv dtype, N_q, N_kv passed, D, V dim, MLA value prefix, sink, antiquant mode)
    ("paged", "f32", 6, 2, 8, 8, False, False, "channel"),
    ("paged", "bf16", 6, 2, 8, 8, False, True, "channel"),
    ("bnsd", "f16", 4, 4, 8, 8, False, True, "channel"),
    ("bnsd", "f32", 4, 0, 4, 4, False, False, "channel"),
    ("paged", "i8", 8, 2, 8, 8, False, True, "channel"),
    ("paged_bsh", "i8", 6, 3, 8, 8, False, False, "tensor"),
    ("bsnd", "bf16", 6, 3, 8, 8, False, True, "channel"),
    ("paged", "bf16", 4, 1, 12, 8, True, False, "channel"),
    ("paged", "i8", 6, 2, 8, 8, False, True, "token"),
    ("bnsd", "i8", 6, 3, 8, 8, False, False, "token_head"),
]


def _stored(cache, layout, bt, bs, b, g, j):
    """Token j of sequence b, KV head g, read by its storage index alone
    (aclnnIncreFlashAttentionV3 "Constraints", page attention scenario)."""
    if layout == "paged":
        return cache[bt[b][j // bs], g, j % bs]
    if layout == "paged_bsh":
        return cache[bt[b][j // bs], j % bs, g]
    if layout == "bnsd":
        return cache[b, g, j]
    return cache[b, j, g]


@pytest.mark.parametrize("case", range(len(_ROWS_CASES)))
def test_decode_rows_matches_bruteforce(case):
    """decode_rows, the per-row entry used wherever only some rows are
    checked, against the literal formula evaluated in pure Python for every
    requested (b, h), in a shuffled order with repeats: GQA (query head h
    reads KV head h // (N_q / N_kv), reading R3), MHA, numKeyValueHeads = 0
    meaning N_kv = N_q (aclnnIncreFlashAttentionV3 "Parameters"), paged,
    token-major and contiguous layouts, a learnable sink
    (aclnnFlashAttentionScoreV4 formula), int8 with per-channel and
    per-tensor (x + offset) * scale (reading R2), and the MLA value prefix
    (V = the first v_dim channels of the key row).  It must also return
    exactly what decode returns for those rows."""
    layout, kv, nq, nkv, d, dv, mla, use_sink, aq = _ROWS_CASES[case]
    B, bs = 3, 4
    lengths = [9, 0, 6] if case % 2 else [5, 11, 1]
    w = make_workload(batch=B, n_q=nq, n_kv=nkv, qk_dim=d, v_dim=dv, kv_dtype=kv, layout=layout,
                      block_size=bs, lengths=lengths, s_cap=12, seed=90 + case, sink=use_sink,
                      antiquant_mode=aq, v_aliases_k=mla, extra_blocks=1)
    n_kv = nq if nkv == 0 else nkv
    G = nq // n_kv
    kc = w.k_cache.double().numpy()
    vc = kc if mla else w.v_cache.double().numpy()
    bt = w.block_table.long().tolist() if w.block_table is not None else None
    qf = w.q.double().numpy()
    sc = w.antiquant_scale.double().numpy() if w.antiquant_scale is not None else None
    off = w.antiquant_offset.double().numpy() if w.antiquant_offset is not None else None
    rng = np.random.default_rng(case)
    rows = [(b, h) for b in range(B) for h in range(nq)]
    rows = [rows[i] for i in rng.permutation(len(rows))] + rows[:3]
    out, lse = oracle.decode_rows(w.q, w.k_cache, w.v_cache, layout, w.seq_lens, nkv, w.scale, rows,
                                  block_table=w.block_table, block_size=w.block_size, sink=w.sink,
                                  antiquant_scale=w.antiquant_scale, antiquant_offset=w.antiquant_offset,
                                  v_dim=dv, v_from_k=mla, antiquant_mode=w.antiquant_mode)
    assert out.shape == (len(rows), dv) and lse.shape == (len(rows),)

    def deq(x, i, g, c, b, j):
        if sc is None:
            return float(x)
        if aq == "tensor":
            return (float(x) + off[i]) * sc[i]
        if aq == "token":
            return (float(x) + off[i, b, j]) * sc[i, b, j]
        if aq == "token_head":
            return (float(x) + off[i, b, g, j]) * sc[i, b, g, j]
        return (float(x) + off[i, g, c]) * sc[i, g, c]

    for r, (b, h) in enumerate(rows):
        g = h // G
        L = lengths[b]
        K = [[deq(_stored(kc, layout, bt, bs, b, g, j)[c], 0, g, c, b, j) for c in range(d)] for j in range(L)]
        V = [[deq(_stored(vc, layout, bt, bs, b, g, j)[c], 1, g, c, b, j) for c in range(dv)] for j in range(L)]
        sk = float(w.sink[h]) if use_sink else None
        if L == 0 and sk is None:
            assert np.all(out[r] == 0) and lse[r] == -np.inf
            continue
        ob, lb = _bruteforce_row(qf[b, h].tolist(), K, V if L else [[0.0] * dv], w.scale, sk)
        np.testing.assert_allclose(out[r], ob, rtol=1e-11, atol=1e-13)
        assert abs(lse[r] - lb) < 1e-11
    full_o, full_l = oracle.decode_workload(w)
    for r, (b, h) in enumerate(rows):
        np.testing.assert_array_equal(out[r], full_o[b, h])
        assert lse[r] == full_l[b, h] or (np.isinf(lse[r]) and np.isinf(full_l[b, h]))


# ---------------------------------------------------------------- attn_update rows
def test_attn_update_rows_match_full_attention():
    """Row-wise aclnnRingAttentionUpdate over several (b, h) rows: merging the
    two halves' triples reproduces full attention per row."""
    rng = np.random.default_rng(71)
    rows, D = 6, 32
    q = _rand(rng, rows, D)
    K, V = _rand(rng, rows, 50, D), _rand(rng, rows, 50, D)
    prev = [oracle.partial_triple(q[r], K[r, :20], V[r, :20], 0.2) for r in range(rows)]
    cur = [oracle.partial_triple(q[r], K[r, 20:], V[r, 20:], 0.2) for r in range(rows)]
    po = np.stack([p[0] for p in prev]); pm = np.array([p[1] for p in prev]); ps = np.array([p[2] for p in prev])
    co = np.stack([p[0] for p in cur]); cm = np.array([p[1] for p in cur]); cs = np.array([p[2] for p in cur])
    o, m, s = oracle.attn_update(po, pm, ps, co, cm, cs)
    for r in range(rows):
        full, lse = oracle.attention_row(q[r], K[r], V[r], 0.2)
        np.testing.assert_allclose(o[r], full, atol=1e-12)
        assert abs(m[r] + math.log(s[r]) - lse) < 1e-12


# ---------------------------------------------------------------- sensitivity
def test_planted_mistakes_are_caught(monkeypatch):
    """Plant plausible slips in the oracle (on the CPU) and check that the
    brute-force pin, the split pin or the GQA pin notices each one."""
    orig_row = attn_ref.attention_row
    orig_merge = attn_ref.merge
    orig_gather = attn_ref.gather_kv

    def run_pins():
        failed = []
        for name, fn in [("bruteforce", lambda: test_bruteforce_tiny(1)),
                         ("split", lambda: test_split_invariance_merge_equals_full(0)),
                         ("sink", lambda: test_sink_closed_form(8.0)),
                         ("paged", lambda: test_paged_equals_contiguous(16, [1, 15, 16, 17, 40])),
                         ("token-major", lambda: test_token_major_layouts_equal_logical_kv(16, [0, 1, 15, 16, 17, 40])),
                         ("per-tensor", test_per_tensor_antiquant_is_per_channel_with_constant_vectors),
                         ("rows", lambda: test_decode_rows_matches_bruteforce(0)),
                         ("rows-int8", lambda: test_decode_rows_matches_bruteforce(4)),
                         ("per-token", lambda: test_per_token_antiquant_bruteforce("paged", "token")),
                         ("per-token-head", lambda: test_per_token_antiquant_bruteforce("bnsd", "token_head"))]:
            try:
                fn()
            except (AssertionError, IndexError):  # a wrong index may also fall outside the cache
                failed.append(name)
        return failed

    def no_scale(q, K, V, scale, sink=None):
        return orig_row(q, K, V, 1.0, sink)

    def sink_in_numerator(q, K, V, scale, sink=None):
        o, l = orig_row(q, K, V, scale, None)
        return o, l if sink is None else np.logaddexp(l, sink)

    def transposed(q, K, V, scale, sink=None):
        return orig_row(q, K, V[::-1].copy(), scale, sink)

    def unweighted_merge(po, pm, ps, co, cm, cs):
        return orig_merge(po, pm, 1.0 + 0 * np.asarray(ps), co, cm, 1.0 + 0 * np.asarray(cs))

    def wrong_batch_row(cache, layout, b, g, length, block_table=None, block_size=0, dim=None):
        return orig_gather(cache, layout, 0 if layout == "paged" else b, g, length, block_table, block_size, dim)

    def wrong_head(cache, layout, b, g, length, block_table=None, block_size=0, dim=None):
        return orig_gather(cache, layout, b, (g + 1) % cache.shape[1], length, block_table, block_size, dim)

    def token_major_read_as_head_major(cache, layout, b, g, length, block_table=None, block_size=0, dim=None):
        if layout == "paged_bsh":  # the same memory taken as (blocknum, KV_N, blocksize, D)
            n, bs, nkv, d = cache.shape
            return orig_gather(cache.reshape(n, nkv, bs, d), "paged", b, g, length, block_table, block_size, dim)
        if layout == "bsnd":
            bb, sc, nkv, d = cache.shape
            return orig_gather(cache.reshape(bb, nkv, sc, d), "bnsd", b, g, length, block_table, block_size, dim)
        return orig_gather(cache, layout, b, g, length, block_table, block_size, dim)

    orig_kv_rows = attn_ref._kv_rows

    def per_tensor_k_v_swapped(k_cache, v_cache, layout, b, g, L, block_table, block_size, qk_dim, v_dim, v_from_k,
                               aq_scale, aq_offset, aq_mode=None):
        if aq_scale is not None and aq_scale.ndim == 1:
            aq_scale, aq_offset = aq_scale[::-1].copy(), aq_offset[::-1].copy()
        return orig_kv_rows(k_cache, v_cache, layout, b, g, L, block_table, block_size, qk_dim, v_dim, v_from_k,
                            aq_scale, aq_offset, aq_mode)

    def per_token_reversed(k_cache, v_cache, layout, b, g, L, block_table, block_size, qk_dim, v_dim, v_from_k,
                           aq_scale, aq_offset, aq_mode=None):
        # token parameters read from the end of the sequence's row backwards
        if aq_mode == "token":
            aq_scale, aq_offset = aq_scale.copy(), aq_offset.copy()
            aq_scale[:, b, :L] = aq_scale[:, b, :L][:, ::-1]
            aq_offset[:, b, :L] = aq_offset[:, b, :L][:, ::-1]
        return orig_kv_rows(k_cache, v_cache, layout, b, g, L, block_table, block_size, qk_dim, v_dim, v_from_k,
                            aq_scale, aq_offset, aq_mode)

    def per_token_first_sequence(k_cache, v_cache, layout, b, g, L, block_table, block_size, qk_dim, v_dim,
                                 v_from_k, aq_scale, aq_offset, aq_mode=None):
        # every sequence reads the token parameters of sequence 0
        if aq_mode in ("token", "token_head"):
            aq_scale, aq_offset = aq_scale.copy(), aq_offset.copy()
            aq_scale[:, b], aq_offset[:, b] = aq_scale[:, 0], aq_offset[:, 0]
        return orig_kv_rows(k_cache, v_cache, layout, b, g, L, block_table, block_size, qk_dim, v_dim, v_from_k,
                            aq_scale, aq_offset, aq_mode)

    def rows_wrong_group(q, k_cache, v_cache, layout, seq_lens, n_kv, scale, rows, block_table=None,
                         block_size=0, sink=None, antiquant_scale=None, antiquant_offset=None, v_dim=None,
                         v_from_k=False, antiquant_mode=None):
        # decode_rows with query head h sent to KV head h % N_kv (interleaved
        # instead of contiguous groups), everything else as in the oracle
        qf = attn_ref.as_f64(q)
        n_q, qk_dim = qf.shape[1], qf.shape[2]
        n_kv = n_q if n_kv == 0 else n_kv
        v_dim = qk_dim if v_dim is None else v_dim
        lens = attn_ref._as_int(seq_lens)
        sinkf = attn_ref.as_f64(sink)
        aq_s, aq_o = attn_ref.as_f64(antiquant_scale), attn_ref.as_f64(antiquant_offset)
        out, lse = np.zeros((len(rows), v_dim)), np.zeros(len(rows))
        for i, (b, h) in enumerate(rows):
            K, V = attn_ref._kv_rows(k_cache, v_cache, layout, b, h % n_kv, int(lens[b]), block_table, block_size,
                                     qk_dim, v_dim, v_from_k, aq_s, aq_o, antiquant_mode)
            out[i], lse[i] = attn_ref.attention_row(qf[b, h], K, V, scale, None if sinkf is None else float(sinkf[h]))
        return out, lse

    slips = [("decode_rows", rows_wrong_group), ("attention_row", no_scale), ("attention_row", sink_in_numerator),
             ("attention_row", transposed), ("merge", unweighted_merge),
             ("gather_kv", wrong_batch_row), ("gather_kv", wrong_head),
             ("gather_kv", token_major_read_as_head_major), ("_kv_rows", per_tensor_k_v_swapped),
             ("_kv_rows", per_token_reversed), ("_kv_rows", per_token_first_sequence)]
    for fn_name, bad in slips:
        with monkeypatch.context() as mp:
            mp.setattr(attn_ref, fn_name, bad)
            if hasattr(oracle, fn_name):
                mp.setattr(oracle, fn_name, bad)
            assert run_pins(), f"planted slip {bad.__name__} went unnoticed"
    assert run_pins() == []

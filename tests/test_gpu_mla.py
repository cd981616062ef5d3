"""GPU parity of the MLA-shaped decode (MFMA path) against the float64 oracle.

The shape of the MlaProlog pages (aclnnMlaPrologV3WeightNz): all query heads
share one cached row of 576 channels per token (512 latent + 64 rope) and V is
the first 512 channels of that row.  Tolerances as for every bf16 input:
max-abs 1e-2 beyond half an output ulp, |lse| within 1e-3.  P is rounded to
bf16 before the PV product (weights up to 2^8 relative to the running
reference), which stays far inside that bound for unit-variance V.
"""

import math

import numpy as np
import pytest
import torch

import attention_ifa_decode_amd as ifa
import oracle
from synth import config_workload, make_workload

from test_gpu_decode import _announce, _compare, _full_check, _gpu, _sampled_rows, whole_sequence_rows

pytestmark = pytest.mark.gpu


def _mla(**kw):
    base = dict(batch=2, n_q=128, n_kv=1, qk_dim=576, v_dim=512, kv_dtype="bf16", layout="paged",
                block_size=128, lengths=[300, 77], scale=1.0 / math.sqrt(192.0), v_aliases_k=True, seed=50)
    base.update(kw)
    return make_workload(**base)


@pytest.mark.parametrize("seed", [500, 501])
def test_c5_mla_reduced(seed):
    """The MLA config with a few sequences of ragged length (tile tails, a
    one-token sequence) and the automatic split count."""
    w = config_workload(5, seed=seed, batch=3, lengths=[1100, 40, 1], max_blocks_per_seq=9)
    _full_check(w)


@pytest.mark.parametrize("n_q", [32, 64, 96, 256])
def test_mla_head_counts(n_q):
    """1, 2 and 4 waves per workgroup, and two head groups per sequence."""
    _full_check(_mla(n_q=n_q, seed=51 + n_q), 2)


@pytest.mark.parametrize("splits", [1, 3, 16, 40])
def test_mla_split_counts(splits):
    _full_check(_mla(lengths=[700, 33, 129], batch=3, seed=52), splits)


@pytest.mark.parametrize("batch", [130, 257])
def test_mla_longest_first_batch_sizes(batch):
    """Longest-first ranking over three chunks of 64 sequences with many
    equal lengths, and a batch beyond its 256 limit (index order)."""
    lens = [int(x) for x in np.random.default_rng(batch).choice([0, 1, 33, 70], size=batch)]
    _full_check(_mla(n_q=32, batch=batch, lengths=lens, seed=batch), 2)


@pytest.mark.parametrize("bs", [16, 64, 256])
def test_mla_block_sizes(bs):
    """Tiles of 32 tokens that straddle cache blocks (block size 16) and
    blocks longer than a tile."""
    _full_check(_mla(block_size=bs, lengths=[bs * 3 + 5, bs - 1], seed=53), 3)


def test_mla_contiguous_layout():
    _full_check(_mla(layout="bnsd", lengths=[200, 129], s_cap=256, seed=54), 2)


@pytest.mark.parametrize("length", [0, 1, 7, 128])
def test_mla_sink(length):
    w = _mla(lengths=[length, max(1, length)], sink=True, seed=55)
    w.sink = torch.full_like(w.sink, 3.0)
    _full_check(w, 2)


def test_mla_rescale_path():
    """Scores that jump upward late in each split force the running reference
    to move (the lazy rescale of the accumulators).  Only the 64 rope channels
    of the later rows are scaled, so V (the first 512 channels) keeps unit
    variance, the setting the tolerance is stated for."""
    w = _mla(lengths=[640, 333], seed=56)
    bt = w.block_table
    for b, L in enumerate(w.lengths()):
        for j in range(L // 2, L):
            blk = int(bt[b, j // w.block_size])
            w.k_cache[blk, :, j % w.block_size, 512:] *= 6
    _full_check(w, 2)


def test_mla_partials_match_oracle_triples():
    """ifa_decode_splitkv leaves, per (b, h, split), the triple of the split's
    token span [i*c, min(L, (i+1)*c)), c = 16*ceil(ceil(L/n)/16)."""
    w = _mla(lengths=[250, 33], seed=57)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg, num_splits=3)
    call.splitkv()
    torch.cuda.synchronize()
    po, pm, ps = (x.double().cpu().numpy() for x in call.partials())
    n = call.num_splits
    qf = w.q.double().numpy()
    for b, L in enumerate(w.lengths()):
        c = 16 * math.ceil(math.ceil(L / n) / 16)
        K = oracle.gather_kv(w.k_cache, "paged", b, 0, L, w.block_table, w.block_size)
        V = K[:, :512]
        for h in range(0, 128, 7):
            for i in range(n):
                a, e = i * c, min(L, (i + 1) * c)
                if a >= e:
                    continue
                o, m, s = oracle.partial_triple(qf[b, h], K[a:e], V[a:e], w.scale)
                assert np.max(np.abs(po[b, h, i] - o)) < 1e-2
                assert abs(pm[b, h, i] - m) < 1e-3 * max(1, abs(m))
                assert abs(ps[b, h, i] - s) < 1e-2 * s


def test_c5_full_size_sampled_rows():
    """The MLA config at its full size, in the launch configuration the
    benchmark times (balanced split: the longest sequence spans about eight
    runs); the oracle recomputes all 128 heads of the longest, the shortest
    and a median sequence, and a few random rows."""
    wg = config_workload(5, device="cuda")
    _announce(f"full size config 5: {wg.name}")
    out, lse = ifa.decode_workload(wg)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    assert not np.isnan(out).any()
    w = wg.to("cpu")
    del wg
    torch.cuda.empty_cache()
    rows = whole_sequence_rows(w, 5)
    ref_out, ref_lse = oracle.decode_workload(w, rows=rows)
    _compare(w, out, lse, ref_out, ref_lse, rows=rows)


def test_mla_wide_offsets_path():
    """A pool that the call declares larger than 4 GiB takes the 64-bit
    addressing path; every block-table entry still points into the real
    (small) pool, so the result must not change."""
    w = _mla(lengths=[260, 97], seed=58)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg, num_splits=2)
    call.args.num_blocks = 1 << 22  # 4M blocks x 128 rows x 1152 bytes > 4 GiB
    out, lse = call.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_workload(w)
    _compare(w, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse)


def test_mla_token_major_pool():
    """With one KV head the (blocknum, blocksize, H) pool holds the same bytes
    as the head-major one."""
    _full_check(_mla(layout="paged_bsh", lengths=[300, 77], seed=58), 3)


PIECE_COST = 7  # units a sequence weighs for the start of a piece on it


def _balanced_runs(lengths, n):
    """Host model of the balanced split: per sequence, its first unit (its
    first tile's unit is PIECE_COST later), and the runs
    [floor(r V / R), floor((r + 1) V / R)) of the batch's units."""
    cost = [(L + 31) // 32 + PIECE_COST if L > 0 else 0 for L in lengths]
    pref = np.concatenate([[0], np.cumsum(cost)]).astype(np.int64)
    V = int(pref[-1])
    R = min(n, V)
    bounds = [(r * V // R, (r + 1) * V // R) for r in range(R)]
    return pref, bounds


@pytest.mark.parametrize("n_q,lengths", [(128, [20000, 33, 0, 1, 9000, 700]), (256, [1, 0, 4100, 31, 32, 65])])
def test_mla_balanced_partials_match_oracle_triples(n_q, lengths):
    """The balanced split: every run is a workgroup of consecutive units of
    the whole batch (a sequence's tiles, after PIECE_COST units for its
    start); run r's piece of sequence b is slot r + b, and (first slot,
    count) per sequence names them.  Each piece's triple is the oracle's
    over exactly its tokens."""
    w = _mla(n_q=n_q, batch=len(lengths), lengths=lengths, seed=59)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg)
    assert call.balanced
    call.splitkv()
    torch.cuda.synchronize()
    po, pm, ps, desc = call.partial_slots()  # attn_out partials in fp16 on the MLA shape
    assert po.dtype == torch.float16
    po, pm, ps, desc = po.double().cpu().numpy(), pm.double().cpu().numpy(), ps.double().cpu().numpy(), desc.cpu().numpy()
    pref, bounds = _balanced_runs(lengths, call.num_splits)
    qf = w.q.double().numpy()
    checked = 0
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        z = pref[b] + PIECE_COST  # unit of the sequence's first tile
        runs = [r for r, (t0, t1) in enumerate(bounds) if t0 < pref[b + 1] and t1 > z]
        assert tuple(desc[b]) == (runs[0] + b, len(runs)), (b, desc[b], runs[0], len(runs))
        K = oracle.gather_kv(w.k_cache, "paged", b, 0, L, w.block_table, w.block_size)
        for r in runs:
            t0, t1 = bounds[r]
            a = (max(t0, z) - z) * 32
            e = min(L, (min(t1, pref[b + 1]) - z) * 32)
            for h in range(r % 5, n_q, 9):
                o, m, s = oracle.partial_triple(qf[b, h], K[a:e], K[a:e, :512], w.scale)
                slot = r + b
                assert np.max(np.abs(po[slot, h] - o)) < 1e-2, (b, r, h)
                assert abs(pm[slot, h] - m) < 1e-3 * max(1, abs(m)), (b, r, h)
                assert abs(ps[slot, h] - s) < 1e-2 * s, (b, r, h)
                checked += 1
    assert checked > 100


@pytest.mark.parametrize("n_q,bs,layout", [(128, 16, "paged"), (64, 128, "paged"), (256, 64, "paged_bsh"),
                                           (128, 128, "bnsd")])
def test_mla_balanced_decode(n_q, bs, layout):
    """The automatic (balanced) split end to end: runs that cover several
    short sequences, empty sequences, head groups, two waves per workgroup,
    small cache blocks and the contiguous layout."""
    lens = [3000, 0, 1, 31, 33, 700, 0, 1500]
    w = _mla(n_q=n_q, batch=len(lens), lengths=lens, block_size=bs, layout=layout, seed=60 + n_q + bs)
    _full_check(w)


def test_mla_balanced_wide_offsets_path():
    """The balanced split on the 64-bit addressing path."""
    w = _mla(lengths=[2600, 97, 1], batch=3, seed=61)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg)
    assert call.balanced
    call.args.num_blocks = 1 << 22
    out, lse = call.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_workload(w)
    _compare(w, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse)


def test_mla_balanced_batch_limit():
    """The balanced split at its batch limit (256 sequences): many empty and
    one-token sequences, so that runs hold many pieces and many sequences
    start inside a run; a few long ones span several runs."""
    rng = np.random.default_rng(62)
    lens = [int(x) for x in rng.choice([0, 1, 33, 70], size=256)]
    for i in (3, 100, 201):
        lens[i] = 4000 + 37 * i
    w = _mla(n_q=32, batch=256, lengths=lens, seed=62)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg)
    assert call.balanced
    _full_check(w)


def test_mla_large_values_within_fp16_partials():
    """Partial outputs are fp16 on the MLA shape: a normalised partial is a
    convex combination of V rows, so V up to 6e4 in magnitude passes through
    them.  Cache rows scaled by 1e4 (then clipped to 6e4): the output matches
    the oracle to the bf16 output's relative precision, with no inf."""
    w = _mla(lengths=[700, 90], seed=61)
    w.k_cache.copy_((w.k_cache.float() * 1e4).clamp(-6e4, 6e4).to(torch.bfloat16))  # in place: V aliases K
    _announce(f"mla large values {w.name} lens={w.lengths()}")
    out, lse = _gpu(w)
    ref_out, ref_lse = oracle.decode_workload(w)
    assert np.isfinite(out).all()
    scale = float(np.max(np.abs(ref_out)))
    assert scale > 1e3
    err = float(np.max(np.abs(out - ref_out)))
    print(f"[parity] large values: max-abs {err:.3e} of max |oracle| {scale:.3e}", flush=True)
    assert err <= 5e-3 * scale
    assert float(np.max(np.abs(lse - ref_lse))) <= 1e-3 * max(1.0, float(np.max(np.abs(ref_lse))))


def test_mla_values_beyond_fp16_overflow_visibly():
    """Beyond 65504 an fp16 partial overflows: one V channel held at 7e4 in
    every cached row (the same shift of every score, so the weights do not
    change) comes out inf for every row, and the other channels and lse stay
    those of the oracle.  The limit shows in the output rather than as a
    finite error."""
    w = _mla(lengths=[300, 41], seed=62)
    c = 17
    w.k_cache[..., c] = 7e4
    _announce(f"mla fp16 overflow {w.name} lens={w.lengths()}")
    out, lse = _gpu(w)
    ref_out, ref_lse = oracle.decode_workload(w)
    assert np.isinf(out[..., c]).all()
    keep = np.ones(out.shape[-1], dtype=bool)
    keep[c] = False
    err = float(np.max(np.abs(out[..., keep] - ref_out[..., keep])))
    assert err <= 1e-2, err
    assert float(np.max(np.abs(lse - ref_lse))) <= 1e-3 * max(1.0, float(np.max(np.abs(ref_lse))))

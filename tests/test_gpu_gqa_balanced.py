"""GPU parity of the balanced split of the GQA shapes on the matrix cores
(head dim 128, 16-bit or int8 K/V), the automatic choice for batch <= 256.

The batch's 32-token tiles, sequence after sequence, each sequence weighing
PIECE_COST more units for the start of a piece on it, are cut into equal runs;
run r's piece of sequence b is partial slot r + b, and the combine merges a
sequence's slots with the RingAttentionUpdate rule (aclnnRingAttentionUpdate,
"功能说明").  Each piece's triple is checked against the oracle's triple over
exactly its tokens, and whole decodes against the oracle's attention, with the
tolerances of the other GPU tests.
"""

import numpy as np
import pytest
import torch

import attention_ifa_decode_amd as ifa
import oracle
from synth import make_workload

from test_gpu_decode import _announce, _compare, _full_check
from test_gpu_spec import _check as _check_multi, _query, _tree

pytestmark = pytest.mark.gpu

PIECE_COST = 8  # units a sequence weighs for the start of a piece on it


def _balanced_runs(lengths, n):
    """Host model of the balanced split: the prefix of the sequences' units
    (first unit of sequence b = pref[b]; its first tile's unit is PIECE_COST
    later) and the runs [floor(r V / R), floor((r + 1) V / R)), R = min(n, V)."""
    cost = [(L + 31) // 32 + PIECE_COST if L > 0 else 0 for L in lengths]
    pref = np.concatenate([[0], np.cumsum(cost)]).astype(np.int64)
    V = int(pref[-1])
    R = min(n, V)
    return pref, [(r * V // R, (r + 1) * V // R) for r in range(R)]


@pytest.mark.parametrize("kv,layout,bs", [("bf16", "paged", 16), ("f16", "bnsd", 0), ("bf16", "paged_bsh", 64)])
def test_gqa_balanced_partials_match_oracle_triples(kv, layout, bs):
    """Slots, (first slot, count) pairs and every piece's triple: runs that
    end one sequence and start the next, whole short sequences inside a run,
    an empty sequence, a one-token one."""
    lengths = [2000, 33, 0, 1, 900, 64, 1500]
    kw = dict(block_size=bs) if bs else dict(s_cap=2048)
    w = make_workload(batch=len(lengths), n_q=8, n_kv=2, qk_dim=128, kv_dtype=kv, layout=layout,
                      lengths=lengths, seed=700 + bs, **kw)
    _announce(f"gqa balanced triples kv={kv} layout={layout} bs={bs}")
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg)
    assert call.balanced
    call.splitkv()
    torch.cuda.synchronize()
    po, pm, ps, desc = (x.cpu().numpy() for x in call.partial_slots())
    po, pm, ps = po.astype(np.float64), pm.astype(np.float64), ps.astype(np.float64)
    pref, bounds = _balanced_runs(lengths, call.num_splits)
    assert len(bounds) > len(lengths)  # several runs per long sequence
    tol_o = 1e-2 if kv == "bf16" else 1e-3
    qf = w.q.double().numpy()
    checked = 0
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        z = pref[b] + PIECE_COST  # unit of the sequence's first tile
        runs = [r for r, (t0, t1) in enumerate(bounds) if t0 < pref[b + 1] and t1 > z]
        assert tuple(desc[b]) == (runs[0] + b, len(runs)), (b, desc[b], runs[0], len(runs))
        for g in range(2):
            K = oracle.gather_kv(w.k_cache, layout, b, g, L, w.block_table, w.block_size)
            V = oracle.gather_kv(w.v_cache, layout, b, g, L, w.block_table, w.block_size)
            for r in runs:
                t0, t1 = bounds[r]
                a = (max(t0, z) - z) * 32
                e = min(L, (min(t1, pref[b + 1]) - z) * 32)
                assert a < e
                for h in range(4 * g, 4 * g + 4):
                    o, m, s = oracle.partial_triple(qf[b, h], K[a:e], V[a:e], w.scale)
                    slot = r + b
                    assert np.max(np.abs(po[slot, h] - o)) < tol_o, (b, r, h)
                    assert abs(pm[slot, h] - m) < 1e-4 * max(1, abs(m)), (b, r, h)
                    assert abs(ps[slot, h] - s) < 1e-4 * s, (b, r, h)
                    checked += 1
    assert checked > 100


@pytest.mark.parametrize("kv,layout,n_q,n_kv,sink", [
    ("bf16", "paged", 32, 8, False), ("f16", "bnsd", 16, 2, True), ("bf16", "bsnd", 8, 8, False),
    ("f16", "paged_bsh", 64, 4, False), ("i8", "paged", 64, 8, True), ("i8", "bnsd", 16, 2, False)])
def test_gqa_balanced_decode(kv, layout, n_q, n_kv, sink):
    """The automatic (balanced) split end to end, over the layouts, group
    sizes of 1 to 16 query rows per KV head, int8 with its per-channel
    antiquant, and the sink."""
    lens = [3000, 0, 1, 31, 33, 700, 0, 1500, 96]
    kw = dict(block_size=32) if layout.startswith("paged") else dict(s_cap=3072)
    w = make_workload(batch=len(lens), n_q=n_q, n_kv=n_kv, qk_dim=128, kv_dtype=kv, layout=layout, lengths=lens,
                      seed=710 + n_q, sink=sink, **kw)
    assert ifa.call_for_workload(w.to("cuda")).balanced
    _full_check(w)


@pytest.mark.parametrize("aq", ["token", "token_head", "tensor"])
def test_gqa_balanced_int8_antiquant_modes(aq):
    lens = [2100, 5, 0, 640, 77]
    w = make_workload(batch=len(lens), n_q=32, n_kv=4, qk_dim=128, kv_dtype="i8", layout="paged", block_size=64,
                      lengths=lens, seed=720, sink=True, antiquant_mode=aq)
    assert ifa.call_for_workload(w.to("cuda")).balanced
    _full_check(w)


def test_gqa_balanced_batch_limit():
    """256 sequences, mostly empty or a few tokens long, so that runs hold many
    pieces and many sequences start inside a run; a few long ones span
    several runs."""
    rng = np.random.default_rng(730)
    lens = [int(x) for x in rng.choice([0, 1, 33, 70], size=256)]
    for i in (3, 100, 201):
        lens[i] = 4000 + 37 * i
    w = make_workload(batch=256, n_q=16, n_kv=4, qk_dim=128, kv_dtype="bf16", layout="paged", block_size=64,
                      lengths=lens, seed=730)
    assert ifa.call_for_workload(w.to("cuda")).balanced
    _full_check(w)


def test_gqa_balanced_all_empty():
    """No tokens at all: no run has work; every row gets out 0 and lse -inf
    (the sink's value with a sink)."""
    w = make_workload(batch=4, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", layout="paged", block_size=32,
                      lengths=[0, 0, 0, 0], seed=740, sink=True, extra_blocks=1)
    assert ifa.call_for_workload(w.to("cuda")).balanced
    _full_check(w)


@pytest.mark.parametrize("mode", ["none", "causal", "tree"])
@pytest.mark.parametrize("kv", ["f16", "bf16", "i8"])
def test_gqa_balanced_multi_token(mode, kv):
    """S_q 4 x group 4 = 16 query rows per KV head through the balanced
    split: slots hold S_q * N_q rows, the masks follow each piece's
    sequence."""
    q_seq, lens = 4, [1, 4, 5, 17, 1300, 333, 0, 2500]
    w = make_workload(batch=len(lens), n_q=8, n_kv=2, qk_dim=128, kv_dtype=kv, layout="paged", block_size=32,
                      lengths=lens, seed=750, sink=(kv == "i8"), extra_blocks=1)
    q = _query(len(lens), q_seq, 8, 128, w.q.dtype, 751)
    _check_multi(w, q, mode, _tree(len(lens), q_seq, 752) if mode == "tree" else None, 0)


def test_gqa_balanced_multi_token_two_row_groups():
    """S_q 8 x group 8 = 64 rows per KV head: two 32-column row groups per run."""
    q_seq, lens = 8, [8, 40, 2000, 700]
    w = make_workload(batch=len(lens), n_q=16, n_kv=2, qk_dim=128, kv_dtype="bf16", layout="paged",
                      block_size=64, lengths=lens, seed=760)
    q = _query(len(lens), q_seq, 16, 128, torch.bfloat16, 761)
    _check_multi(w, q, "causal", None, 0)


def test_gqa_balanced_stale_workspace():
    """A workspace full of stale values from another call: the combine reads
    only the slots the (first slot, count) pairs name."""
    lens = [1200, 3, 0, 800]
    w = make_workload(batch=len(lens), n_q=8, n_kv=2, qk_dim=128, kv_dtype="f16", layout="paged", block_size=16,
                      lengths=lens, seed=770)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg)
    assert call.balanced
    call.workspace.fill_(0x7F)  # large finite fp32 values everywhere
    out, lse = call.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_workload(w)
    _compare(w, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse)

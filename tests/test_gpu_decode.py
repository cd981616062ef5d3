"""GPU parity: the HIP decode path (through the C ABI) against the float64
oracle on the same seeded inputs.

Tolerances (max-abs over every output element, against the unrounded oracle):
1e-5 for fp32 inputs, 1e-2 for fp16 / bf16 / int8-KV inputs; |lse| within
1e-3.  The output is stored in its dtype with round-to-nearest-even, which by
itself moves a value by up to half an ulp of that dtype (1/64 for bf16 values
in [4, 8)), so each element may differ from the unrounded oracle by the
tolerance plus half an output ulp at its magnitude; where the oracle's
magnitude is below 2 the plain bound is asserted as well.  An empty row must give out == 0 and lse == -inf exactly (or lse ==
sink with a sink).  Stored KV slots that must never be read are NaN-poisoned
(127 for int8), and unused block-table entries are -1.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import attention_ifa_decode_amd as ifa
import oracle
from synth import config_workload, make_workload

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_LOWP = 1e-2
TOL_LSE = 1e-3


def _announce(msg):
    print(f"[gpu case] {msg}", flush=True)


def _gpu(w, num_splits=None):
    wg = w.to("cuda")
    out, lse = ifa.decode_workload(wg, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


_MANT_BITS = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


def half_ulp(x, dtype):
    """Half the spacing of ``dtype`` at magnitude |x| (normal range; the
    subnormal spacing below it)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float64).tiny)
    e = np.floor(np.log2(ax))
    emin = {torch.float32: -126, torch.float16: -14, torch.bfloat16: -126}[dtype]
    return 0.5 * np.exp2(np.maximum(e, emin) - _MANT_BITS[dtype])


def _log(record):
    """Append one parity record (test, plain max-abs, excess over half an
    output ulp, lse error) to the file IFA_PARITY_LOG names, if set."""
    path = os.environ.get("IFA_PARITY_LOG")
    if path:
        record["test"] = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


def _compare(w, out, lse, ref_out, ref_lse, rows=None):
    """Two bounds on every output element, both asserted:
    - plain: |gpu - oracle| <= tol wherever |oracle| < 2, where half an ulp
      of the output dtype (bf16: 2^-8 at most) leaves the bound room;
    - with output rounding (reading T1): |gpu - oracle| - half an ulp of the
      output dtype at that magnitude <= tol everywhere (a bf16 value in
      [4, 8) moves by up to 1/64 from its rounding alone).
    The plain max-abs over all elements is returned and logged."""
    tol = TOL_F32 if w.kv_dtype == torch.float32 else TOL_LOWP
    if rows is not None:
        out = np.stack([out[b, h] for b, h in rows])
        lse = np.array([lse[b, h] for b, h in rows])
    assert out.shape == ref_out.shape
    assert not np.isnan(out).any(), "NaN in GPU output"
    err = np.abs(out - ref_out)
    mag = np.maximum(np.abs(out), np.abs(ref_out))
    excess = err - half_ulp(mag, w.out_dtype)
    worst = float(np.max(excess)) if out.size else 0.0
    small = np.abs(ref_out) < 2.0
    plain_small = float(np.max(err[small])) if small.any() else 0.0
    plain = float(np.max(err)) if out.size else 0.0
    fin = np.isfinite(ref_lse)
    lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    _log({"max_abs": plain, "max_abs_below_2": plain_small, "t1_excess": worst, "lse_err": lerr,
          "max_abs_over_tol": plain > tol, "elements": int(out.size), "tol": tol})
    print(f"[parity] max-abs {plain:.3e} (|ref| < 2: {plain_small:.3e}), beyond half an output ulp {worst:.3e}, "
          f"lse {lerr:.3e}", flush=True)
    assert plain_small <= tol, f"max-abs {plain_small:.3e} > {tol} where |oracle| < 2"
    assert worst <= tol, f"error beyond output rounding {worst:.3e} > {tol} (max-abs {plain:.3e})"
    np.testing.assert_array_equal(lse[~fin], ref_lse[~fin])
    assert lerr <= TOL_LSE, f"lse error {lerr:.3e}"
    return plain


def _full_check(w, num_splits=None):
    _announce(f"{w.name} B={w.batch} nq={w.n_q} nkv={w.n_kv} d={w.qk_dim} kv={w.kv_dtype} "
              f"layout={w.layout} bs={w.block_size} lens={w.lengths()[:8]} splits={num_splits}")
    out, lse = _gpu(w, num_splits)
    ref_out, ref_lse = oracle.decode_workload(w)
    return _compare(w, out, lse, ref_out, ref_lse)


# ------------------------------------------------------------ the configs
@pytest.mark.parametrize("splits", [2, 1, 3])
def test_c1_tiny_fp32(splits):
    """Tiny fp32 config at full size: B=2, N=4, D=64, 128 tokens; 2 splits
    are the two halves of 64."""
    w = config_workload(1, seed=100)
    _full_check(w, splits)


@pytest.mark.parametrize("seed", [200, 201, 202])
def test_c2_f16_gqa_padded_reduced(seed):
    w = config_workload(2, seed=seed, batch=5, lengths=("uniform", 1, 700), s_cap=768)
    _full_check(w)


@pytest.mark.parametrize("seed", [300, 301, 302])
def test_c3_bf16_paged_reduced(seed):
    w = config_workload(3, seed=seed, batch=6, lengths=("uniform", 100, 1100), max_blocks_per_seq=9)
    _full_check(w)


@pytest.mark.parametrize("seed", [400, 401])
def test_c4_int8_antiquant_sink_reduced(seed):
    w = config_workload(4, seed=seed, batch=3, lengths=[300, 1, 129], max_blocks_per_seq=3)
    _full_check(w)


# ------------------------------------------------------------ edge cases
@pytest.mark.parametrize("kv,layout,n_q,d", [("bf16", "paged", 32, 128), ("f16", "bnsd", 32, 128),
                                              ("bf16", "paged", 64, 128), ("f16", "paged", 32, 64)])
def test_many_workgroups_ragged(kv, layout, n_q, d):
    """More items than resident workgroups (64 sequences x 8 KV heads x 4
    splits, about three rounds of dispatch), with lengths from a small set
    that includes empty and one-token splits, and eight heads per workgroup
    (n_q 64)."""
    lens = [int(x) for x in np.random.default_rng(n_q + d).choice([0, 1, 15, 16, 17, 100, 129, 300, 700], size=64)]
    kw = dict(block_size=64) if layout == "paged" else dict(s_cap=768)
    w = make_workload(batch=64, n_q=n_q, n_kv=8, qk_dim=d, kv_dtype=kv, layout=layout, lengths=lens,
                      seed=n_q + d + 11, **kw)
    _full_check(w, 4)


@pytest.mark.parametrize("layout", ["paged", "bnsd"])
def test_int8_group_32(layout):
    """One query token with 32 query heads per KV head: the 32-column int8
    kernel at S_q 1 (per-channel antiquant, sink), per-sequence splits and the
    balanced split."""
    lens = [1, 33, 64, 700, 2049]
    kw = dict(block_size=64, extra_blocks=1) if layout == "paged" else dict(s_cap=2112)
    w = make_workload(batch=len(lens), n_q=64, n_kv=2, qk_dim=128, kv_dtype="i8", layout=layout, lengths=lens,
                      seed=160, sink=True, antiquant=True, **kw)
    for splits in (3, None):
        _full_check(w, splits)


@pytest.mark.parametrize("batch", [65, 130, 256, 257])
@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_longest_first_batch_sizes(batch, kv):
    """Batches that span one to four 64-wide chunks of the longest-first
    ranking (bf16: each workgroup ranks; int8: the planning kernel ranks) and
    one beyond its 256 limit (index order), with many equal lengths, so that
    a lost, doubled or misplaced sequence would leave rows wrong."""
    lens = [int(x) for x in np.random.default_rng(batch).choice([0, 1, 17, 40, 64, 129], size=batch)]
    w = make_workload(batch=batch, n_q=8, n_kv=2, qk_dim=128, kv_dtype=kv, layout="paged", block_size=64,
                      lengths=lens, antiquant=kv == "i8", seed=batch + 7)
    _full_check(w, 2)


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16", "i8"])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths_every_dtype(kv, d):
    lens = [0, 1, 15, 16, 17, 31, 127, 128, 129, 300]
    w = make_workload(batch=len(lens), n_q=8, n_kv=2, qk_dim=d, kv_dtype=kv, layout="paged",
                      block_size=32, lengths=lens, seed=7, sink=(kv == "i8"), extra_blocks=2)
    _full_check(w, 3)


@pytest.mark.parametrize("kv,d,bs,lens,layout", [
    ("bf16", 128, 16, [3000, 1029, 17], "paged"),      # MFMA kernel, 16-bit K/V
    ("bf16", 128, 16, [3000, 1029, 17], "paged_bsh"),
    ("i8", 128, 32, [4100, 2080, 33], "paged"),        # MFMA kernel, int8 K/V
    ("f16", 64, 16, [1500, 1040, 5], "paged"),         # VALU kernel (head dim 64)
    ("f32", 64, 16, [1500, 1040, 5], "paged"),         # VALU kernel (fp32 K/V)
])
def test_split_spans_more_than_64_blocks(kv, d, bs, lens, layout):
    """One split per sequence over more than 64 cache blocks (up to 188):
    block ids past the 64 that a wave holds in lanes come from the block
    table through scalar loads (aclnnIncreFlashAttentionV3 "Constraints",
    page attention scenario: blockTable's second dimension covers
    maxBlockNumPerSeq)."""
    assert max(lens) // bs > 64
    w = make_workload(batch=len(lens), n_q=8, n_kv=2, qk_dim=d, kv_dtype=kv, layout=layout, block_size=bs,
                      lengths=lens, seed=31 + bs + d, sink=(kv == "i8"), extra_blocks=3)
    _full_check(w, 1)


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_block_sizes(bs):
    kv = "bf16"
    w = make_workload(batch=4, n_q=8, n_kv=8, qk_dim=128, kv_dtype=kv, layout="paged", block_size=bs,
                      lengths=[bs - 1, bs, bs + 1, 3 * bs + 5], seed=11)
    _full_check(w, 2)


@pytest.mark.parametrize("splits", [1, 2, 4, 7, 16, 64])
def test_split_counts(splits):
    """More splits than tiles leaves empty splits; every count gives the same answer."""
    w = make_workload(batch=3, n_q=16, n_kv=4, qk_dim=128, kv_dtype="f16", layout="bnsd",
                      lengths=[1000, 17, 1], s_cap=1024, seed=12)
    _full_check(w, splits)


@pytest.mark.parametrize("d,splits", [(64, 100), (64, 256), (128, 70), (128, 256)])
def test_many_splits(d, splits):
    """More than 64 non-empty splits in a row (the merge reduces statistics in
    chunks of 64 and reads partials in batches); short rows leave most of
    their splits empty."""
    w = make_workload(batch=4, n_q=8, n_kv=2, qk_dim=d, kv_dtype="f16", layout="bnsd",
                      lengths=[4096, 2001, 5, 0], s_cap=4096, seed=19)
    _full_check(w, splits)


def test_stale_workspace_slots_ignored():
    """Workspace slots of empty splits are never written; NaN left in them by
    earlier use must not reach the output."""
    w = make_workload(batch=3, n_q=16, n_kv=4, qk_dim=128, kv_dtype="bf16", layout="paged", block_size=16,
                      lengths=[700, 17, 1], seed=20)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg, num_splits=16)
    call.workspace.view(torch.float32).fill_(float("nan"))
    out, lse = call.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_workload(w)
    _compare(w, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_unaligned_output_buffer(out_dtype):
    """attention_out one element past a 16-byte boundary (element-wise stores)."""
    w = make_workload(batch=2, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", out_dtype=out_dtype, layout="paged",
                      block_size=64, lengths=[300, 45], seed=21)
    wg = w.to("cuda")
    n = w.batch * w.n_q * w.v_dim
    buf = torch.full((n + 1,), float("nan"), dtype=wg.out_dtype, device="cuda")
    out_view = buf[1:].view(w.batch, w.n_q, w.v_dim)
    call = ifa.call_for_workload(wg, num_splits=3, out=out_view)
    out, lse = call.run()
    torch.cuda.synchronize()
    assert out.data_ptr() % 16 != 0
    assert torch.isnan(buf[0]).item()
    ref_out, ref_lse = oracle.decode_workload(w)
    _compare(w, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("kv", ["f16", "bf16"])
def test_unaligned_query_buffer(kv):
    """query one element past a 16-byte boundary (element-wise q loads)."""
    w = make_workload(batch=2, n_q=8, n_kv=2, qk_dim=128, kv_dtype=kv, layout="paged", block_size=64,
                      lengths=[300, 45], seed=22)
    wg = w.to("cuda")
    buf = torch.empty(wg.q.numel() + 1, dtype=wg.q.dtype, device="cuda")
    q = buf[1:].view(wg.q.shape)
    q.copy_(wg.q)
    assert q.data_ptr() % 16 != 0
    out, lse = ifa.decode(q, wg.k_cache, wg.v_cache, wg.block_table, wg.seq_lens, w.n_q, w.n_kv, w.scale,
                          learnable_sink=wg.sink, num_splits=3, v_dim=w.v_dim, out_dtype=wg.out_dtype)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_workload(w)
    _compare(w, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
def test_gqa_group_sizes(group):
    w = make_workload(batch=2, n_q=8 * group if group < 16 else 32, n_kv=8 if group < 16 else 2,
                      qk_dim=128, kv_dtype="bf16", layout="paged", block_size=64, lengths=[200, 77], seed=13)
    _full_check(w)


def test_num_key_value_heads_zero_means_mha():
    w = make_workload(batch=2, n_q=4, n_kv=0, qk_dim=64, kv_dtype="f16", layout="bnsd",
                      lengths=[50, 64], s_cap=64, seed=14)
    assert w.n_kv == 4
    wg = w.to("cuda")
    out, lse = ifa.decode(wg.q, wg.k_cache, wg.v_cache, None, wg.seq_lens, 4, 0, wg.scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_workload(w)
    _compare(w, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("length", [0, 1, 7, 128])
@pytest.mark.parametrize("sink", [-5.0, 0.0, 8.0])
def test_sink_dedicated(length, sink):
    """The sink adds e^(sink - m) to the denominator (aclnnFlashAttentionScoreV4
    formula); short rows make its effect large enough to see."""
    w = make_workload(batch=2, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", layout="paged", block_size=32,
                      lengths=[length, max(1, length)], seed=15, sink=True)
    w.sink = torch.full_like(w.sink, sink)
    _full_check(w, 2)


def test_empty_batch_gives_zero_and_neg_inf_lse():
    w = make_workload(batch=3, n_q=4, n_kv=4, qk_dim=64, kv_dtype="f32", layout="bnsd",
                      lengths=[0, 0, 0], s_cap=16, seed=16)
    out, lse = _gpu(w, 2)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_output_dtype_f32_from_bf16():
    w = make_workload(batch=2, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", out_dtype="f32", layout="paged",
                      block_size=128, lengths=[333, 1], seed=17)
    _full_check(w)


def test_deterministic_bitwise():
    w = config_workload(3, seed=303, batch=4, lengths=("uniform", 100, 1100), max_blocks_per_seq=9).to("cuda")
    o1, l1 = ifa.decode_workload(w)
    o2, l2 = ifa.decode_workload(w)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_partials_match_oracle_triples():
    """ifa_decode_splitkv leaves, per (b, h, split), the triple of the
    split's token span [i*c, min(L, (i+1)*c)), c = 16*ceil(ceil(L/n)/16)."""
    w = make_workload(batch=3, n_q=8, n_kv=2, qk_dim=128, kv_dtype="f16", layout="paged", block_size=16,
                      lengths=[250, 33, 1], seed=18)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg, num_splits=4)
    call.splitkv()
    torch.cuda.synchronize()
    po, pm, ps = (x.double().cpu().numpy() for x in call.partials())
    n = call.num_splits
    qf = w.q.double().numpy()
    for b, L in enumerate(w.lengths()):
        c = 16 * math.ceil(math.ceil(L / n) / 16)
        for g in range(2):
            K = oracle.gather_kv(w.k_cache, "paged", b, g, L, w.block_table, 16)
            V = oracle.gather_kv(w.v_cache, "paged", b, g, L, w.block_table, 16)
            for h in range(g * 4, g * 4 + 4):
                for i in range(n):
                    a, e = i * c, min(L, (i + 1) * c)
                    if a >= e:
                        continue
                    o, m, s = oracle.partial_triple(qf[b, h], K[a:e], V[a:e], w.scale)
                    assert np.max(np.abs(po[b, h, i] - o)) < 1e-3
                    assert abs(pm[b, h, i] - m) < 1e-4 * max(1, abs(m))
                    assert abs(ps[b, h, i] - s) < 1e-4 * s


def test_timed_splitkv_same_partials():
    """ifa_decode_splitkv_timed leaves the same workspace as
    ifa_decode_splitkv and records a positive kernel time."""
    w = make_workload(batch=3, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", layout="paged", block_size=64,
                      lengths=[900, 33, 1], seed=23)
    wg = w.to("cuda")
    c1 = ifa.call_for_workload(wg, num_splits=4)
    c2 = ifa.call_for_workload(wg, num_splits=4)
    c1.workspace.zero_()  # slots of empty splits are never written
    c2.workspace.zero_()
    c1.splitkv()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c2.splitkv_timed(e0, e1)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) > 0
    for x, y in zip(c1.partials(), c2.partials()):
        assert torch.equal(x, y)


# ------------------------------------------------------------ full sizes, sampled rows
def _sampled_rows(w, k, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(0, w.batch)), int(rng.integers(0, w.n_q))) for _ in range(k)]


def whole_sequence_rows(w, seed, extra=6):
    """Every query head of the longest, the shortest and a median-length
    sequence, plus ``extra`` random (sequence, head) pairs."""
    lens = w.lengths()
    order = sorted(range(w.batch), key=lambda b: (lens[b], b))
    picks = []
    for b in (order[-1], order[0], order[len(order) // 2]):
        if b not in picks:
            picks.append(b)
    rows = [(b, h) for b in picks for h in range(w.n_q)]
    return rows + _sampled_rows(w, extra, seed)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_sampled_rows(cfg):
    """Each config at its full size and in the launch configuration the
    benchmark times; the oracle recomputes every head of the longest, the
    shortest and a median sequence (all their splits) and a few random rows."""
    wg = config_workload(cfg, device="cuda")
    _announce(f"full size config {cfg}: {wg.name}")
    out, lse = ifa.decode_workload(wg)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    assert not np.isnan(out).any()
    w = wg.to("cpu")
    del wg
    torch.cuda.empty_cache()
    rows = whole_sequence_rows(w, cfg)
    ref_out, ref_lse = oracle.decode_workload(w, rows=rows)
    _compare(w, out, lse, ref_out, ref_lse, rows=rows)


# ------------------------------------------------ token-major layouts, per-tensor antiquant
@pytest.mark.parametrize("layout", ["paged_bsh", "bsnd"])
@pytest.mark.parametrize("kv", ["f32", "f16", "bf16", "i8"])
@pytest.mark.parametrize("d", [64, 128])
def test_token_major_layouts(layout, kv, d):
    """The (blocknum, blocksize, H) pool and the contiguous (B, S, H) cache:
    consecutive tokens of a KV head are N_kv rows apart.  Ragged lengths
    across block and tile boundaries, NaN-poisoned unused slots."""
    lens = [0, 1, 15, 16, 17, 31, 127, 128, 129, 300]
    kw = dict(block_size=32, extra_blocks=2) if layout == "paged_bsh" else dict(s_cap=320)
    w = make_workload(batch=len(lens), n_q=8, n_kv=2, qk_dim=d, kv_dtype=kv, layout=layout,
                      lengths=lens, seed=71 + d, sink=(kv == "i8"), **kw)
    _full_check(w, 3)


@pytest.mark.parametrize("layout", ["paged", "paged_bsh", "bsnd"])
@pytest.mark.parametrize("splits", [1, 3])
def test_per_tensor_antiquant(layout, splits):
    """int8 K/V with one scale and offset for K and one for V (shape (2))."""
    kw = dict(block_size=64) if layout != "bsnd" else dict(s_cap=704)
    w = make_workload(batch=4, n_q=16, n_kv=4, qk_dim=128, kv_dtype="i8", layout=layout,
                      lengths=[700, 1, 64, 333], seed=81 + splits, sink=True, antiquant_mode="tensor", **kw)
    assert tuple(w.antiquant_scale.shape) == (2,)
    _full_check(w, splits)


@pytest.mark.parametrize("layout", ["paged", "paged_bsh", "bnsd", "bsnd"])
@pytest.mark.parametrize("mode", ["token", "token_head"])
@pytest.mark.parametrize("splits", [1, 3])
def test_per_token_antiquant(layout, mode, splits):
    """int8 K/V with one (scale, offset) pair per logical token position
    (FusedInferAttentionScore blog antiquantMode 1, and 3 with per-head
    pairs; reading R24): ragged lengths across tile and block boundaries,
    a sink, a permuted paged pool, NaN-poisoned unread slots."""
    lens = [0, 1, 31, 32, 33, 129, 300, 517]
    kw = dict(block_size=32, extra_blocks=2) if layout.startswith("paged") else dict(s_cap=520)
    w = make_workload(batch=len(lens), n_q=16, n_kv=4, qk_dim=128, kv_dtype="i8", layout=layout, lengths=lens,
                      seed=91 + splits, sink=True, antiquant_mode=mode, **kw)
    assert w.antiquant_scale.dim() == (3 if mode == "token" else 4)
    _full_check(w, splits)


def test_per_token_antiquant_full_size_sampled_rows():
    """The int8 workload at full size (B=32, N_q=64, N_kv=8, 16384 tokens,
    paged block 128, sink) with per-token antiquant pairs (2, 32, 16384);
    every head of three whole sequences against the oracle."""
    wg = config_workload(4, device="cuda", antiquant_mode="token")
    _announce("full size config 4 with per-token antiquant")
    out, lse = ifa.decode_workload(wg)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    assert not np.isnan(out).any()
    w = wg.to("cpu")
    del wg
    torch.cuda.empty_cache()
    rows = whole_sequence_rows(w, 44)
    ref_out, ref_lse = oracle.decode_workload(w, rows=rows)
    _compare(w, out, lse, ref_out, ref_lse, rows=rows)


def test_per_token_antiquant_rejects_head_dim_64():
    w = make_workload(batch=2, n_q=4, n_kv=2, qk_dim=64, kv_dtype="i8", layout="paged", block_size=32,
                      lengths=[40, 7], seed=95, antiquant_mode="token").to("cuda")
    with pytest.raises(ValueError, match="head dim 128"):
        ifa.decode_workload(w)


def test_full_size_token_major_pool_sampled_rows():
    """The paged bf16 GQA workload at full size (B=64, N_q=32, N_kv=8,
    lengths U[512, 8192]) with its pool in the (blocknum, blocksize, H)
    layout; the oracle recomputes a sample of rows."""
    wg = config_workload(3, device="cuda", layout="paged_bsh")
    _announce(f"full size config 3 in the paged_bsh layout")
    out, lse = ifa.decode_workload(wg)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    assert not np.isnan(out).any()
    w = wg.to("cpu")
    del wg
    torch.cuda.empty_cache()
    rows = whole_sequence_rows(w, 33)
    ref_out, ref_lse = oracle.decode_workload(w, rows=rows)
    _compare(w, out, lse, ref_out, ref_lse, rows=rows)


def test_check_inputs_reports_out_of_range_arguments():
    """ifa_decode_check_inputs: 0 for in-range lengths and tables (unused
    entries hold -1 and are not read); the bad-block bit for a used entry
    outside the pool; the bad-length bit for a length above the capacity or
    below 0; contiguous layouts check lengths against s_cap."""
    w = make_workload(batch=3, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", layout="paged", block_size=32,
                      lengths=[100, 40, 7], max_blocks_per_seq=5, seed=60)
    wg = w.to("cuda")
    _announce("input check")

    def flags(table=None, lens=None, layout_w=wg):
        c = ifa.DecodeCall(layout_w.q, layout_w.k_cache, layout_w.v_cache,
                           layout_w.block_table if table is None else table,
                           layout_w.seq_lens if lens is None else lens, w.n_q, w.n_kv, w.scale,
                           kv_layout=layout_w.layout)
        f = c.check_inputs()
        torch.cuda.synchronize()
        return int(f.item())

    assert flags() == 0
    bad = wg.block_table.clone()
    bad[1, 1] = 10_000  # sequence 1 reads blocks 0 and 1
    assert flags(table=bad) == ifa.IFA_CHECK_BAD_BLOCK
    bad = wg.block_table.clone()
    bad[0, 3] = -7
    assert flags(table=bad) == ifa.IFA_CHECK_BAD_BLOCK
    bad = wg.block_table.clone()
    bad[2, 4] = 10_000  # beyond sequence 2's one block: never read
    assert flags(table=bad) == 0
    lens = wg.seq_lens.clone()
    lens[2] = -1
    assert flags(lens=lens) == ifa.IFA_CHECK_BAD_LENGTH
    lens = wg.seq_lens.clone()
    lens[1] = 161  # capacity 5 x 32 = 160; the clamped length reads all five entries, three of them -1
    assert flags(lens=lens) == ifa.IFA_CHECK_BAD_LENGTH | ifa.IFA_CHECK_BAD_BLOCK
    c = make_workload(batch=2, n_q=8, n_kv=2, qk_dim=128, kv_dtype="bf16", layout="bnsd", lengths=[10, 64],
                      s_cap=64, seed=61).to("cuda")
    assert flags(layout_w=c) == 0
    lens = c.seq_lens.clone()
    lens[0] = 65
    assert flags(lens=lens, layout_w=c) == ifa.IFA_CHECK_BAD_LENGTH

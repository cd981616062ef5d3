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

from test_gpu_decode import _announce, _compare, _full_check, _sampled_rows

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
    benchmark times; the oracle recomputes a sample of rows one by one."""
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
    rows = _sampled_rows(w, 8, 5)
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

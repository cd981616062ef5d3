"""GPU parity of attn_update (aclnnRingAttentionUpdate) against the oracle's
merge, read in its sum-weighted form."""

import math

import numpy as np
import pytest
import torch

import attention_ifa_decode_amd as ifa
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.float16: 1e-2, torch.bfloat16: 1e-2}


def _stats(rng, rows, stride):
    m = torch.tensor(rng.standard_normal(rows) * 3, dtype=torch.float32)
    s = torch.tensor(rng.uniform(0.5, 40, rows), dtype=torch.float32)
    return m[:, None].repeat(1, stride).contiguous(), s[:, None].repeat(1, stride).contiguous()


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("stride", [1, 8])
@pytest.mark.parametrize("d", [64, 128, 512, 768, 100])
def test_update_matches_oracle(dtype, stride, d):
    rng = np.random.default_rng(d + stride)
    rows = 37
    po = torch.tensor(rng.standard_normal((rows, d)), dtype=torch.float32).to(dtype)
    co = torch.tensor(rng.standard_normal((rows, d)), dtype=torch.float32).to(dtype)
    pm, ps = _stats(rng, rows, stride)
    cm, cs = _stats(rng, rows, stride)
    out, mo, so = ifa.attn_update(*(t.cuda() for t in (po, pm, ps, co, cm, cs)))
    torch.cuda.synchronize()
    ro, rm, rs = oracle.attn_update(po, pm[:, 0], ps[:, 0], co, cm[:, 0], cs[:, 0])
    err = np.max(np.abs(out.double().cpu().numpy() - ro))
    assert err <= TOL[dtype], err
    mo, so = mo.cpu().double().numpy(), so.cpu().double().numpy()
    for k in range(stride):
        np.testing.assert_allclose(mo[:, k], rm, rtol=0, atol=0)  # max is exact
        np.testing.assert_allclose(so[:, k], rs, rtol=1e-5)


def test_update_in_place_and_empty_sides():
    rng = np.random.default_rng(5)
    rows, d = 6, 64
    po = torch.tensor(rng.standard_normal((rows, d)), dtype=torch.float32).cuda()
    co = torch.tensor(rng.standard_normal((rows, d)), dtype=torch.float32).cuda()
    pm = torch.tensor(rng.standard_normal(rows), dtype=torch.float32).cuda()
    ps = torch.tensor(rng.uniform(1, 3, rows), dtype=torch.float32).cuda()
    cm, cs = pm.clone(), ps.clone()
    # rows 0-1: prev empty (its out holds NaN); rows 2-3: cur empty; row 4: both empty
    po[0:2] = float("nan"); pm[0:2] = -math.inf; ps[0:2] = 0
    co[2:4] = float("nan"); cm[2:4] = -math.inf; cs[2:4] = 0
    po[4] = co[4] = float("nan"); pm[4] = cm[4] = -math.inf; ps[4] = cs[4] = 0
    ref = oracle.attn_update(*(t.cpu() for t in (po.nan_to_num(), pm, ps, co.nan_to_num(), cm, cs)))
    co_before = co.clone()
    ifa.attn_update(po, pm, ps, co, cm, cs, out=po, max_out=pm, sum_out=ps)  # accumulate into prev
    torch.cuda.synchronize()
    out = po.double().cpu().numpy()
    assert not np.isnan(out).any()
    np.testing.assert_allclose(out, ref[0], atol=1e-6)
    np.testing.assert_array_equal(out[0:2], co_before[0:2].double().cpu().numpy())
    assert np.all(out[4] == 0) and pm[4].item() == -math.inf and ps[4].item() == 0


def test_chain_reproduces_full_attention():
    """Three partial results of one KV axis (computed by the oracle), merged
    pairwise on the GPU, give the attention over the whole axis."""
    rng = np.random.default_rng(9)
    rows, D, L = 16, 128, 300
    q = rng.standard_normal((rows, D))
    K = rng.standard_normal((rows, L, D))
    V = rng.standard_normal((rows, L, D))
    cuts = [0, 90, 91, 300]
    parts = []
    for a, e in zip(cuts[:-1], cuts[1:]):
        tr = [oracle.partial_triple(q[r], K[r, a:e], V[r, a:e], 0.1) for r in range(rows)]
        parts.append(tuple(torch.tensor(np.array(x), dtype=torch.float32).cuda() for x in zip(*tr)))
    o, m, s = parts[0]
    for (o2, m2, s2) in parts[1:]:
        o, m, s = ifa.attn_update(o, m, s, o2, m2, s2)
    torch.cuda.synchronize()
    for r in range(rows):
        full, lse = oracle.attention_row(q[r], K[r], V[r], 0.1)
        assert np.max(np.abs(o[r].double().cpu().numpy() - full)) < 1e-5
        assert abs(m[r].item() + math.log(s[r].item()) - lse) < 1e-4

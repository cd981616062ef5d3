"""GPU parity over a seeded random sample of the supported argument space.

Each case draws one combination of what the decode accepts: K/V dtype
(f32, f16, bf16, int8 with an f32, f16 or bf16 query), head dim 64 or 128,
KV heads and group size (N_q = G * N_kv up to 256, G not always a power of
two), every KV layout, block sizes from 16 to 256, ragged lengths with empty
and one-token sequences, automatic or explicit split counts, a learnable
sink or none, every int8 antiquant mode, an output dtype other than the
query's, and 1 to 6 query tokens per sequence under no mask,
rightDownCausal or a tree mask; one case in ten is the MLA shape (32 to 128
heads over one 576-wide latent KV head).  The oracle recomputes every
output; the tolerances are those of the other parity tests.
"""

import numpy as np
import pytest
import torch

from synth import make_workload

from test_gpu_decode import _full_check
from test_gpu_spec import _check, _query, _tree

N_CASES = 96


def _lengths(rng, B, hi):
    """Ragged lengths: about one in eight empty, one in eight a single token,
    the rest spread over short, medium and long."""
    out = []
    for _ in range(B):
        r = rng.random()
        if r < 0.125:
            out.append(0)
        elif r < 0.25:
            out.append(1)
        elif r < 0.5:
            out.append(int(rng.integers(2, 48)))
        elif r < 0.8:
            out.append(int(rng.integers(48, 700)))
        else:
            out.append(int(rng.integers(700, hi + 1)))
    if max(out) == 0:
        out[0] = int(rng.integers(1, 300))
    return out


def _case(i):
    """The arguments of case i (seeded), as keyword arguments of make_workload
    plus the query tokens, mask and split count."""
    rng = np.random.default_rng(7100 + i)
    B = int(rng.integers(1, 7))
    splits = [0, 0, 1, 2, 3, 5, 16][int(rng.integers(0, 7))]  # 0: automatic
    if i % 10 == 9:  # MLA shape
        layout = ["paged", "bnsd"][int(rng.integers(0, 2))]
        lens = _lengths(rng, B, 2500)
        kw = dict(batch=B, n_q=int(rng.choice([32, 64, 128])), n_kv=1, qk_dim=576, v_dim=512, kv_dtype="bf16",
                  layout=layout, block_size=int(rng.choice([16, 32, 64, 128])), lengths=lens,
                  v_aliases_k=True, sink=bool(rng.random() < 0.5), scale=192 ** -0.5)
        if layout == "bnsd":
            kw["s_cap"] = max(lens) + int(rng.integers(0, 40))
        return kw, 1, "none", splits
    kv = ["f32", "f16", "bf16", "i8"][int(rng.integers(0, 4))]
    aq = None
    if kv == "i8":
        aq = ["channel", "tensor", "token", "token_head"][int(rng.integers(0, 4))]
    d = 128 if (aq in ("token", "token_head") or rng.random() < 0.6) else 64
    n_kv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32]))
    while g * n_kv > 256:
        g //= 2
    layout = ["paged", "paged_bsh", "bnsd", "bsnd"][int(rng.integers(0, 4))]
    bs = int(rng.choice([32, 64, 96, 128, 256] if kv == "i8" else [16, 32, 48, 64, 96, 128, 256]))
    lens = _lengths(rng, B, 2500)
    q_seq = 1 if rng.random() < 0.65 else int(rng.integers(2, 7))
    mode = "none" if q_seq == 1 and rng.random() < 0.7 else ["none", "causal", "tree"][int(rng.integers(0, 3))]
    kw = dict(batch=B, n_q=g * n_kv, n_kv=n_kv, qk_dim=d, kv_dtype=kv, layout=layout, block_size=bs, lengths=lens,
              sink=bool(rng.random() < 0.5), extra_blocks=int(rng.integers(0, 3)))
    if kv == "i8":
        kw["q_dtype"] = ["bf16", "f16", "f32"][int(rng.integers(0, 3))]
        kw["antiquant_mode"] = aq
    if rng.random() < 0.25:
        kw["out_dtype"] = "f32" if kv != "f32" else "bf16"
    if layout in ("bnsd", "bsnd"):
        kw["s_cap"] = max(lens) + int(rng.integers(0, 40))
    return kw, q_seq, mode, splits


def test_case_generator_draws_the_space():
    """Host-side: the sample reaches every dtype, layout, mode and shape kind."""
    cases = [_case(i) for i in range(N_CASES)]
    kinds = {c[0]["kv_dtype"] for c in cases}
    layouts = {c[0]["layout"] for c in cases}
    modes = {c[2] for c in cases}
    assert kinds == {"f32", "f16", "bf16", "i8"}
    assert layouts == {"paged", "paged_bsh", "bnsd", "bsnd"}
    assert modes == {"none", "causal", "tree"}
    assert any(c[0]["qk_dim"] == 576 for c in cases)
    assert any(0 in c[0]["lengths"] for c in cases) and any(1 in c[0]["lengths"] for c in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    kw, q_seq, mode, splits = _case(i)
    w = make_workload(name=f"sweep{i}", seed=7300 + i, **kw)
    if kw["qk_dim"] == 576:
        _full_check(w, splits)
        return
    q = _query(w.batch, q_seq, w.n_q, w.qk_dim, w.q.dtype, 7500 + i)
    _check(w, q, mode, _tree(w.batch, q_seq, 7700 + i) if mode == "tree" else None, splits)

"""Seeded synthetic decode-attention workloads.

Shapes and value distributions follow the decode-attention workloads of the
aclnnIncreFlashAttentionV3 page (query sequence length 1, per-batch actual KV
lengths, GQA, paged KV with a block table, int8 KV with per-channel
antiquant parameters) and the MLA shapes of the aclnnMlaPrologV3WeightNz page
(one 512-wide latent KV head plus a 64-wide rope part).

Structure (lengths, block permutation, block table) is always drawn on the
CPU from ``torch.Generator().manual_seed(seed)`` so it does not depend on the
device; tensor values are drawn from a generator on the target device seeded
with ``seed + 1``.  No attention arithmetic lives here.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Union

import torch

DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "i8": torch.int8,
}

LAYOUT_BNSD = "bnsd"  # contiguous (B, N_kv, S_cap, D)
LAYOUT_BSND = "bsnd"  # contiguous (B, S_cap, N_kv, D), i.e. (B, S_cap, H)
LAYOUT_PAGED = "paged"  # block pool (num_blocks, N_kv, block_size, D)
LAYOUT_PAGED_BSH = "paged_bsh"  # block pool (num_blocks, block_size, N_kv, D), i.e. (num_blocks, block_size, H)
PAGED_LAYOUTS = (LAYOUT_PAGED, LAYOUT_PAGED_BSH)


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor  # (B, N_q, qk_dim)
    k_cache: torch.Tensor
    v_cache: torch.Tensor  # the same tensor as k_cache when v aliases k (MLA)
    layout: str
    block_table: Optional[torch.Tensor]  # int32 (B, max_blocks_per_seq), -1 past use
    seq_lens: torch.Tensor  # int64 (B,)
    n_q: int
    n_kv: int
    qk_dim: int
    v_dim: int
    block_size: int
    s_cap: int  # BNSD: padded length; paged: max_blocks_per_seq * block_size
    scale: float
    out_dtype: torch.dtype
    sink: Optional[torch.Tensor] = None  # fp32 (N_q,)
    # fp32 (2, N_kv, D) per channel, (2,) per tensor, (2, B, s_cap) per token,
    # (2, B, N_kv, s_cap) per token and KV head
    antiquant_scale: Optional[torch.Tensor] = None
    antiquant_offset: Optional[torch.Tensor] = None  # the same shape as antiquant_scale
    antiquant_mode: Optional[str] = None  # "channel", "tensor", "token", "token_head" (None without antiquant)
    num_splits: int = 0

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def v_aliases_k(self) -> bool:
        return self.v_cache.data_ptr() == self.k_cache.data_ptr()

    @property
    def kv_dtype(self) -> torch.dtype:
        return self.k_cache.dtype

    def lengths(self) -> list:
        return [int(x) for x in self.seq_lens.cpu().tolist()]

    def kv_bytes(self) -> int:
        """Bytes of K and V that belong to valid tokens (V once if it aliases K)."""
        esz = self.k_cache.element_size()
        tok = sum(self.lengths())
        per_tok = self.n_kv * self.qk_dim * esz
        if not self.v_aliases_k:
            per_tok += self.n_kv * self.v_dim * esz
        return tok * per_tok

    def to(self, device) -> "Workload":
        def mv(t):
            return None if t is None else t.to(device)

        k = self.k_cache.to(device)
        v = k if self.v_aliases_k else self.v_cache.to(device)
        return dataclasses.replace(
            self,
            q=mv(self.q),
            k_cache=k,
            v_cache=v,
            block_table=mv(self.block_table),
            seq_lens=mv(self.seq_lens),
            sink=mv(self.sink),
            antiquant_scale=mv(self.antiquant_scale),
            antiquant_offset=mv(self.antiquant_offset),
        )


def blocks_needed(lengths: Sequence[int], block_size: int) -> int:
    """Number of pool blocks the lengths occupy, one partial block rounded up."""
    return sum((int(L) + block_size - 1) // block_size for L in lengths)


def paged_block_table(
    lengths: Sequence[int],
    block_size: int,
    max_blocks_per_seq: int,
    gen: torch.Generator,
    extra_blocks: int = 0,
):
    """Seeded random block assignment.

    The pool holds ``blocks_needed(lengths) + extra_blocks`` blocks.  A random
    permutation of the pool is dealt out batch-major: batch b takes the next
    ceil(L_b / block_size) entries.  Unused table entries are -1 so that any
    read past a sequence's last block would be visible.
    """
    B = len(lengths)
    need = blocks_needed(lengths, block_size)
    pool = need + extra_blocks
    perm = torch.randperm(pool, generator=gen)
    table = torch.full((B, max_blocks_per_seq), -1, dtype=torch.int32)
    off = 0
    for b, L in enumerate(lengths):
        nb = (int(L) + block_size - 1) // block_size
        if nb > max_blocks_per_seq:
            raise ValueError("length exceeds max_blocks_per_seq * block_size")
        table[b, :nb] = perm[off:off + nb].to(torch.int32)
        off += nb
    return table, pool


def _draw_lengths(spec, B: int, gen: torch.Generator):
    """spec: int (all equal), list of ints, or ("uniform", lo, hi) inclusive."""
    if isinstance(spec, int):
        return [spec] * B
    if isinstance(spec, tuple) and spec and spec[0] == "uniform":
        lo, hi = int(spec[1]), int(spec[2])
        return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=gen).tolist()]
    vals = [int(x) for x in spec]
    if len(vals) != B:
        raise ValueError("length list must have B entries")
    return vals


def _randn_as(shape, dtype, gen, device, chunk_elems=1 << 26):
    """N(0,1) in fp32 then cast (round-to-nearest-even) to dtype; int8 gets
    round(clip(N(0,1) * 32, -128, 127)) with ties to even."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if dtype == torch.int8:
            x = torch.round(torch.clamp(x * 32.0, -128.0, 127.0))
        flat[s:e] = x.to(dtype)
    return out


def _poison_value(dtype):
    if dtype == torch.int8:
        return 127
    return float("nan")


def make_workload(
    *,
    name: str = "custom",
    batch: int,
    n_q: int,
    n_kv: int,
    qk_dim: int,
    v_dim: Optional[int] = None,
    kv_dtype: str = "bf16",
    q_dtype: Optional[str] = None,
    out_dtype: Optional[str] = None,
    layout: str = LAYOUT_PAGED,
    block_size: int = 128,
    lengths: Union[int, Sequence[int], tuple] = 128,
    s_cap: Optional[int] = None,
    max_blocks_per_seq: Optional[int] = None,
    scale: Optional[float] = None,
    sink: bool = False,
    antiquant: bool = False,
    antiquant_mode: str = "channel",
    v_aliases_k: bool = False,
    seed: int = 0,
    device: Union[str, torch.device] = "cpu",
    poison: bool = True,
    extra_blocks: int = 0,
    value_seed: Optional[int] = None,
    num_splits: int = 0,
) -> Workload:
    """Build one seeded workload.

    ``v_aliases_k`` builds the MLA form: one cache whose first ``v_dim``
    channels serve as V.  ``poison`` fills every stored slot that the decode
    must never read (contiguous padding past the length, tail slots of a
    sequence's last block, unused pool blocks) with NaN (127 for int8).
    ``antiquant_mode`` "channel" gives (2, N_kv, D) parameters, "tensor" (2,),
    "token" (2, B, s_cap) (one pair per logical token position) and
    "token_head" (2, B, N_kv, s_cap), with s_cap the paged capacity
    max_blocks_per_seq * block_size or the contiguous padded length.
    ``value_seed`` (default ``seed + 1``) seeds the tensor values alone, so
    that workloads with one ``seed`` and different ``value_seed`` share their
    lengths, block table and poisoned slots and differ only in the values.
    """
    v_dim = qk_dim if v_dim is None else v_dim
    n_kv_eff = n_q if n_kv == 0 else n_kv
    if kv_dtype == "i8":
        q_dtype = q_dtype or "bf16"
        antiquant = True
    q_dtype = q_dtype or kv_dtype
    out_dtype = out_dtype or q_dtype
    sgen = torch.Generator().manual_seed(seed)
    lens = _draw_lengths(lengths, batch, sgen)
    dev = torch.device(device)
    vgen = torch.Generator(device=dev).manual_seed(seed + 1 if value_seed is None else value_seed)
    kdt = DTYPES[kv_dtype]

    q = _randn_as((batch, n_q, qk_dim), DTYPES[q_dtype], vgen, dev)

    if layout in PAGED_LAYOUTS:
        bsh = layout == LAYOUT_PAGED_BSH
        if max_blocks_per_seq is None:
            max_blocks_per_seq = max(1, max((L + block_size - 1) // block_size for L in lens))
        table, pool = paged_block_table(lens, block_size, max_blocks_per_seq, sgen, extra_blocks)
        kshape = (pool, block_size, n_kv_eff, qk_dim) if bsh else (pool, n_kv_eff, block_size, qk_dim)
        vshape = (pool, block_size, n_kv_eff, v_dim) if bsh else (pool, n_kv_eff, block_size, v_dim)
        k_cache = _randn_as(kshape, kdt, vgen, dev)
        v_cache = k_cache if v_aliases_k else _randn_as(vshape, kdt, vgen, dev)
        if poison:
            pv = _poison_value(kdt)
            used = torch.zeros(pool, dtype=torch.bool)
            for b, L in enumerate(lens):
                nb = (L + block_size - 1) // block_size
                blks = table[b, :nb].long()
                used[blks] = True
                if nb and L % block_size:
                    last = int(blks[-1])
                    for c in (k_cache,) if v_aliases_k else (k_cache, v_cache):
                        if bsh:
                            c[last, L % block_size:] = pv
                        else:
                            c[last, :, L % block_size:] = pv
            unused = (~used).nonzero().flatten().to(dev)
            if unused.numel():
                k_cache[unused] = pv
                if not v_aliases_k:
                    v_cache[unused] = pv
        s_cap_eff = max_blocks_per_seq * block_size
        block_table = table.to(dev)
    elif layout in (LAYOUT_BNSD, LAYOUT_BSND):
        bsnd = layout == LAYOUT_BSND
        s_cap_eff = s_cap if s_cap is not None else max(1, max(lens))
        if max(lens) > s_cap_eff:
            raise ValueError("length exceeds s_cap")
        kshape = (batch, s_cap_eff, n_kv_eff, qk_dim) if bsnd else (batch, n_kv_eff, s_cap_eff, qk_dim)
        vshape = (batch, s_cap_eff, n_kv_eff, v_dim) if bsnd else (batch, n_kv_eff, s_cap_eff, v_dim)
        k_cache = _randn_as(kshape, kdt, vgen, dev)
        v_cache = k_cache if v_aliases_k else _randn_as(vshape, kdt, vgen, dev)
        if poison:
            pv = _poison_value(kdt)
            for b, L in enumerate(lens):
                for c in (k_cache,) if v_aliases_k else (k_cache, v_cache):
                    if bsnd:
                        c[b, L:] = pv
                    else:
                        c[b, :, L:] = pv
        block_table = None
        block_size = 0
    else:
        raise ValueError(f"unknown layout {layout}")

    if scale is None:
        scale = 1.0 / math.sqrt(qk_dim)
    sink_t = torch.randn(n_q, generator=vgen, device=dev, dtype=torch.float32) if sink else None
    aq_s = aq_o = None
    if antiquant:
        ashape = {"tensor": (2,), "channel": (2, n_kv_eff, qk_dim), "token": (2, batch, s_cap_eff),
                  "token_head": (2, batch, n_kv_eff, s_cap_eff)}[antiquant_mode]
        aq_s = torch.rand(ashape, generator=vgen, device=dev, dtype=torch.float32) * 0.02 + 0.02
        aq_o = torch.rand(ashape, generator=vgen, device=dev, dtype=torch.float32) * 2.0 - 1.0
    return Workload(
        name=name,
        q=q,
        k_cache=k_cache,
        v_cache=v_cache,
        layout=layout,
        block_table=block_table,
        seq_lens=torch.tensor(lens, dtype=torch.int64, device=dev),
        n_q=n_q,
        n_kv=n_kv_eff,
        qk_dim=qk_dim,
        v_dim=v_dim,
        block_size=block_size,
        s_cap=s_cap_eff,
        scale=float(scale),
        out_dtype=DTYPES[out_dtype],
        sink=sink_t,
        antiquant_scale=aq_s,
        antiquant_offset=aq_o,
        antiquant_mode=antiquant_mode if antiquant else None,
        num_splits=num_splits,
    )


# The five decode workloads, at full size.  Index 1..5.
CONFIGS = {
    1: dict(
        name="c1_tiny_f32_bnsd", batch=2, n_q=4, n_kv=4, qk_dim=64, kv_dtype="f32",
        layout=LAYOUT_BNSD, lengths=128, s_cap=128, scale=1.0 / 8.0, num_splits=2,
    ),
    2: dict(
        name="c2_f16_gqa_bnsd_padded", batch=16, n_q=32, n_kv=8, qk_dim=128, kv_dtype="f16",
        layout=LAYOUT_BNSD, lengths=("uniform", 1, 4096), s_cap=4096,
    ),
    3: dict(
        name="c3_bf16_paged_gqa", batch=64, n_q=32, n_kv=8, qk_dim=128, kv_dtype="bf16",
        layout=LAYOUT_PAGED, block_size=128, lengths=("uniform", 512, 8192),
        max_blocks_per_seq=64, num_splits=4,
    ),
    4: dict(
        name="c4_i8_paged_antiquant_sink", batch=32, n_q=64, n_kv=8, qk_dim=128, kv_dtype="i8",
        q_dtype="bf16", out_dtype="bf16", layout=LAYOUT_PAGED, block_size=128, lengths=16384,
        max_blocks_per_seq=128, sink=True,
    ),
    5: dict(
        name="c5_mla_bf16_paged", batch=32, n_q=128, n_kv=1, qk_dim=576, v_dim=512, kv_dtype="bf16",
        layout=LAYOUT_PAGED, block_size=128, lengths=("uniform", 1024, 32768),
        max_blocks_per_seq=256, scale=1.0 / math.sqrt(192.0), v_aliases_k=True,
    ),
}


def config_workload(idx: int, seed: Optional[int] = None, device="cpu", poison=True, **overrides) -> Workload:
    """Workload for config ``idx`` (1..5); overrides shrink it for parity tests."""
    p = dict(CONFIGS[idx])
    p.update(overrides)
    if seed is None:
        seed = 1000 + idx
    return make_workload(seed=seed, device=device, poison=poison, **p)

"""Argument checks of the Python binding, run before anything is queued.

The C ABI sees only pointers and sizes, so a tensor whose shape disagrees with
the sizes passed beside it would turn into an out-of-bounds device access.
These pure-Python checks tie every tensor argument to the sizes the call
derives (batch, heads, head dims, block table, pool, outputs) and raise
``ValueError`` on any mismatch.  They touch no device memory and need no GPU:
``device_check=False`` skips only the "is a GPU tensor on the query's device"
part, for host-side tests.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

FLOAT_DTYPES = (torch.float32, torch.float16, torch.bfloat16)
KV_DTYPES = FLOAT_DTYPES + (torch.int8,)
LAYOUTS = ("paged", "paged_bsh", "bnsd", "bsnd")
MASK_NONE, MASK_CAUSAL, MASK_TREE = 0, 3, 9


@dataclasses.dataclass
class DecodeShape:
    """Sizes of one decode call, derived from its tensors."""

    batch: int
    q_seq: int
    multi: bool  # the query carries an explicit S_q axis
    n_q: int
    n_kv: int  # effective (numKeyValueHeads 0 means N_q)
    qk_dim: int
    v_dim: int
    alias: bool  # value_cache is key_cache (MLA: V = the first v_dim channels)
    layout: str
    paged: bool
    num_blocks: int
    block_size: int
    max_blocks: int
    s_cap: int
    out_dtype: torch.dtype
    antiquant_mode: str  # "", "channel", "tensor" or "token"

    @property
    def lead(self):
        return (self.batch, self.q_seq) if self.multi else (self.batch,)


def _need_tensor(t, name: str, device, device_check: bool, dtype=None, dtypes=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if device_check:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the query on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; supported: {', '.join(str(d) for d in dtypes)}")


def _shape(t, want, name):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def check_decode(q, k_cache, v_cache, block_table, actual_seq_lengths, num_heads: int, num_key_value_heads: int,
                 learnable_sink=None, antiquant_scale=None, antiquant_offset=None, v_dim: Optional[int] = None,
                 out_dtype: Optional[torch.dtype] = None, out=None, lse=None, kv_layout: Optional[str] = None,
                 sparse_mode: int = MASK_NONE, tree_mask=None, device_check: bool = True,
                 antiquant_mode: Optional[str] = None) -> DecodeShape:
    """Check every tensor of a decode call against the others; return its sizes.

    Layouts (aclnnIncreFlashAttentionV3 "Constraints", page attention
    scenario, and "Parameters"): "paged" (blocks, N_kv, block_size, D);
    "paged_bsh" (blocks, block_size, N_kv, D) or (blocks, block_size, N_kv*D);
    "bnsd" (B, N_kv, S, D); "bsnd" (B, S, N_kv, D) or (B, S, N_kv*D).
    """
    _need_tensor(q, "q", None, False, dtypes=FLOAT_DTYPES)
    device = q.device
    if device_check and not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    if q.dim() not in (3, 4):
        raise ValueError(f"q must be (B, N_q, D) or (B, S_q, N_q, D), got {tuple(q.shape)}")
    multi = q.dim() == 4
    B, q_seq, n_q, qk_dim = q.shape if multi else (q.shape[0], 1, q.shape[1], q.shape[2])
    B, q_seq, n_q, qk_dim = int(B), int(q_seq), int(n_q), int(qk_dim)
    if n_q != num_heads:
        raise ValueError(f"the query's head dimension ({n_q}) must equal num_heads ({num_heads})")
    if num_key_value_heads < 0 or num_key_value_heads > num_heads:
        raise ValueError("num_key_value_heads must be in [0, num_heads]")
    n_kv = num_heads if num_key_value_heads == 0 else int(num_key_value_heads)
    if num_heads % n_kv:
        raise ValueError("num_heads must be a multiple of num_key_value_heads")

    _need_tensor(k_cache, "k_cache", device, device_check, dtypes=KV_DTYPES)
    _need_tensor(v_cache, "v_cache", device, device_check, dtype=k_cache.dtype)
    _need_tensor(actual_seq_lengths, "actual_seq_lengths", device, device_check, dtype=torch.int64)
    _shape(actual_seq_lengths, (B,), "actual_seq_lengths")
    if k_cache.dtype != torch.int8 and k_cache.dtype != q.dtype:
        raise ValueError(f"a float KV cache must have the query dtype ({q.dtype}), got {k_cache.dtype}")

    alias = v_cache.data_ptr() == k_cache.data_ptr()
    if alias and v_cache.shape != k_cache.shape:
        raise ValueError("value_cache shares key_cache's memory with another shape")
    if kv_layout is None:
        kv_layout = "paged" if block_table is not None else "bnsd"
    if kv_layout not in LAYOUTS:
        raise ValueError(f"unknown kv_layout {kv_layout!r}")
    paged = kv_layout in ("paged", "paged_bsh")
    token_major = kv_layout in ("paged_bsh", "bsnd")

    if v_dim is None:
        if alias:
            v_dim = qk_dim
        elif token_major and v_cache.dim() == 3:  # (.., .., H): H = N_kv * v_dim
            v_dim = int(v_cache.shape[-1]) // n_kv
        else:
            v_dim = int(v_cache.shape[-1])
    v_dim = int(v_dim)
    if alias and v_dim > qk_dim:
        raise ValueError("with value_cache == key_cache, v_dim must not exceed the key row")

    def cache_dims(t, d, name):
        """(leading extent, per-token extent) of a cache, checked against N_kv and d."""
        if token_major and t.dim() == 3:
            if int(t.shape[2]) != n_kv * d:
                raise ValueError(f"{name} has H = {int(t.shape[2])}, expected N_kv * D = {n_kv * d}")
            return int(t.shape[0]), int(t.shape[1])
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D in the {kv_layout} layout, got {tuple(t.shape)}")
        if token_major:
            n0, s, nk, dd = (int(x) for x in t.shape)
        else:
            n0, nk, s, dd = (int(x) for x in t.shape)
        if nk != n_kv:
            raise ValueError(f"{name} holds {nk} KV heads, expected {n_kv}")
        if dd != d:
            raise ValueError(f"{name} rows hold {dd} channels, expected {d}")
        return n0, s

    n0, s = cache_dims(k_cache, qk_dim, "k_cache")
    if not alias:
        n0v, sv = cache_dims(v_cache, v_dim, "v_cache")
        if (n0v, sv) != (n0, s):
            raise ValueError("k_cache and v_cache disagree in their leading dimensions")
    if paged:
        if block_table is None:
            raise ValueError("the paged layouts need a block_table")
        _need_tensor(block_table, "block_table", device, device_check, dtype=torch.int32)
        if block_table.dim() != 2 or int(block_table.shape[0]) != B:
            raise ValueError(f"block_table must be (B={B}, max_blocks_per_seq), got {tuple(block_table.shape)}")
        num_blocks, block_size, max_blocks, s_cap = n0, s, int(block_table.shape[1]), 0
    else:
        if block_table is not None:
            raise ValueError(f"the contiguous {kv_layout} layout takes no block_table")
        if n0 != B:
            raise ValueError(f"the contiguous cache holds {n0} sequences, the query {B}")
        num_blocks = block_size = max_blocks = 0
        s_cap = s

    if learnable_sink is not None:
        _need_tensor(learnable_sink, "learnable_sink", device, device_check, dtype=torch.float32)
        _shape(learnable_sink, (num_heads,), "learnable_sink")

    aq_mode = ""
    if k_cache.dtype == torch.int8:
        if antiquant_scale is None or antiquant_offset is None:
            raise ValueError("an int8 KV cache needs antiquant_scale and antiquant_offset")
        _need_tensor(antiquant_scale, "antiquant_scale", device, device_check, dtype=torch.float32)
        _need_tensor(antiquant_offset, "antiquant_offset", device, device_check, dtype=torch.float32)
        if antiquant_offset.shape != antiquant_scale.shape:
            raise ValueError("antiquant_offset must have the shape of antiquant_scale")
        shp = tuple(antiquant_scale.shape)
        S = max_blocks * block_size if paged else s_cap  # logical positions of a sequence
        shapes = {"tensor": (2,), "channel": (2, n_kv, qk_dim), "token": (2, B, S), "token_head": (2, B, n_kv, S)}
        if antiquant_mode is None:  # by shape; per channel where (2, N_kv, D) and (2, B, S) coincide
            aq_mode = next((m for m in ("tensor", "channel", "token", "token_head") if shapes[m] == shp), None)
            if aq_mode is None:
                raise ValueError(f"antiquant parameters must be (2,), (2, N_kv={n_kv}, D={qk_dim}), "
                                 f"(2, B={B}, S={S}) or (2, B, N_kv, S), got {shp}")
        else:
            if antiquant_mode not in shapes:
                raise ValueError(f"unknown antiquant_mode {antiquant_mode!r}")
            if shp != shapes[antiquant_mode]:
                raise ValueError(f"antiquant_mode {antiquant_mode!r} needs parameters of shape "
                                 f"{shapes[antiquant_mode]}, got {shp}")
            aq_mode = antiquant_mode
        if aq_mode in ("token", "token_head") and qk_dim != 128:
            raise ValueError("per-token antiquant needs head dim 128")
    elif antiquant_scale is not None or antiquant_offset is not None or antiquant_mode is not None:
        raise ValueError("antiquant parameters are for an int8 KV cache only")

    if sparse_mode not in (MASK_NONE, MASK_CAUSAL, MASK_TREE):
        raise ValueError(f"sparse_mode {sparse_mode} not supported (0, 3 or 9)")
    if sparse_mode == MASK_TREE:
        if tree_mask is None:
            raise ValueError("sparse_mode 9 needs a tree_mask")
        _need_tensor(tree_mask, "tree_mask", device, device_check, dtype=torch.uint8)
        _shape(tree_mask, (B, q_seq, q_seq), "tree_mask")
    elif tree_mask is not None:
        raise ValueError("a tree_mask is used with sparse_mode 9 only")

    if out is not None:
        if out_dtype is None:
            out_dtype = out.dtype
        _need_tensor(out, "out", device, device_check, dtype=out_dtype)
    out_dtype = out_dtype or q.dtype
    if out_dtype not in FLOAT_DTYPES:
        raise ValueError(f"out_dtype {out_dtype} not supported")
    lead = (B, q_seq) if multi else (B,)
    if out is not None:
        _shape(out, lead + (num_heads, v_dim), "out")
    if lse is not None:
        _need_tensor(lse, "lse", device, device_check, dtype=torch.float32)
        _shape(lse, lead + (num_heads,), "lse")
    return DecodeShape(batch=B, q_seq=q_seq, multi=multi, n_q=num_heads, n_kv=n_kv, qk_dim=qk_dim, v_dim=v_dim,
                       alias=alias, layout=kv_layout, paged=paged, num_blocks=num_blocks, block_size=block_size,
                       max_blocks=max_blocks, s_cap=s_cap, out_dtype=out_dtype, antiquant_mode=aq_mode)


def check_update(prev_out, prev_max, prev_sum, cur_out, cur_max, cur_sum, out=None, max_out=None, sum_out=None,
                 device_check: bool = True):
    """Check the operands of attn_update (aclnnRingAttentionUpdate "参数说明"):
    outputs (..., D) of one float dtype and one shape; statistics fp32 with one
    value per row (optionally in a trailing dimension of size 1), or 8 copies
    of it in a trailing dimension of size 8.
    Returns (rows, head_dim, stat_stride)."""
    _need_tensor(prev_out, "prev_out", None, False, dtypes=FLOAT_DTYPES)
    device = prev_out.device
    if device_check and not prev_out.is_cuda:
        raise ValueError("prev_out must be a GPU tensor")
    if prev_out.dim() < 1:
        raise ValueError("prev_out must have a head dimension")
    D = int(prev_out.shape[-1])
    rows = prev_out.numel() // D if D else 0
    for t, nm in ((cur_out, "cur_out"), (out, "out")):
        if t is None:
            continue
        _need_tensor(t, nm, device, device_check, dtype=prev_out.dtype)
        _shape(t, prev_out.shape, nm)
    stats = [(prev_max, "prev_max"), (prev_sum, "prev_sum"), (cur_max, "cur_max"), (cur_sum, "cur_sum"),
             (max_out, "max_out"), (sum_out, "sum_out")]
    for t, nm in stats:
        if t is None:
            continue
        _need_tensor(t, nm, device, device_check, dtype=torch.float32)
        _shape(t, prev_max.shape, nm)
    lead = tuple(prev_out.shape[:-1])
    shp = tuple(prev_max.shape)
    if shp in (lead, lead + (1,)) or (rows and shp in ((rows,), (rows, 1))):
        stride = 1
    elif shp == lead + (8,) or (rows and shp == (rows, 8)):
        stride = 8
    else:
        raise ValueError(f"statistics of shape {shp} do not match outputs {tuple(prev_out.shape)}: "
                         f"expected {lead} or {lead + (8,)}")
    return rows, D, stride

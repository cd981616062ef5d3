"""Python binding of the MI355X decode-attention library (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/ifa_decode.h.  PyTorch provides device
memory (outputs and the workspace are torch tensors) and the stream (torch's
current stream).  There is no CPU fallback: without the built library every
call raises.

    out, lse = decode(q, k_cache, v_cache, block_table, actual_seq_lengths,
                      num_heads, num_key_value_heads, scale_value,
                      learnable_sink=None, antiquant_scale=None,
                      antiquant_offset=None, num_splits=0)

Layouts: q (B, N_q, D); paged KV pools (num_blocks, N_kv, block_size, D)
with block_table int32 (B, max_blocks_per_seq); or, with block_table None,
contiguous padded KV (B, N_kv, S_cap, D).  ``kv_layout="paged_bsh"`` takes
pools (num_blocks, block_size, N_kv * D) and ``kv_layout="bsnd"`` contiguous
(B, S_cap, N_kv * D).  Antiquant parameters of shape (2,) are per tensor.
For the MLA shape pass the same tensor as k_cache and v_cache and
``v_dim=512``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

from ._checks import check_decode, check_update

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libifa_decode.so")

IFA_OK = 0
IFA_ERR_PARAM_NULLPTR = 161001
IFA_ERR_PARAM_INVALID = 161002
IFA_ERR_RUNTIME = 361001
IFA_ERR_PLAN = 561002

IFA_F32, IFA_F16, IFA_BF16, IFA_I8 = 0, 1, 2, 3
IFA_KV_BNSD, IFA_KV_PAGED, IFA_KV_PAGED_BSH, IFA_KV_BSND = 0, 1, 2, 3
IFA_ANTIQUANT_PER_CHANNEL, IFA_ANTIQUANT_PER_TENSOR, IFA_ANTIQUANT_PER_TOKEN, IFA_ANTIQUANT_PER_TOKEN_HEAD = 0, 1, 2, 3
IFA_MASK_NONE, IFA_MASK_CAUSAL, IFA_MASK_TREE = 0, 3, 9
IFA_CHECK_BAD_LENGTH, IFA_CHECK_BAD_BLOCK = 1, 2
_LAYOUT_CODE = {"bnsd": IFA_KV_BNSD, "paged": IFA_KV_PAGED, "paged_bsh": IFA_KV_PAGED_BSH, "bsnd": IFA_KV_BSND}

_AQ_CODE = {"": 0, "channel": 0, "tensor": 1, "token": 2, "token_head": 3}

_DTYPE_CODE = {torch.float32: IFA_F32, torch.float16: IFA_F16, torch.bfloat16: IFA_BF16, torch.int8: IFA_I8}

# Every function the header declares.
EXPORTED = (
    "ifa_decode_workspace_size",
    "ifa_decode_num_splits",
    "ifa_decode_split_mode",
    "ifa_decode",
    "ifa_decode_noalloc",
    "ifa_decode_splitkv",
    "ifa_decode_splitkv_timed",
    "ifa_decode_combine",
    "attn_update",
    "ifa_kv_cache_write",
    "ifa_paged_block_count",
    "ifa_read_bandwidth_probe",
    "ifa_decode_check_inputs",
    "ifa_last_error",
)


class IfaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ifa status {status}: {message}")
        self.status = status


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("query", ctypes.c_void_p),
        ("key_cache", ctypes.c_void_p),
        ("value_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("actual_seq_lengths", ctypes.c_void_p),
        ("learnable_sink", ctypes.c_void_p),
        ("antiquant_scale", ctypes.c_void_p),
        ("antiquant_offset", ctypes.c_void_p),
        ("attention_out", ctypes.c_void_p),
        ("softmax_lse", ctypes.c_void_p),
        ("batch", ctypes.c_int64),
        ("num_heads", ctypes.c_int64),
        ("num_key_value_heads", ctypes.c_int64),
        ("qk_dim", ctypes.c_int64),
        ("v_dim", ctypes.c_int64),
        ("block_size", ctypes.c_int64),
        ("max_blocks_per_seq", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
        ("s_cap", ctypes.c_int64),
        ("scale_value", ctypes.c_double),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("antiquant_mode", ctypes.c_int32),
        ("q_seq_len", ctypes.c_int64),
        ("tree_mask", ctypes.c_void_p),
        ("sparse_mode", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"HIP library not built: {p} is missing (run attention_ifa_decode_amd.build)")
    lib = ctypes.CDLL(p)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    args_p = ctypes.POINTER(DecodeArgs)
    lib.ifa_decode_workspace_size.argtypes = [args_p, ctypes.POINTER(SZ)]
    lib.ifa_decode_num_splits.argtypes = [args_p, ctypes.POINTER(I32)]
    lib.ifa_decode_split_mode.argtypes = [args_p, ctypes.POINTER(I32)]
    for fn in (lib.ifa_decode, lib.ifa_decode_splitkv):
        fn.argtypes = [args_p, P, SZ, P]
    lib.ifa_decode_splitkv_timed.argtypes = [args_p, P, SZ, P, P, P]
    lib.ifa_decode_noalloc.argtypes = [args_p, P]
    lib.ifa_decode_combine.argtypes = [args_p, P, SZ, P]
    lib.attn_update.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I32, I32, P]
    lib.ifa_kv_cache_write.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, I64, I32, I32, P]
    lib.ifa_paged_block_count.argtypes = [ctypes.POINTER(I64), I64, I64]
    lib.ifa_paged_block_count.restype = I64
    lib.ifa_read_bandwidth_probe.argtypes = [P, SZ, P, I32, P]
    lib.ifa_decode_check_inputs.argtypes = [args_p, P, P]
    lib.ifa_last_error.argtypes = []
    lib.ifa_last_error.restype = ctypes.c_char_p
    for name in ("ifa_decode_workspace_size", "ifa_decode_num_splits", "ifa_decode_split_mode", "ifa_decode",
                 "ifa_decode_splitkv",
                 "ifa_decode_splitkv_timed", "ifa_decode_combine", "attn_update", "ifa_kv_cache_write",
                 "ifa_decode_noalloc", "ifa_decode_check_inputs",
                 "ifa_read_bandwidth_probe"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def last_error() -> str:
    return load_library().ifa_last_error().decode()


def _check(status: int):
    if status != IFA_OK:
        raise IfaError(status, last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


class DecodeCall:
    """A prepared decode call: argument struct, outputs and workspace.

    ``run()`` queues the split-KV kernel and the combine on the current stream;
    ``splitkv()`` and ``combine()`` queue the two halves separately.
    """

    def __init__(self, q, k_cache, v_cache, block_table, actual_seq_lengths, num_heads: int,
                 num_key_value_heads: int, scale_value: float, learnable_sink=None, antiquant_scale=None,
                 antiquant_offset=None, num_splits: int = 0, v_dim: Optional[int] = None,
                 out_dtype: Optional[torch.dtype] = None, with_lse: bool = True, out=None, lse=None,
                 kv_layout: Optional[str] = None, sparse_mode: int = IFA_MASK_NONE, tree_mask=None,
                 noalloc: bool = False, antiquant_mode: Optional[str] = None):
        lib = load_library()
        sh = check_decode(q, k_cache, v_cache, block_table, actual_seq_lengths, num_heads, num_key_value_heads,
                          learnable_sink, antiquant_scale, antiquant_offset, v_dim, out_dtype, out, lse, kv_layout,
                          sparse_mode, tree_mask, antiquant_mode=antiquant_mode)
        B, q_seq, n_q, qk_dim, v_dim = sh.batch, sh.q_seq, sh.n_q, sh.qk_dim, sh.v_dim
        kv_layout, out_dtype = sh.layout, sh.out_dtype
        num_blocks, block_size, max_blocks, s_cap = sh.num_blocks, sh.block_size, sh.max_blocks, sh.s_cap
        dev = q.device
        self.out = out if out is not None else torch.empty(sh.lead + (n_q, v_dim), dtype=out_dtype, device=dev)
        self.lse = lse if lse is not None else (
            torch.empty(sh.lead + (n_q,), dtype=torch.float32, device=dev) if with_lse else None)
        a = DecodeArgs()
        a.query = _ptr(q)
        a.key_cache = _ptr(k_cache)
        a.value_cache = _ptr(v_cache)
        a.block_table = _ptr(block_table)
        a.actual_seq_lengths = _ptr(actual_seq_lengths)
        a.learnable_sink = _ptr(learnable_sink)
        a.antiquant_scale = _ptr(antiquant_scale)
        a.antiquant_offset = _ptr(antiquant_offset)
        a.attention_out = _ptr(self.out)
        a.softmax_lse = _ptr(self.lse)
        a.batch = B
        a.num_heads = num_heads
        a.num_key_value_heads = num_key_value_heads
        a.qk_dim = qk_dim
        a.v_dim = v_dim
        a.block_size = block_size
        a.max_blocks_per_seq = max_blocks
        a.num_blocks = num_blocks
        a.s_cap = s_cap
        a.scale_value = float(scale_value)
        a.q_dtype = _DTYPE_CODE[q.dtype]
        a.kv_dtype = _DTYPE_CODE[k_cache.dtype]
        a.out_dtype = _DTYPE_CODE[out_dtype]
        a.kv_layout = _LAYOUT_CODE[kv_layout]
        a.num_splits = int(num_splits)
        a.antiquant_mode = _AQ_CODE[sh.antiquant_mode]
        a.q_seq_len = q_seq
        a.tree_mask = _ptr(tree_mask)
        a.sparse_mode = int(sparse_mode)
        a.reserved = 0
        self.args = a
        sz = ctypes.c_size_t(0)
        _check(lib.ifa_decode_workspace_size(ctypes.byref(a), ctypes.byref(sz)))
        ns = ctypes.c_int32(0)
        _check(lib.ifa_decode_num_splits(ctypes.byref(a), ctypes.byref(ns)))
        self.num_splits = ns.value
        bal = ctypes.c_int32(0)
        _check(lib.ifa_decode_split_mode(ctypes.byref(a), ctypes.byref(bal)))
        self.balanced = bool(bal.value)
        # partial outputs: fp16 on the MLA shape (qk_dim 576, v_dim 512), else fp32
        self.mla = qk_dim == 576 and v_dim == 512
        self.partial_dtype = torch.float16 if self.mla else torch.float32
        self.noalloc = noalloc
        if noalloc:  # partials in the library's fixed array (ifa_decode_noalloc)
            self.workspace_bytes, self.workspace = 0, None
        else:
            self.workspace_bytes = sz.value
            self.workspace = torch.empty(max(1, sz.value), dtype=torch.uint8, device=dev)
        # keep the inputs alive as long as the call object
        self._keep = (q, k_cache, v_cache, block_table, actual_seq_lengths, learnable_sink,
                      antiquant_scale, antiquant_offset, tree_mask)
        self.q_seq = q_seq
        self._lib = lib

    def run(self):
        if self.noalloc:
            _check(self._lib.ifa_decode_noalloc(ctypes.byref(self.args), _stream_handle()))
        else:
            _check(self._lib.ifa_decode(ctypes.byref(self.args), self.workspace.data_ptr(), self.workspace_bytes,
                                        _stream_handle()))
        return self.out, self.lse

    def check_inputs(self) -> torch.Tensor:
        """Queue the input check (ifa_decode_check_inputs) on the current
        stream; returns a one-element int32 GPU tensor holding, once the
        stream has run it, IFA_CHECK_BAD_LENGTH | IFA_CHECK_BAD_BLOCK bits for
        the lengths and block-table entries the decode would clamp (0: none)."""
        flags = torch.empty(1, dtype=torch.int32, device=self.out.device)
        _check(self._lib.ifa_decode_check_inputs(ctypes.byref(self.args), flags.data_ptr(), _stream_handle()))
        return flags

    def _ws(self) -> int:
        if self.noalloc:
            raise ValueError("a call made with noalloc=True has no workspace of its own")
        return self.workspace.data_ptr()

    def splitkv(self):
        _check(self._lib.ifa_decode_splitkv(ctypes.byref(self.args), self._ws(), self.workspace_bytes,
                                            _stream_handle()))

    def splitkv_timed(self, start: "torch.cuda.Event", stop: "torch.cuda.Event"):
        """splitkv() with `start` / `stop` (timing events of this device)
        recorded at the kernel's own start and end."""
        for e in (start, stop):
            if not e.cuda_event:  # torch creates the event at its first record
                e.record()
        _check(self._lib.ifa_decode_splitkv_timed(ctypes.byref(self.args), self._ws(), self.workspace_bytes,
                                                  _stream_handle(), start.cuda_event, stop.cuda_event))

    def combine(self):
        _check(self._lib.ifa_decode_combine(ctypes.byref(self.args), self._ws(), self.workspace_bytes,
                                            _stream_handle()))
        return self.out, self.lse

    def partials(self):
        """Views of the workspace after ``splitkv()``: (attn_out, softmax_max,
        softmax_sum) with shapes (B, N_q, n, v_dim), (B, N_q, n), (B, N_q, n),
        attn_out in ``partial_dtype`` (fp16 on the MLA shape, else fp32);
        with S_q query tokens B counts (sequence, query token) pairs.  The
        per-sequence split only; see ``partial_slots`` for the balanced one."""
        if self.balanced:
            raise ValueError("this call uses the balanced split: read its partials with partial_slots()")
        a = self.args
        B, nq, n, dv = a.batch * self.q_seq, a.num_heads, self.num_splits, a.v_dim
        f = self.workspace.view(torch.float32) if self.workspace_bytes else None
        rows = B * nq * n
        al = lambda x: (x + 255) // 256 * 256  # noqa: E731
        ob = 2 if self.mla else 4  # attn_out fp16 on the MLA shape
        off_m = al(rows * dv * ob) // 4
        off_l = off_m + al(rows * 4) // 4
        o = self.workspace.view(self.partial_dtype)[:rows * dv].view(B, nq, n, dv)
        return (o, f[off_m:off_m + rows].view(B, nq, n), f[off_l:off_l + rows].view(B, nq, n))

    def partial_slots(self):
        """Views of the workspace after ``splitkv()`` with the balanced split:
        (attn_out (n + B, S_q * N_q, v_dim) in ``partial_dtype``, softmax_max (n + B, S_q * N_q),
        softmax_sum (n + B, S_q * N_q), (first slot, slot count) int32 (B, 2));
        run r's piece of sequence b is slot r + b, and query token t of head h
        is row t * N_q + h of a slot."""
        if not self.balanced:
            raise ValueError("this call splits per sequence: read its partials with partials()")
        a = self.args
        B, nq, dv = a.batch, self.q_seq * a.num_heads, a.v_dim
        slots = self.num_splits + B
        f = self.workspace.view(torch.float32)
        rows = slots * nq
        al = lambda x: (x + 255) // 256 * 256  # noqa: E731
        ob = 2 if self.mla else 4  # attn_out fp16 on the MLA shape
        off_m = al(rows * dv * ob) // 4
        off_l = off_m + al(rows * 4) // 4
        off_p = off_l + al(rows * 4) // 4
        desc = self.workspace.view(torch.int32)[off_p:off_p + 2 * B].view(B, 2)
        o = self.workspace.view(self.partial_dtype)[:rows * dv].view(slots, nq, dv)
        return (o, f[off_m:off_m + rows].view(slots, nq), f[off_l:off_l + rows].view(slots, nq), desc)


def decode(q, k_cache, v_cache, block_table, actual_seq_lengths, num_heads: int, num_key_value_heads: int,
           scale_value: float, learnable_sink=None, antiquant_scale=None, antiquant_offset=None,
           num_splits: int = 0, v_dim: Optional[int] = None,
           out_dtype: Optional[torch.dtype] = None, kv_layout: Optional[str] = None,
           sparse_mode: int = IFA_MASK_NONE, tree_mask=None,
           antiquant_mode: Optional[str] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode attention; returns (attention_out (B, N_q, v_dim), softmax_lse (B, N_q) fp32).
    kv_layout: "paged" (default with a block table), "paged_bsh", "bnsd"
    (default without one) or "bsnd"; antiquant parameters of shape (2,) are
    per tensor.  A query of shape (B, S_q, N_q, D) decodes S_q tokens per
    sequence (the last S_q of its length) under ``sparse_mode`` (IFA_MASK_NONE,
    IFA_MASK_CAUSAL, or IFA_MASK_TREE with ``tree_mask`` uint8 (B, S_q, S_q));
    then out is (B, S_q, N_q, v_dim) and lse (B, S_q, N_q).  int8 antiquant
    parameters are per tensor (2,), per channel (2, N_kv, D), per token
    (2, B, S) or per token and KV head (2, B, N_kv, S), S the logical
    capacity; ``antiquant_mode`` ("channel", "tensor", "token", "token_head")
    names the mode where shapes coincide."""
    call = DecodeCall(q, k_cache, v_cache, block_table, actual_seq_lengths, num_heads, num_key_value_heads,
                      scale_value, learnable_sink, antiquant_scale, antiquant_offset, num_splits, v_dim,
                      out_dtype, kv_layout=kv_layout, sparse_mode=sparse_mode, tree_mask=tree_mask,
                      antiquant_mode=antiquant_mode)
    out, lse = call.run()
    # the workspace must outlive the queued kernels: the caching allocator
    # keeps it reserved for this stream
    call.workspace.record_stream(torch.cuda.current_stream())
    return out, lse


def attn_update(prev_out, prev_max, prev_sum, cur_out, cur_max, cur_sum, out=None, max_out=None,
                sum_out=None):
    """RingAttentionUpdate of two results.  *_out: (rows, D) or (..., D);
    *_max / *_sum: fp32 with one value per row, optionally repeated 8 times in
    a trailing dimension of size 8.  Returns (attn_out, softmax_max,
    softmax_sum); outputs may alias inputs."""
    lib = load_library()
    rows, D, stride = check_update(prev_out, prev_max, prev_sum, cur_out, cur_max, cur_sum, out, max_out, sum_out)
    out = out if out is not None else torch.empty_like(prev_out)
    max_out = max_out if max_out is not None else torch.empty_like(prev_max)
    sum_out = sum_out if sum_out is not None else torch.empty_like(prev_sum)
    _check(lib.attn_update(prev_out.data_ptr(), prev_max.data_ptr(), prev_sum.data_ptr(), cur_out.data_ptr(),
                           cur_max.data_ptr(), cur_sum.data_ptr(), out.data_ptr(), max_out.data_ptr(),
                           sum_out.data_ptr(), rows, D, _DTYPE_CODE[prev_out.dtype], stride,
                           _stream_handle()))
    return out, max_out, sum_out


def kv_cache_write(src, slot_index, cache, layout: str = "paged_bsh", col_offset: int = 0):
    """Write new K/V rows into a paged pool in place (the step before a
    decode step): src (T, N_kv, d) rows go to the slots slot_index (T) int64
    of ``cache``, "paged_bsh" (num_blocks, block_size, N_kv, W) or "paged"
    (num_blocks, N_kv, block_size, W), at channels col_offset .. col_offset
    + d - 1.  Slots outside the pool are skipped.  Returns ``cache``."""
    lib = load_library()
    if layout not in ("paged", "paged_bsh"):
        raise ValueError("layout must be 'paged' or 'paged_bsh'")
    _need(src, "src", cache.dtype)
    _need(slot_index, "slot_index", torch.int64)
    _need(cache, "cache", cache.dtype)
    T, n_kv, d = src.shape
    if layout == "paged_bsh":
        num_blocks, block_size, n_kv_c, w = cache.shape
    else:
        num_blocks, n_kv_c, block_size, w = cache.shape
    if n_kv_c != n_kv or slot_index.numel() != T:
        raise ValueError("src, slot_index and cache disagree")
    _check(lib.ifa_kv_cache_write(src.data_ptr(), slot_index.data_ptr(), cache.data_ptr(), T, n_kv, d, w,
                                  int(col_offset), num_blocks, block_size, _LAYOUT_CODE[layout],
                                  _DTYPE_CODE[cache.dtype], _stream_handle()))
    return cache


def read_bandwidth_probe(buf: torch.Tensor, workgroups: int = 4096) -> torch.Tensor:
    """Queue one read of every byte of ``buf`` (a contiguous GPU tensor of
    16-byte aligned size) on the current stream; returns the per-workgroup
    words the probe writes.  For measuring the device's read rate."""
    lib = load_library()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    out = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    _check(lib.ifa_read_bandwidth_probe(buf.data_ptr(), nbytes, out.data_ptr(), int(workgroups), _stream_handle()))
    return out


def paged_block_count(lengths, block_size: int) -> int:
    """Pool size sum_b ceil(L_b / block_size) (host helper of the C ABI)."""
    lib = load_library()
    vals = [int(x) for x in lengths]
    arr = (ctypes.c_int64 * max(1, len(vals)))(*vals)
    r = lib.ifa_paged_block_count(arr, len(vals), int(block_size))
    if r < 0:
        raise ValueError("invalid lengths or block_size")
    return r


def decode_workload(w, num_splits: Optional[int] = None, **kw):
    """Convenience: decode a synthetic workload object on its device."""
    return decode(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.n_q, w.n_kv, w.scale,
                  learnable_sink=w.sink, antiquant_scale=w.antiquant_scale, antiquant_offset=w.antiquant_offset,
                  num_splits=w.num_splits if num_splits is None else num_splits,
                  v_dim=w.v_dim, out_dtype=w.out_dtype, kv_layout=w.layout,
                  antiquant_mode=getattr(w, "antiquant_mode", None), **kw)


def call_for_workload(w, num_splits: Optional[int] = None, **kw) -> DecodeCall:
    return DecodeCall(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.n_q, w.n_kv, w.scale,
                      learnable_sink=w.sink, antiquant_scale=w.antiquant_scale,
                      antiquant_offset=w.antiquant_offset,
                      num_splits=w.num_splits if num_splits is None else num_splits, v_dim=w.v_dim,
                      out_dtype=w.out_dtype, kv_layout=w.layout, antiquant_mode=getattr(w, "antiquant_mode", None),
                      **kw)

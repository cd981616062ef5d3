"""GPU check of ifa_decode_noalloc, the entry point for callers that cannot
allocate: called through the C ABI, its output must equal ifa_decode's (same
kernels, same split plan, partials in the library's fixed array instead of a
caller workspace), bit for bit, on calls in a row, the last three each
smaller than the one before, so that contents the array keeps from a larger
call cannot leak into a smaller one."""

import ctypes

import pytest
import torch

import attention_ifa_decode_amd as ifa
from synth import config_workload, make_workload

pytestmark = pytest.mark.gpu


def _pair(w):
    """(ifa_decode result, ifa_decode_noalloc result) for one workload."""
    wg = w.to("cuda")
    ref = ifa.call_for_workload(wg)
    ref.run()
    na = ifa.call_for_workload(wg, noalloc=True)
    na.out.fill_(float("nan"))
    na.lse.fill_(float("nan"))
    lib = ifa.load_library()
    st = lib.ifa_decode_noalloc(ctypes.byref(na.args), torch.cuda.current_stream().cuda_stream)
    assert st == ifa.IFA_OK, ifa.last_error()
    torch.cuda.synchronize()
    return (ref.out, ref.lse), (na.out, na.lse)


def _same(a, b):
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.view(torch.int16) if o1.dtype != torch.float32 else o1,
                       o2.view(torch.int16) if o2.dtype != torch.float32 else o2)
    assert torch.equal(l1, l2)


def test_noalloc_equals_ifa_decode_on_shrinking_calls():
    calls = [
        # the paged bf16 GQA workload, reduced: 4 splits, 12 sequences
        config_workload(3, seed=700, batch=12, lengths=("uniform", 512, 4000), max_blocks_per_seq=32),
        # the MLA shape (balanced split: slot-indexed partials and the plan region)
        config_workload(5, seed=701, batch=3, lengths=[3000, 1100, 40], max_blocks_per_seq=24),
        # smaller again: int8 K/V with antiquant and a sink
        config_workload(4, seed=702, batch=2, lengths=[300, 1], max_blocks_per_seq=3),
        # smallest: fp32 contiguous, the tiny config
        config_workload(1, seed=703),
    ]
    sizes = []
    for w in calls:
        print(f"[gpu case] noalloc {w.name} B={w.batch} lens={w.lengths()}", flush=True)
        a, b = _pair(w)
        _same(a, b)
        sizes.append(ifa.call_for_workload(w.to("cuda")).workspace_bytes)
    # the MLA call's partials are the largest; the calls after it shrink
    assert sizes[1] > max(sizes[0], sizes[2]) and sizes[2] > sizes[3] > 0


def test_noalloc_rejects_calls_beyond_its_array():
    """The MLA shape with 256 splits per sequence over 40 sequences needs more
    partials than the fixed array holds: IFA_ERR_PLAN, nothing queued."""
    w = make_workload(batch=40, n_q=128, n_kv=1, qk_dim=576, v_dim=512, kv_dtype="bf16", layout="paged",
                      block_size=128, lengths=[20] * 40, v_aliases_k=True, seed=704, device="cuda")
    call = ifa.call_for_workload(w, num_splits=256)
    assert call.workspace_bytes > (128 << 20)
    na = ifa.call_for_workload(w, num_splits=256, noalloc=True)
    with pytest.raises(ifa.IfaError) as e:
        na.run()
    assert e.value.status == ifa.IFA_ERR_PLAN and "scratch" in str(e.value)

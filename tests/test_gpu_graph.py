"""GPU: the decode captured in a HIP graph (torch.cuda.graph) gives, on every
replay, exactly the output of the same call made eagerly.  The library only
launches kernels on the caller's stream (no allocation, no memset), so a
captured step replays as is.  Each replay is checked separately, with eager
work and synchronisations between replays and fresh inputs copied into the
captured buffers before some of them."""

import pytest
import torch

import attention_ifa_decode_amd as ifa
from synth import config_workload, make_workload

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


@pytest.mark.parametrize("cfg", ["c2", "c3", "c5", "i8_token"])
def test_graph_replays_equal_eager(cfg):
    if cfg == "c2":
        w = config_workload(2, seed=210, batch=6, lengths=("uniform", 1, 900), s_cap=1024)
    elif cfg == "c3":
        w = config_workload(3, seed=310, batch=8, lengths=("uniform", 200, 1500), max_blocks_per_seq=12)
    elif cfg == "c5":
        w = config_workload(5, seed=510, batch=3, lengths=[1500, 600, 33], max_blocks_per_seq=12)
    else:
        w = make_workload(batch=4, n_q=16, n_kv=4, qk_dim=128, kv_dtype="i8", layout="paged", block_size=32,
                          lengths=[300, 31, 700, 2], seed=511, sink=True, antiquant_mode="token")
    print(f"[gpu case] graph replay {cfg}", flush=True)
    wg = w.to("cuda")
    call = ifa.call_for_workload(wg)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call.run()
    torch.cuda.synchronize()
    q0 = wg.q.clone()
    for rep in range(4):
        if rep == 2:  # new query values in the captured buffer
            wg.q.copy_(torch.randn(q0.shape, device="cuda").to(q0.dtype))
        ref = ifa.call_for_workload(wg)  # eager, its own workspace
        ro, rl = ref.run()
        torch.cuda.synchronize()
        call.out.fill_(float("nan"))
        call.lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(call.out), _bits(ro)), f"replay {rep}: output differs from eager"
        assert torch.equal(call.lse, rl), f"replay {rep}: lse differs from eager"
        _ = (wg.q.float() * 2).sum().item()  # unrelated eager work between replays

"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]
                    [--num-splits N] [--kv-layout L] [--q-seq S --mask M]
                    [--no-cpu-baseline] [--no-read-ceiling] [--reps R] [--graph]

One step = one pass of the whole path over one batch: the split-KV decode
kernel (block-table gather, QK^T, online softmax, PV, partial triples) and the
combine kernel (n-way merge, sink, output cast, lse).  Inputs are synthetic,
seeded and resident in HBM before timing starts.  The default workload is the
paged bf16 GQA decode: B=64, N_q=32, N_kv=8, D=128, block size 128, lengths
U[512, 8192], 4 KV splits.  ``--kv-layout`` measures the same workload with
its cache in another layout (paged_bsh: (blocknum, blocksize, H) pool; bsnd:
contiguous (B, S, H)).  ``--q-seq S`` decodes S query tokens per sequence
(speculative verification) under ``--mask`` none / causal / tree (a seeded
random tree over the S draft tokens); ``value`` still counts each KV byte once.

Prints one JSON line.  ``value`` is KV-cache GB/s: the bytes of K and V that
belong to valid tokens, per step, divided by the mean step time of the timed
region (K plain ifa_decode calls, events only around the loop).  ``step_us``
adds the median, p10 and p90 of 100 steps timed one by one.  ``roofline``
relates the split-KV kernel's own average duration (HIP events that the
runtime records at the start and end of the kernel, hipExtLaunchKernel, over
100 launches in a loop after the timed region) to the 8 TB/s HBM peak and to
the read rate of this device measured in the same run (a probe kernel reading
a 4 GiB buffer).  ``cpu_baseline`` times the float64 oracle on a bounded
sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
MALL_BYTES = 256 << 20
# kernel sources of each split-KV kernel, hashed so that stored counter
# readings are used only while the kernel code they were taken on is unchanged
GQA_MFMA_SOURCES = ["attention_ifa_decode_amd/csrc/decode_spec.hip", "attention_ifa_decode_amd/csrc/common.hpp"]
MLA_SOURCES = ["attention_ifa_decode_amd/csrc/decode_mla.hip", "attention_ifa_decode_amd/csrc/common.hpp"]
# HBM counter summaries per workload (in its own layout and query length)
TRAFFIC_FILES = {
    2: ("gqa_mfma_c2_f16_bnsd_traffic.txt", GQA_MFMA_SOURCES),
    3: ("gqa_mfma_c3_bf16_paged_traffic.txt", GQA_MFMA_SOURCES),
    4: ("gqa_mfma_c4_i8_paged_sink_traffic.txt", GQA_MFMA_SOURCES),
    5: ("mla_splitkv_c5_bf16_paged_traffic.txt", MLA_SOURCES),
}


# SQ / GRBM counter summaries (MFMA busy fraction, VALU issue fraction) per workload
COUNTER_FILES = {
    3: ("gqa_mfma_c3_bf16_paged_sq_counters.txt", GQA_MFMA_SOURCES),
    4: ("gqa_mfma_c4_i8_paged_sink_sq_counters.txt", GQA_MFMA_SOURCES),
    5: ("mla_splitkv_c5_bf16_paged_sq_counters.txt", MLA_SOURCES),
}


def kernel_source_hash(sources=GQA_MFMA_SOURCES) -> str:
    """Hash of the split-KV kernel's source with comments and whitespace
    removed, so that only a change to the code itself invalidates the stored
    counter readings."""
    import re

    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()[:16]


def kernel_name(w) -> str:
    """The split-KV kernel a workload runs: MLA shape on MFMA, 16-bit or int8
    K/V with head dim 128 on the MFMA GQA kernel, the rest on the VALU kernel."""
    import torch

    if w.qk_dim == 576:
        return "mla_splitkv_kernel"
    if w.qk_dim == 128 and w.kv_dtype in (torch.float16, torch.bfloat16, torch.int8):
        return "gqa_mfma_kernel"
    return "gqa_splitkv_kernel"


def read_traffic(config_idx: int):
    """HBM bytes per launch of the split-KV kernel from the committed counter
    summary, or None if absent or taken on a different kernel source."""
    if config_idx not in TRAFFIC_FILES:
        return None
    name, sources = TRAFFIC_FILES[config_idx]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _summary_fields(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip().split()[0] if v.strip() else ""
    return kv


def read_counters(config_idx: int):
    """MFMA busy and VALU issue fractions of the split-KV kernel from the
    committed SQ counter summary, or None if absent or taken on a different
    kernel source."""
    if config_idx not in COUNTER_FILES:
        return None
    name, sources = COUNTER_FILES[config_idx]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = _summary_fields(path)
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return {"mfma_busy_frac": float(kv["mfma_busy_frac"]), "valu_issue_frac": float(kv["valu_issue_frac"]),
                "source": "profiles/" + name}
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 15.0):
    """The float64 oracle on the host cores: whole sequences (all heads),
    from the first one on, spread over one worker thread per core this
    process may run on (os.sched_getaffinity, at most OMP_NUM_THREADS or 16)
    with single-threaded BLAS, so
    that the core count reported is the number of threads that computed.  The
    oracle's array operations release the interpreter lock; the sample is
    sized so that the run takes about ``budget_s`` seconds."""
    import concurrent.futures as cf

    import oracle

    # one thread per core this process may run on, within the host share the
    # run is given (OMP_NUM_THREADS, else 16)
    cores = max(1, min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    wc = w.to("cpu")
    lens = wc.lengths()
    esz = wc.k_cache.element_size()
    per_tok = wc.n_kv * wc.qk_dim * esz + (0 if wc.v_aliases_k else wc.n_kv * wc.v_dim * esz)

    def one(b):
        return oracle.decode_workload(wc, rows=[(b, h) for h in range(wc.n_q)])

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx is not None:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()  # calibration: the first sequence on one thread
        one(0)
        t1 = time.perf_counter() - t0
        rate = max(lens[0], 1) / max(t1, 1e-6)  # tokens (all heads) per second and thread
        sample, tok = [], 0
        for b in range(wc.batch):
            if tok / (rate * cores * 0.7) > budget_s:
                break
            sample.append(b)
            tok += lens[b]
        # whole passes over the sample until about 3 s have passed (at most 20),
        # so that a small workload is still timed over a measurable span
        order = sorted(sample, key=lambda b: -lens[b])
        passes = 0
        with cf.ThreadPoolExecutor(max_workers=cores) as ex:
            t0 = time.perf_counter()
            while True:
                list(ex.map(one, order))
                passes += 1
                if passes >= 20 or time.perf_counter() - t0 > 3.0:
                    break
            dt = (time.perf_counter() - t0) / passes
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {
        "value": round(tok * per_tok / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"sequences {sample[0]}..{sample[-1]} ({len(sample)} of {wc.batch}, {tok} tokens, all heads), "
                  f"{dt:.2f} s per pass of float64 NumPy on {cores} threads (one per core, BLAS single-threaded), "
                  f"mean of {passes} passes",
        "cpu_model": _cpu_model(),
        "seconds": round(dt, 3),
        "qtok_per_s": round(len(sample) / dt, 3),
    }


def _pct(xs, p):
    xs = sorted(xs)
    k = min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))
    return xs[k]


def read_ceiling(ifa, torch, dev, gib: int = 4):
    """HBM read rate of this device: the probe kernel over a buffer far larger
    than the 256 MB Infinity Cache, best of a few launch shapes, median of
    5 reads each."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    best = 0.0
    for wg in (2048, 4096, 8192):
        ifa.read_bandwidth_probe(buf, wg)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ifa.read_bandwidth_probe(buf, wg)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        best = max(best, buf.numel() / (sorted(ts)[2] * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the clock of the matrix-core-heavy workload settles over 10-20 ms of load")
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--kv-layout", default=None, choices=["paged", "paged_bsh", "bnsd", "bsnd"],
                    help="cache layout instead of the config's own (paged <-> paged_bsh, bnsd <-> bsnd)")
    ap.add_argument("--q-seq", type=int, default=1, help="query tokens per sequence (1..16)")
    ap.add_argument("--mask", default="causal", choices=["none", "causal", "tree"])
    ap.add_argument("--antiquant-mode", default=None, choices=["channel", "tensor", "token", "token_head"],
                    help="int8 workloads: where the antiquant scale and offset vary (default: the config's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--reps", type=int, default=100, help="reps of the step-median and kernel-time loops")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of a captured HIP graph (one step per input copy)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first, so that HBM byte "
                         "counters can be scaled against a transfer of known size")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by batch, KV head or sequence; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_ifa_decode_amd as ifa
    from synth import config_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    over = {} if args.kv_layout is None else {"layout": args.kv_layout}
    if args.antiquant_mode is not None:
        over["antiquant_mode"] = args.antiquant_mode
    w = config_workload(args.config, seed=args.seed, device=dev, **over)
    if args.antiquant_mode is not None and w.kv_dtype != torch.int8:
        sys.exit("--antiquant-mode applies to int8 K/V workloads (config 4)")
    kv_bytes = w.kv_bytes()
    # enough independent copies that the 256 MB infinity cache never serves KV
    copies = 1 if kv_bytes > 3 * MALL_BYTES else min(4, -(-3 * MALL_BYTES // max(kv_bytes, 1)))
    # the copies share the workload's lengths, block table and poisoned slots
    # (its seed) and differ in their values only
    seed = args.seed if args.seed is not None else 1000 + args.config
    works = [w] + [config_workload(args.config, seed=seed, value_seed=seed + 1 + 17 * i, device=dev, **over)
                   for i in range(1, copies)]
    modes = {"none": ifa.IFA_MASK_NONE, "causal": ifa.IFA_MASK_CAUSAL, "tree": ifa.IFA_MASK_TREE}

    def make_call(x, i):
        if args.q_seq == 1:
            return ifa.call_for_workload(x, num_splits=args.num_splits)
        # S_q query tokens per sequence; the tree keeps each draft token's own position
        g = torch.Generator(device=dev).manual_seed(7000 + i)
        q4 = torch.randn((x.batch, args.q_seq, x.n_q, x.qk_dim), generator=g, device=dev).to(x.q.dtype)
        tm = None
        if args.mask == "tree":
            tm = (torch.rand((x.batch, args.q_seq, args.q_seq), generator=g, device=dev) < 0.5).to(torch.uint8)
            tm *= 1 - torch.eye(args.q_seq, dtype=torch.uint8, device=dev)
        return ifa.DecodeCall(q4, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.n_q, x.n_kv, x.scale,
                              learnable_sink=x.sink, antiquant_scale=x.antiquant_scale,
                              antiquant_offset=x.antiquant_offset,
                              num_splits=x.num_splits if args.num_splits is None else args.num_splits,
                              v_dim=x.v_dim, out_dtype=x.out_dtype, kv_layout=x.layout,
                              sparse_mode=modes[args.mask], tree_mask=tm, antiquant_mode=x.antiquant_mode)

    calls = [make_call(x, i) for i, x in enumerate(works)]

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        calls[i % copies].run()
    torch.cuda.synchronize()

    # The timed region: K whole steps (ifa_decode: the split-KV kernel, then
    # the combine), plain calls on the stream, events only around the loop.
    # With --graph the K steps are replays of one captured HIP graph that
    # holds `copies` steps (one per input copy), so the host does not pace
    # small workloads.
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for c in calls:
                c.run()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in calls:
                c.run()
        torch.cuda.synchronize()
        K = -(-K // copies) * copies  # whole replays
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t_start.record(stream)
    if graph is not None:
        for _ in range(K // copies):
            graph.replay()
    else:
        for i in range(K):
            calls[i % copies].run()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / K

    # Step distribution: R steps, each between two events on the stream
    # (median, p10, p90).
    R = max(args.reps, 1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(R):
        calls[i % copies].run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(R)]

    # The split-KV kernel's own duration: R more steps whose split-KV launch
    # records a pair of events at the kernel's start and end
    # (hipExtLaunchKernel).  Those events delay the next dispatch, which is
    # why they stay out of the timed region above.
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(R)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(R)]
    for e in ev_a + ev_b:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(R):
        c = calls[i % copies]
        c.splitkv_timed(ev_a[i], ev_b[i])
        c.combine()
    torch.cuda.synchronize()
    kern = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
    kern_ms = sum(kern) / R

    ceiling = None if args.no_read_ceiling else read_ceiling(ifa, torch, dev)

    achieved = kv_bytes / (kern_ms * 1e-3) / 1e9
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    # algorithmic flops: QK^T and PV for every valid token and query head
    flops = sum(w.lengths()) * w.n_q * args.q_seq * 2 * (w.qk_dim + w.v_dim)  # masked tokens counted too
    default_shape = args.kv_layout is None and args.q_seq == 1 and args.antiquant_mode is None
    traffic = read_traffic(args.config) if default_shape else None
    dtype_name = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.int8: "i8"}
    lens = w.lengths()
    result = {
        "metric": "Paged decode attention: KV-cache HBM GB/s (% of MI355X peak) and query tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name[w.kv_dtype],
        "data": "synthetic",
        "qtok_per_s": round(w.batch * args.q_seq / (ms_step * 1e-3), 1),
        "step_us": {"mean": round(ms_step * 1e3, 2), "median": round(_pct(step_ms, 50) * 1e3, 2),
                    "p10": round(_pct(step_ms, 10) * 1e3, 2), "p90": round(_pct(step_ms, 90) * 1e3, 2),
                    "reps": R, "step_frac_of_peak": round(kv_bytes / (_pct(step_ms, 50) * 1e-3) / 1e9
                                                          / HBM_PEAK_GBS, 4)},
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "num_heads": w.n_q,
            "num_kv_heads": w.n_kv,
            "qk_dim": w.qk_dim,
            "v_dim": w.v_dim,
            "kv_layout": w.layout,
            "block_size": w.block_size,
            "seq_len_mean": round(sum(lens) / len(lens), 1),
            "seq_len_range": [min(lens), max(lens)],
            "num_splits": calls[0].num_splits,
            "q_seq_len": args.q_seq,
            "mask": args.mask if args.q_seq > 1 else "none",
            "antiquant_mode": w.antiquant_mode if w.kv_dtype == torch.int8 else None,
            "kv_bytes_per_step": kv_bytes,
            "input_copies": copies,
            "timed_as": "HIP graph replays" if args.graph else "plain ifa_decode calls",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name(w),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_us": round(kern_ms * 1e3, 2),
            "kernel_us_median": round(_pct(kern, 50) * 1e3, 2),
            "kernel_timing": f"mean of {R} launches, events recorded at the split-KV kernel's own start and end "
                             "(hipExtLaunchKernel), in a loop after the timed region",
            "combine_and_gaps_us": round((ms_step - kern_ms) * 1e3, 2),
            "read_ceiling_gbs": None if ceiling is None else round(ceiling, 1),
            "frac_of_read_ceiling": None if ceiling is None else round(achieved / ceiling, 4),
            "flops_per_launch": flops,
            "counters": read_counters(args.config) if default_shape else None,
            "mfma_tflops": round(flops / (kern_ms * 1e-3) / 1e12, 2) if w.qk_dim == 576 else None,
            "mfma_frac_bf16_dense": round(flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
            if w.qk_dim == 576 else None,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.q_seq == 1:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

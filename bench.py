#!/usr/bin/env python3
"""Benchmark of the batched speculative-decoding verify on one MI355X.

Workload: B=64 requests, k=6 drafts, V=128256, bf16 logits (32 greedy,
16 one-hot-draft sampled, 16 draft-logit sampled requests; synthetic, seeded).
A step is one call of the whole verify (every kernel of the path) on one
batch.  Inputs are resident in HBM before the timed region; R rotating copies
of the inputs (sized to three times the 256 MB Infinity Cache) make every step
read from HBM rather than from the cache.

Prints one JSON line: verify rows/s (the value), tokens committed/s, achieved
algorithmic HBM bandwidth against the 8 TB/s peak, and the fp64 CPU oracle
timed on the host (the cpu_baseline leg, which also checks the GPU outputs of
the timed data against the oracle).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 << 20
METRIC = "verify rows/sec + achieved HBM GB/s, B=64 k=6 V=128256 bf16 sampled"
KERNEL_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                          "lossless_rejection_sampling_spec_amd", "csrc", "specverify.hip")

# HBM bytes per verify launch on this workload, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
# counter reads for a copy kernel of known size in the same run (the input
# clones: FETCH_SIZE reads 0.5x the bytes copied, WRITE_SIZE 1.0x).  Keyed by
# the SHA-256 of the kernel source the counters were taken on: for any other
# source the figure is stale and the bench reports null.
TRAFFIC_BYTES = {
    # 71818.4 KiB fetched x 1.99920, 343.6 KiB written: 1.056x the algorithmic bytes
    "5bc33a8f72dc453088e0967b922118bbe14e6d9160d873d609cc25c7c34df854": 147376862,
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions; the median is reported")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the steps from a captured HIP graph")
    return ap.parse_args()


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this verify benchmark runs on exactly one GPU (--gpus 1); the batch "
              "shards across GPUs with no communication, so per-GPU throughput is the figure",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from lossless_rejection_sampling_spec_amd import binding, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()                       # fails loudly without the HIP library

    w = synth.make(2, seed=args.seed)
    rows = w.total_rows
    alg_bytes = synth.algorithmic_bytes(w)
    R = max(2, math.ceil(3 * MALL_BYTES / alg_bytes))

    base = binding.workload_tensors(w, dev)
    copies = [base]
    for _ in range(R - 1):
        copies.append({k: (None if v is None else v.clone()) for k, v in base.items()})
    B = w.batch
    n_draft = rows - B
    outs = (torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(rows, dtype=torch.int32, device=dev),
            torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(n_draft, dtype=torch.float32, device=dev),
            torch.empty(n_draft, dtype=torch.float32, device=dev))
    ws = binding.get_workspace(dev, binding.workspace_bytes(B, rows, w.vocab, w.max_k))

    L = binding.lib()
    stream = torch.cuda.current_stream(dev)

    def args_for(t):
        return (t["target"].data_ptr(), binding.SV_BF16, t["target"].stride(0),
                t["draft"].data_ptr(), binding.SV_BF16, t["draft"].stride(0),
                t["draft_kind"].data_ptr(), t["cu_seqlens"].data_ptr(),
                t["draft_tokens"].data_ptr(), t["uniforms"].data_ptr(),
                t["temperature"].data_ptr(), None, None, B, rows, w.max_k, w.vocab,
                outs[0].data_ptr(), outs[1].data_ptr(), outs[3].data_ptr(), outs[4].data_ptr(),
                outs[2].data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream)

    call_args = [args_for(t) for t in copies]
    fn = L.spec_verify_sampled

    def step(i):
        rc = fn(*call_args[i % R])
        if rc != 0:
            raise RuntimeError(binding.status_string(rc))

    graph = None
    if args.graph:
        s = torch.cuda.Stream(dev)
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            step(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            cap_args = [list(a) for a in call_args]
            for a in cap_args:
                a[-1] = s.cuda_stream
                rc = fn(*a)
                if rc != 0:
                    raise RuntimeError(binding.status_string(rc))
        torch.cuda.synchronize()

    # warm-up
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    times = []
    for rep in range(args.reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if graph is not None:
            n_rep = max(1, args.steps // R)
            e0.record(stream)
            for _ in range(n_rep):
                graph.replay()
            e1.record(stream)
            n_steps = n_rep * R
        else:
            e0.record(stream)
            for i in range(args.steps):
                step(i)
            e1.record(stream)
            n_steps = args.steps
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n_steps)     # ms per step
    ms = float(np.median(times))
    t = ms * 1e-3

    accepted = outs[0].cpu().numpy()
    status = outs[2].cpu().numpy()
    committed = int(np.sum(accepted[status == 0] + 1))
    value = rows / t
    gbps = alg_bytes / t / 1e9

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "verify B=64 k=6 V=128256 bf16: 32 greedy, 16 one-hot-draft "
                               "and 16 draft-logit sampled requests",
                   "batch": B, "k": int(w.max_k), "vocab": w.vocab, "rows": rows,
                   "rotating_copies": R, "graph": bool(args.graph)},
        "tokens_committed_per_s": committed / t,
        "mean_tokens_per_request": committed / B,
        "achieved_GBps": gbps,
        "algorithmic_bytes_per_step": alg_bytes,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS, "traffic": kernel_traffic(),
                     "timed": "one verify launch per step (the only kernel of the call on "
                              "this workload), hipEvents on the launch stream"},
        "step_ms_reps": times,
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, outs, args.cpu_seconds)

    print(json.dumps(line), flush=True)
    return 0


def kernel_traffic():
    """Measured HBM bytes per launch for the kernel source in the tree, or
    None when the counters were taken on another source."""
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    return TRAFFIC_BYTES.get(digest)


def cpu_baseline(w, outs, budget_s):
    """The fp64 oracle as it stands, timed on the host on the same workload
    (whole batches repeated until the budget is used), and the GPU outputs of
    the timed data checked against it."""
    import numpy as np

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle

    def run():
        return oracle.verify(w.target, w.target_dtype, w.cu_seqlens, w.draft_tokens,
                             uniforms=w.uniforms, temperature=w.temperature, draft=w.draft,
                             draft_dtype=w.draft_dtype, draft_kind=w.draft_kind,
                             vocab=w.vocab, max_k=w.max_k, keep_cdf=True)

    t0 = time.perf_counter()
    n = 0
    ref = None
    while True:
        ref = run()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    rows = w.total_rows * n

    gpu_acc = outs[0].cpu().numpy()
    gpu_tok = outs[1].cpu().numpy()
    gpu_st = outs[2].cpu().numpy()
    cu = w.cu_seqlens
    res = {"match": 0, "excused": 0, "fail": 0}
    for b in range(w.batch):
        if gpu_st[b] != ref.status[b]:
            res["fail"] += 1
            continue
        rec = ref.records[b]
        a = int(gpu_acc[b])
        if isinstance(rec, tuple):
            same = a == ref.accepted[b] and np.array_equal(
                gpu_tok[cu[b]:cu[b + 1]], ref.out_tokens[cu[b]:cu[b + 1]])
            res["match" if same else "fail"] += 1
        else:
            v = oracle.excusal(rec, a, int(gpu_tok[cu[b] + a]))
            res["match" if v == "match" else "excused" if v == "excused" else "fail"] += 1
    return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full batches of the benchmark workload ({w.total_rows} rows each), "
                      f"single-threaded NumPy fp64, {el:.1f} s",
            "parity_of_timed_outputs": res}


if __name__ == "__main__":
    sys.exit(main())

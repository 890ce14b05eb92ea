#!/usr/bin/env python3
"""Benchmark of the batched speculative-decoding verify on one MI355X.

Headline workload: B=64 requests, k=6 drafts, V=128256, bf16 logits (32
greedy, 16 one-hot-draft sampled, 16 draft-logit sampled requests; synthetic,
seeded).  A step is one call of the whole verify (every kernel of the path)
on one batch.  Inputs are resident in HBM before the timed region; R rotating
copies of the inputs (sized to three times the 256 MB Infinity Cache) make
every step read from HBM rather than from the cache.

Prints one JSON line: verify rows/s (the value), tokens committed/s, achieved
algorithmic HBM bandwidth against the 8 TB/s peak and against a streaming read
of the same bytes (the ceiling), the other four synthetic workloads
(per_config: B=1000x k=4 V=1024 f32, B=32 k=5 V=32000 f32, the B=256 varlen
workload with top-k/top-p, B=512 k=5 V=152064 with fp32 draft probabilities),
and the fp64 CPU oracle timed on the host's cores (cpu_baseline), which also
checks the GPU outputs of the timed data of every workload.
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
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(ROOT, "lossless_rejection_sampling_spec_amd", "csrc", "specverify.hip")
STREAM_LIB = os.path.join(ROOT, "lossless_rejection_sampling_spec_amd", "libsvstream.so")
MAX_POOL = 16          # host cores a one-GPU machine gives this job

# HBM bytes per verify launch on the headline workload, from two rocprofv3
# --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by
# what the counter reads for a copy kernel of known size in the same run.
# Keyed by the SHA-256 of the kernel source the counters were taken on: for
# any other source the figure is stale and the bench reports null.
TRAFFIC_BYTES: dict = {
    # FETCH 71,889.5 KiB x 1.99963 + WRITE 346.6 KiB x 1.0 per launch
    "0750c227cce21dd05100ef86b9b3c3ed4c763e2db4e00f7b03287371429c1c96": 147557602,
    # the same source with a comment changed (the built library is byte-identical)
    "af37787b3794f5b618de248a8afc3c7c822f5bb2c6fc417db510f4443964ea01": 147557602,
}

# Workloads besides the headline one: (config, steps per repetition, label).
OTHERS = [
    (0, 100, "verify B=1000 replicas of k=4 V=1024 f32, draft logits sigma 0.5, T=1"),
    (1, 200, "verify B=32 k=5 V=32000 f32, draft logits sigma 0.7, T=0.8"),
    (3, 50, "verify B=256 varlen k 1..8 V=128256 bf16, draft logits, top-k/top-p, T~U[0.3,1.2]"),
    (4, 30, "verify B=512 k=5 V=152064 bf16 target, fp32 draft probabilities, T=1"),
]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions; the median is reported")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the multi-core oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other four workloads (per_config)")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--graph", action="store_true",
                    help="replay the headline steps from a captured HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device-to-device copy of 128 MiB, 10 times (the "
                         "reference kernel that scales the HBM byte counters of a profiler run)")
    ap.add_argument("--only", type=int, choices=[c for c, _, _ in OTHERS],
                    help="time only this other workload (for profiler runs); prints its record")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# the oracle baseline (host cores, before the GPU is touched)
# ---------------------------------------------------------------------------
def _oracle_verify(w, keep_cdf=True):
    sys.path.insert(0, ROOT)
    import oracle
    return oracle.verify(w.target, w.target_dtype, w.cu_seqlens, w.draft_tokens,
                         uniforms=w.uniforms, temperature=w.temperature, draft=w.draft,
                         draft_dtype=w.draft_dtype, draft_kind=w.draft_kind, top_k=w.top_k,
                         top_p=w.top_p, vocab=w.vocab, max_k=w.max_k, keep_cdf=keep_cdf)


_W = None     # the workload forked workers see


def _worker(budget):
    t0 = time.perf_counter()
    n = 0
    while True:
        _oracle_verify(_W)
        n += 1
        if time.perf_counter() - t0 >= budget:
            break
    return n, time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s):
    """The fp64 oracle as it stands, timed on the host: whole batches of the
    headline workload repeated until the budget is used, on one core and on
    every core this job has (forked worker processes, before any GPU call)."""
    import multiprocessing as mp
    global _W
    _W = w
    t0 = time.perf_counter()
    n1 = 0
    while True:
        _oracle_verify(w)
        n1 += 1
        if time.perf_counter() - t0 >= budget_s / 2:
            break
    one = w.total_rows * n1 / (time.perf_counter() - t0)
    cores = max(1, min(len(os.sched_getaffinity(0)), MAX_POOL))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        res = pool.map(_worker, [budget_s] * cores)
    wall = time.perf_counter() - t0
    batches = sum(n for n, _ in res)
    return {"value": w.total_rows * batches / wall, "unit": "rows/s", "cores": cores,
            "kind": "oracle", "cpu_model": _cpu_model(), "one_core_value": one,
            "sample": f"{batches} full batches of the benchmark workload ({w.total_rows} rows "
                      f"each) on {cores} worker processes, NumPy fp64, {wall:.1f} s wall; "
                      f"one core: {n1} batches in {budget_s / 2:.0f} s"}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------
def rotating_copies(base, nbytes):
    R = max(2, math.ceil(3 * MALL_BYTES / max(nbytes, 1)))
    copies = [base]
    for _ in range(R - 1):
        copies.append({k: (None if v is None else v.clone()) for k, v in base.items()})
    return copies


def time_workload(w, steps, warmup, reps, graph=False):
    """Median ms per verify call over `reps` repetitions of `steps` calls on
    rotating input copies; returns (ms, rep times, outputs of the last call,
    copies)."""
    import numpy as np
    import torch

    from lossless_rejection_sampling_spec_amd import binding, synth
    dev = torch.device("cuda:0")
    base = binding.workload_tensors(w, dev)
    copies = rotating_copies(base, synth.algorithmic_bytes(w))
    R = len(copies)
    B, rows = w.batch, w.total_rows
    n_draft = max(rows - B, 1)
    outs = (torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(rows, dtype=torch.int32, device=dev),
            torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(n_draft, dtype=torch.float32, device=dev),
            torch.empty(n_draft, dtype=torch.float32, device=dev))
    ws = binding.get_workspace(dev, binding.workspace_bytes(B, rows, w.vocab, w.max_k))
    L = binding.lib()
    stream = torch.cuda.current_stream(dev)

    def args_for(t, s):
        d = t["draft"]
        return (t["target"].data_ptr(), w.target_dtype, t["target"].stride(0),
                None if d is None else d.data_ptr(), w.draft_dtype, 0 if d is None else d.stride(0),
                t["draft_kind"].data_ptr(), t["cu_seqlens"].data_ptr(),
                t["draft_tokens"].data_ptr(), t["uniforms"].data_ptr(),
                t["temperature"].data_ptr(),
                None if t["top_k"] is None else t["top_k"].data_ptr(),
                None if t["top_p"] is None else t["top_p"].data_ptr(),
                B, rows, w.max_k, w.vocab, outs[0].data_ptr(), outs[1].data_ptr(),
                outs[3].data_ptr(), outs[4].data_ptr(), outs[2].data_ptr(), ws.data_ptr(),
                ws.numel(), s)

    call_args = [args_for(t, stream.cuda_stream) for t in copies]
    fn = L.spec_verify_sampled

    def step(i):
        rc = fn(*call_args[i % R])
        if rc != 0:
            raise RuntimeError(binding.status_string(rc))

    g = None
    if graph:
        s = torch.cuda.Stream(dev)
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            step(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for t in copies:
                rc = fn(*args_for(t, s.cuda_stream))
                if rc != 0:
                    raise RuntimeError(binding.status_string(rc))
        torch.cuda.synchronize()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if g is not None:
            n_rep = max(1, steps // R)
            e0.record(stream)
            for _ in range(n_rep):
                g.replay()
            e1.record(stream)
            n_steps = n_rep * R
        else:
            e0.record(stream)
            for i in range(steps):
                step(i)
            e1.record(stream)
            n_steps = steps
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n_steps)
    # the outputs of the first copy's inputs (the ones the oracle checks)
    step(0)
    torch.cuda.synchronize()
    res = {"accepted": outs[0].cpu().numpy(), "out_tokens": outs[1].cpu().numpy(),
           "status": outs[2].cpu().numpy()}
    return float(np.median(times)), times, res


def stream_ceiling(nbytes, steps, reps):
    """The streaming-read kernel over `nbytes` with the same rotation: median
    us per read and GB/s."""
    import ctypes

    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    L = ctypes.CDLL(STREAM_LIB)
    L.sv_stream_read.restype = ctypes.c_int
    L.sv_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.sv_stream_read_words.restype = ctypes.c_size_t
    L.sv_stream_read_words.argtypes = [ctypes.c_size_t]
    R = max(2, math.ceil(3 * MALL_BYTES / nbytes))
    bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(R)]
    out = torch.empty(int(L.sv_stream_read_words(nbytes)), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    for i in range(20):
        L.sv_stream_read(bufs[i % R].data_ptr(), nbytes, out.data_ptr(), stream)
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            rc = L.sv_stream_read(bufs[i % R].data_ptr(), nbytes, out.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"stream read failed ({rc})")
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / steps)
    us = float(np.median(times))
    return {"us": us, "GBps": nbytes / us / 1e3, "bytes": nbytes, "rotating_copies": R,
            "kernel": "one 16 KiB chunk per workgroup, non-temporal 128-bit loads "
                      "(csrc/stream_read.hip)"}


def parity(w, res):
    """GPU outputs of the timed data against the oracle: match / excused / fail."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    ref = _oracle_verify(w)
    cu = w.cu_seqlens
    out = {"match": 0, "excused": 0, "fail": 0}
    for b in range(w.batch):
        if res["status"][b] != ref.status[b]:
            out["fail"] += 1
            continue
        rec = ref.records[b]
        a = int(res["accepted"][b])
        if rec is None:
            out["match"] += 1
        elif isinstance(rec, tuple):
            same = a == ref.accepted[b] and np.array_equal(res["out_tokens"][cu[b]:cu[b + 1]],
                                                           ref.out_tokens[cu[b]:cu[b + 1]])
            out["match" if same else "fail"] += 1
        else:
            t = int(res["out_tokens"][cu[b] + a]) if 0 <= a <= cu[b + 1] - cu[b] - 1 else -1
            v = oracle.excusal(rec, a, t)
            out["match" if v == "match" else "excused" if v == "excused" else "fail"] += 1
    return out


COPY_BYTES = 128 << 20


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, ten times: the profiler's
    FETCH_SIZE / WRITE_SIZE of this kernel against its known bytes give the
    counters' scale on this GPU."""
    import torch
    src = torch.randint(0, 255, (COPY_BYTES,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()


def kernel_traffic():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    return TRAFFIC_BYTES.get(digest)


def workload_record(cfg, label, wc, steps, warmup, reps):
    """Time one of the other workloads and check the timed outputs."""
    import numpy as np
    from lossless_rejection_sampling_spec_amd import synth
    ms_c, times_c, res_c = time_workload(wc, steps, warmup, reps)
    tc = ms_c * 1e-3
    ok = res_c["status"] == 0
    acc = res_c["accepted"]
    bytes_c = synth.algorithmic_bytes(wc, acc)
    gb_c = bytes_c / tc / 1e9
    return {"workload": label, "us_per_call": ms_c * 1e3, "rows_per_s": wc.total_rows / tc,
            "tokens_committed_per_s": float(np.sum(acc[ok] + 1)) / tc,
            "algorithmic_bytes_per_step": bytes_c, "achieved_GBps": gb_c,
            "frac": gb_c / PEAK_HBM_GBPS, "step_ms_reps": times_c,
            "parity_of_timed_outputs": parity(wc, res_c)}


def only_workload(args):
    import torch

    from lossless_rejection_sampling_spec_amd import binding, synth
    cfg, _, label = next(o for o in OTHERS if o[0] == args.only)
    wc = synth.make(cfg, seed=args.seed)
    torch.cuda.set_device(torch.device("cuda:0"))
    binding.lib()
    rec = workload_record(cfg, label, wc, args.steps, args.warmup, args.reps)
    print(json.dumps({"only": cfg, **rec}), flush=True)
    return 0


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this verify benchmark runs on exactly one GPU (--gpus 1); the batch "
              "shards across GPUs with no communication, so per-GPU throughput is the figure",
              file=sys.stderr)
        return 2

    import numpy as np

    sys.path.insert(0, ROOT)
    from lossless_rejection_sampling_spec_amd import synth

    if args.only is not None:
        return only_workload(args)

    # inputs and the host-side baseline first: no GPU call has happened yet,
    # so the forked oracle workers inherit no device state
    w = synth.make(2, seed=args.seed)
    others = [] if args.headline_only else [(c, s, lab, synth.make(c, seed=args.seed))
                                            for c, s, lab in OTHERS]
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)

    import torch

    from lossless_rejection_sampling_spec_amd import binding
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()                       # fails loudly without the HIP library

    if args.copy_calibration:
        copy_calibration()
    ms, times, res = time_workload(w, args.steps, args.warmup, args.reps, graph=args.graph)
    t = ms * 1e-3
    rows = w.total_rows
    alg_bytes = synth.algorithmic_bytes(w)
    committed = int(np.sum(res["accepted"][res["status"] == 0] + 1))
    gbps = alg_bytes / t / 1e9
    R = max(2, math.ceil(3 * MALL_BYTES / alg_bytes))
    ceiling = None if args.no_stream else stream_ceiling(alg_bytes, args.steps, args.reps)

    line = {
        "metric": METRIC,
        "value": rows / t,
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
                   "batch": w.batch, "k": int(w.max_k), "vocab": w.vocab, "rows": rows,
                   "rotating_copies": R, "graph": bool(args.graph)},
        "tokens_committed_per_s": committed / t,
        "mean_tokens_per_request": committed / w.batch,
        "achieved_GBps": gbps,
        "algorithmic_bytes_per_step": alg_bytes,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS, "traffic": kernel_traffic(),
                     "traffic_unit": "HBM bytes per launch (profiler counters, scaled)",
                     "traffic_GBps": (None if kernel_traffic() is None
                                      else kernel_traffic() / t / 1e9),
                     "ceiling_GBps": None if ceiling is None else ceiling["GBps"],
                     "frac_of_ceiling": None if ceiling is None else gbps / ceiling["GBps"],
                     "timed": "one verify launch per step (the only kernel of the call on "
                              "this workload), hipEvents on the launch stream"},
        "step_ms_reps": times,
        "stream_ceiling": ceiling,
        "parity_of_timed_outputs": parity(w, res),
    }

    per = {}
    for cfg, steps, label, wc in others:
        per[str(cfg)] = workload_record(cfg, label, wc, steps, 5, 3)
        torch.cuda.empty_cache()
    if per:
        line["per_config"] = per
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

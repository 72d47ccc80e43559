"""Benchmark of the batched logits sampler on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 5] [--no-cpu-baseline]
    python bench.py --latency [--warm] [--steps K] [--warmup W]

A step is one sampler_run over one batch: the whole hot path (penalty,
temperature, top-k, softmax, top-p, exponential race, dense filtered
logits) on synthetic logits already resident in HBM.  The default workload
is batch 1024 x vocab 262144 bf16 logits (4 x Gumbel), rows cycling through
the eight top-k / top-p / sample combinations, dense output on every row.

Prints one JSON line: rows/s (value), ms per step, achieved HBM GB/s of the
path's algorithmic bytes, a roofline entry for the dominant kernel (timed with
HIP events on the stream it runs on), and the CPU oracle timed on a bounded
sample of the same rows.

--latency instead times single calls of each of the five workloads (batch x
vocab 4 x 32000 up to 1024 x 262144, each with its own stage mix) and prints
one JSON line per workload: the median, p10 and p90 per-call time from HIP
events around each call, with a 1 GiB buffer written between calls so that
the small workloads' inputs are not served from the 256 MB last-level cache
(with --warm, calls back to back: inputs and kernel code stay cached, as in a
decode loop).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "sampled rows/sec and achieved HBM GB/s (% of peak) at batch x vocab"
KERNELS = ["k_plan", "k_pass", "k_rows", "k_fallback", "k_dense", "k_epilogue"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--latency", action="store_true",
                    help="per-call latency of every workload (one JSON line each)")
    ap.add_argument("--warm", action="store_true",
                    help="with --latency: no cache flush between calls")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (fp32) a few times: "
                         "the reference for scaling HBM byte counters")
    return ap.parse_args()


def copy_probe(mib):
    """A plain copy kernel of known size (reads and writes mib MiB each), for
    calibrating the FETCH_SIZE / WRITE_SIZE counters of a profiler run."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib, "launches": 5}), flush=True)


def model_bytes(W, kept):
    """Algorithmic bytes per call, per kernel, from the per-row model:
    logits once (V * elem), the dense fp32 output (4V) when requested, q
    where the method reads it (all V for rows that sample without a filter,
    4 |K| gathered for filtered sampling rows), history ids (4 each), the
    output id (8) and the per-row k, p, flags (9).  The pass reads every
    row's logits and history ids, q of unfiltered sampling rows, and writes
    the dense output of unfiltered rows; the merge gathers q at K; the dense
    writer writes the filtered rows' dense output."""
    B, V = W.B, W.V
    flags = W.row_flags if W.row_flags is not None else np.full(B, 7, np.uint8)
    kmax = min(V, 1024)
    tk = ((flags & 1) != 0) & (W.top_k is not None)
    if W.top_k is not None:
        tk &= (W.top_k >= 1) & (W.top_k <= kmax)
    tp = ((flags & 2) != 0) & (W.top_p is not None)
    if W.top_p is not None:
        tp &= W.top_p < 1.0
    sm = ((flags & 4) != 0) & (W.q is not None)
    filtered = tk | tp
    nids = np.zeros(B, np.int64)
    if W.ids is not None and W.penalty != 1.0:
        nids = np.diff(W.offsets)
    unf = ~filtered
    npass = B * V * W.elem_bytes                      # logits of every row
    npass += int((sm & unf).sum()) * 4 * V            # the race streams q
    ndense = 0
    if W.need_logits:
        npass += int(unf.sum()) * 4 * V               # dense output of unfiltered rows
        ndense += int(filtered.sum()) * 4 * V         # filtered rows: written after the merge
    npass += int(nids.sum()) * 4
    rows = int((kept[sm & filtered]).sum()) * 4 + B * (8 + 9)
    return {"k_plan": 0, "k_pass": npass, "k_rows": rows, "k_fallback": 0, "k_dense": ndense,
            "k_epilogue": 0}


def device_source_sha():
    """sha256 over the sources the kernels are compiled from, in this order:
    csrc/sampler_kernels.hip, csrc/sampler_internal.h, include/sampler.h."""
    import hashlib

    h = hashlib.sha256()
    for rel in (("decode_token_sampling_row_amd", "csrc", "sampler_kernels.hip"),
                ("decode_token_sampling_row_amd", "csrc", "sampler_internal.h"),
                ("include", "sampler.h")):
        with open(os.path.join(ROOT, *rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counted_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE / WRITE_SIZE, scaled by a plain copy's reading), or
    None when no summary covers it or the device code changed since (the
    hash covers every source the kernels are compiled from)."""
    import glob

    sha = device_source_sha()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        txt = open(path).read()
        m_sha = re.search(r"^kernel_source_sha256: ([0-9a-f]{64})$", txt, re.M)
        m_tr = re.search(rf"^traffic_bytes_per_launch {kernel}: ([0-9]+)$", txt, re.M)
        if m_sha and m_tr and m_sha.group(1) == sha:
            return int(m_tr.group(1))
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, cpu_rows):
    """The CPU oracle (plain C, one full sort per row, double precision) on a
    bounded sample of the workload's rows: on the host threads this process
    is given (OMP_NUM_THREADS, else every core) and on one thread.  A
    reported baseline only."""
    from oracle import oracle as orc

    nproc = os.cpu_count() or 1
    threads = max(1, min(nproc, int(os.environ.get("OMP_NUM_THREADS", nproc))))

    def timed(rows, nthreads, budget):
        passes, spent = 0, 0.0
        while passes < 8 and (passes == 0 or spent < budget):
            c0 = time.perf_counter()
            orc.run(W.logits, orc.BF16 if W.dtype == "bf16" else orc.F32, vocab=W.V,
                    top_k=W.top_k, top_p=W.top_p, q=W.q, eps=W.eps,
                    temperature=W.temperature, penalty=W.penalty, ids=W.ids,
                    offsets=W.offsets, row_flags=W.row_flags, need_logits=W.need_logits,
                    rows=rows, threads=nthreads)
            spent += time.perf_counter() - c0
            passes += 1
        return passes, spent

    n = min(W.B, cpu_rows)
    passes, spent = timed(np.arange(n), threads, 10.0)
    n1 = min(W.B, max(8, n // 8))  # one thread: an eighth of the rows
    passes1, spent1 = timed(np.arange(n1), 1, 5.0)
    return {"value": passes * n / spent, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "value_1thread": passes1 * n1 / spent1, "nproc": nproc, "cpu_model": cpu_model(),
            "sample": f"rows 0..{n - 1} of the same workload (all stage combinations), "
                      f"{passes} passes, {spent:.2f} s wall on {threads} threads; rows "
                      f"0..{n1 - 1}, {passes1} passes, {spent1:.2f} s on 1 thread"}


def latency(args):
    """Per-call latency of each workload, caches flushed between calls (or
    warm, back to back, with --warm)."""
    import torch

    from decode_token_sampling_row_amd import workloads as wl
    from decode_token_sampling_row_amd.sampler import Sampler

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    flush = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for cfg in sorted(wl.CONFIGS):
        W = wl.make(cfg, seed=args.seed)
        if W.dtype == wl.BF16:
            logits = torch.from_numpy(W.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            logits = torch.from_numpy(W.logits).to(dev)
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        out_idx = torch.empty(W.B, dtype=torch.int64, device=dev)
        out_l = torch.empty((W.B, W.V), dtype=torch.float32, device=dev)
        s = Sampler(W.B, W.V, torch.bfloat16 if W.dtype == wl.BF16 else torch.float32)
        kw = dict(top_k=t(W.top_k), top_p=t(W.top_p), q=t(W.q), eps=W.eps,
                  temperature=W.temperature, repetition_penalty=W.penalty,
                  penalty_ids=t(W.ids), penalty_offsets=t(W.offsets), row_flags=t(W.row_flags),
                  out_logits=out_l if W.need_logits else None)
        # kept-set sizes for the byte model, from an untimed call with the dense output
        s.run(logits, out_idx, **dict(kw, out_logits=out_l))
        torch.cuda.synchronize()
        kept = torch.isfinite(out_l).sum(dim=1).cpu().numpy()
        for _ in range(args.warmup):
            s.run(logits, out_idx, **kw)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i, (a, b) in enumerate(evs):
            if not args.warm:
                flush.fill_(float(i))
            a.record(stream)
            s.run(logits, out_idx, **kw)
            b.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        med = float(np.median(us))
        nbytes = sum(model_bytes(W, kept).values())
        print(json.dumps({
            "workload": W.name, "batch": W.B, "vocab": W.V, "logits_dtype": W.dtype,
            "calls": args.steps, "us_per_call_median": med,
            "us_per_call_p10": float(np.percentile(us, 10)),
            "us_per_call_p90": float(np.percentile(us, 90)),
            "rows_per_s": W.B / (med * 1e-6), "model_bytes": int(nbytes),
            "hbm_gbps": nbytes / (med * 1e-6) / 1e9,
            "hbm_frac": nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "caches": "warm, calls back to back" if args.warm
                      else "1 GiB written between calls"}), flush=True)
        s.close()
        del out_l, logits
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the sampler is "
              "row-parallel and shards by rows with no communication.", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.latency:
        latency(args)
        return

    import torch

    from decode_token_sampling_row_amd import workloads as wl
    from decode_token_sampling_row_amd.sampler import Sampler

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    t0 = time.time()
    W = wl.make(args.config, seed=args.seed)
    print(f"[bench] workload {W.name} B={W.B} V={W.V} {W.dtype} generated in "
          f"{time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    if W.dtype == wl.BF16:
        logits = torch.from_numpy(W.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        logits = torch.from_numpy(W.logits).to(dev)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, top_k, top_p, flags = t(W.q), t(W.top_k), t(W.top_p), t(W.row_flags)
    ids, offs = t(W.ids), t(W.offsets)
    out_idx = torch.empty(W.B, dtype=torch.int64, device=dev)
    out_l = torch.empty((W.B, W.V), dtype=torch.float32, device=dev) if W.need_logits else None
    s = Sampler(W.B, W.V, torch.bfloat16 if W.dtype == wl.BF16 else torch.float32)
    kw = dict(top_k=top_k, top_p=top_p, q=q, eps=W.eps, temperature=W.temperature,
              repetition_penalty=W.penalty, penalty_ids=ids, penalty_offsets=offs,
              row_flags=flags, out_logits=out_l)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        s.run(logits, out_idx, **kw)
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        s.run(logits, out_idx, **kw)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})",
          file=sys.stderr, flush=True)

    # per-kernel times: a second timed region of the same K steps, with the
    # library recording HIP events on the launch stream around each kernel
    torch.cuda.synchronize()
    for _ in range(args.steps):
        s.run(logits, out_idx, profile=True, **kw)
    per = np.array(s.profile())

    # kept-set sizes for the byte model (outside the timed region)
    if out_l is not None:
        kept = torch.isfinite(out_l).sum(dim=1).cpu().numpy()
    else:
        kept = np.full(W.B, 1, np.int64)
    mb = model_bytes(W, kept)
    total_bytes = sum(mb.values())
    dom = int(np.argmax(per))
    dom_name = KERNELS[dom]
    dom_gbps = mb[dom_name] / (per[dom] * 1e-3) / 1e9 if per[dom] > 0 else 0.0
    path_gbps = total_bytes / (ms * 1e-3) / 1e9
    rows_per_s = W.B / (ms * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, args.cpu_rows)

    out = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": W.name, "batch": W.B, "vocab": W.V, "logits_dtype": W.dtype,
                   "dense_logits": bool(W.need_logits)},
        "hbm_gbps": path_gbps,
        "hbm_frac": path_gbps / HBM_PEAK_GBPS,
        "model_bytes_per_step": total_bytes,
        "kernel_ms": {k: float(v) for k, v in zip(KERNELS, per)},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": dom_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dom_gbps / HBM_PEAK_GBPS,
                     "traffic": counted_traffic(dom_name), "algorithmic_bytes": mb[dom_name],
                     "kernel_ms": float(per[dom])},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    s.close()


if __name__ == "__main__":
    main()

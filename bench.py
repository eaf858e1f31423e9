#!/usr/bin/env python3
"""Benchmark of the grouped-query attention core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--decode-workload NAME|none] [--append-workload NAME|none]
                    [--paged-workload NAME|none]
                    [--no-cpu-baseline]

Prints ONE JSON line on stdout.  A step is one call of the prefill entry point
on the selected workload (default: the pages' worked example, B=32, L=1024,
8 query heads over 4 key/value heads, d=64, bf16, non-causal).  Before the W warmup
steps the same step runs untimed for --settle-seconds (default 0.5 s) so the GPU
reaches its working clocks; then K steps are timed back to back between two
device synchronisations; ``value`` is the
algorithmic TFLOP/s of that timed region (4 * B * h_q * d * visible (query,
key) pairs per step; causal counts L(L+1)/2 pairs per head).  K more steps
follow, each between two HIP events on the launch stream, for the kernel's
average duration in ``roofline``.

The decode entry point is timed next on its own workload (64 sequences, 32
query heads over 8 key/value heads, d=128, S=8192, lengths U{1024..8192}).  A
512 MiB buffer is read before every decode call, outside the timed events, so
the 256 MiB last-level cache holds none of the KV cache (a read, not a write:
evicting with writes would leave dirty lines whose write-back lands inside the
timed kernel); its throughput is
KV-cache bytes actually needed (sum of lengths * h_kv * d * 2 tensors * 2 B)
per second of kernel time, reported under ``decode``.  The decode that appends
the new token's key/value rows itself is timed the same way on its own
workload (the same shape, lengths U{1023..8191} before the append) and
reported under ``decode_append``; its bytes also count the new rows, read
once and written once.  The decode over a paged cache (the batched-decode
inputs in a shuffled pool of 64-row pages) is reported under ``decode_paged``.

``roofline`` divides the algorithmic work of one launch by the launch's
average duration measured with HIP events on the launch stream; ``traffic``
comes from the rocprofv3 HBM counter summary under ``profiles/`` when that
summary was taken on the current kernel source, else null.  ``cpu_baseline``
times the fp64 CPU oracle on a bounded sample of the same workload.

With ``--copy-calibration`` it instead runs a plain 1 GiB device copy (for
scaling the HBM byte counters) and prints nothing else.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA prefill TFLOP/s (% MFMA peak); decode KV-cache GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FLUSH_BYTES = 512 << 20
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic.md")
CSRC = os.path.join(ROOT, "grouped_query_attention_03_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(Lq: int, Lk: int, causal: bool) -> int:
    """(query, key) pairs that take part: the Lq newest of Lk positions, causal or not."""
    if not causal:
        return Lq * Lk
    first = Lk - Lq  # query row i sees keys 0 .. first + i
    return Lq * (first + 1) + Lq * (Lq - 1) // 2


def varlen_pairs(L: int, n: int, causal: bool) -> int:
    """(query, key) pairs of one padded sequence with n valid keys: every one of
    the L rows sees keys j < n (and j <= i when causal)."""
    if not causal:
        return L * n
    return n * (n + 1) // 2 + (L - n) * n


def prefill_flops(w, kv_lens=None) -> float:
    if w.path == "prefill_varlen":
        pairs = sum(varlen_pairs(w.L, int(n), w.causal) for n in kv_lens)
        return 4.0 * w.h_q * w.d * pairs
    Lk = w.Lk if w.path == "prefill_chunk" else w.L
    return 4.0 * w.B * w.h_q * w.d * visible_pairs(w.L, Lk, w.causal)


def decode_kv_bytes(w, seqlens) -> float:
    """Key/value bytes one decode call must move: every valid cache row of K and
    V once per key/value head; with append also the new rows read from
    k_new/v_new and written into the cache."""
    rows = int(seqlens.sum()) + (2 * w.B if w.path == "decode_append" else 0)
    return float(rows) * w.h_kv * w.d * 2 * 2


def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "prefill": ["prefill_bf16.hip", "prefill_f32.hip", "gqa_device.h", "gqa_kernels.h"],
    "decode": ["decode_bf16.hip", "gqa_device.h", "gqa_kernels.h"],
}


def recorded_traffic(kind: str, workload: str, launches_per_step: int = 1):
    """HBM bytes per launch from the committed counter summary, if it matches the source.

    The summary has one table row per (kernel kind, workload) with the source
    digest it was taken on and scaled FETCH/WRITE bytes per launch.
    """
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    digest = source_digest(KERNEL_SOURCES[kind])
    total, found = 0.0, False
    for line in open(TRAFFIC_SUMMARY):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) < 5:
            continue
        # a decode call is the split pass of its workload plus the merge pass
        # (one row, the mean over the decode workloads)
        if not ((cells[0] == kind and cells[1] == workload) or
                (kind == "decode" and cells[0] == "decode_merge")):
            continue
        if cells[2] != digest:
            return None
        try:
            total += float(cells[3]) + float(cells[4])
            found = True
        except ValueError:
            return None
    return total if found else None


def time_launches(fn, steps, before=None):
    """Run fn() `steps` times; returns (wall seconds, per-launch event ms list)."""
    import torch
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if before is not None:
            before()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [s.elapsed_time(e) for s, e in zip(starts, ends)]


def settle_clocks(fn, seconds):
    """Run fn() untimed for about `seconds` of wall time.

    From idle, the GPU's power management takes tens of milliseconds of
    sustained load to reach its working clocks (the worked-example prefill
    runs at 154 us per launch for its first 25 launches and at 84 us after
    about 300); the timed region measures the kernel at those clocks.
    """
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        n += 10
    return n


def bench_prefill(w, steps, warmup, settle_s=0.0):
    import torch
    import gqa_workloads as wl
    import grouped_query_attention_03_amd as gqa
    dev = torch.device("cuda:0")
    ins = [t.to(dev) for t in wl.workload_inputs(w)]
    q, k, v = ins[:3]
    out = torch.empty_like(q)

    kv_lens = None
    if w.path == "prefill_varlen":
        kv_lens = ins[3]

        def step():
            gqa.prefill_varlen(q, k, v, kv_lens, causal=w.causal, scale=w.scale, out=out)
    elif w.path == "prefill_rope":  # two kernels: the key rotation, then the prefill
        cos, sin = ins[3:]
        k_rot = torch.empty_like(k)

        def step():
            gqa.prefill_rope(q, k, v, cos, sin, causal=w.causal, scale=w.scale, out=out,
                             k_rot=k_rot)
    else:
        call = gqa.prefill_chunk if w.path == "prefill_chunk" else gqa.prefill

        def step():
            call(q, k, v, causal=w.causal, scale=w.scale, out=out)

    settle_clocks(step, settle_s)
    for _ in range(warmup):
        step()
    # the K timed steps run back to back between two synchronisations; then K
    # more steps are timed one by one with events on the launch stream for
    # the kernel's own average (an event pair between launches leaves a small
    # gap on the GPU, so it is kept out of the throughput's timed region)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    _, ev = time_launches(step, steps)
    flops = prefill_flops(w, None if kv_lens is None else kv_lens.tolist())
    avg_ms = sum(ev) / len(ev)
    return {
        "value": flops * steps / wall / 1e12,
        "ms_per_step": wall * 1e3 / steps,
        "kernel_ms_avg": avg_ms,
        "kernel_ms_min": min(ev),
        "flops_per_launch": flops,
    }


def bench_decode(w, steps, warmup):
    import torch
    import gqa_workloads as wl
    import grouped_query_attention_03_amd as gqa
    dev = torch.device("cuda:0")
    append = w.path == "decode_append"
    paged = w.path == "decode_paged"
    if append:
        seqlens, q, kn, vn, kc, vc = wl.workload_inputs(w)
        kn, vn = kn.to(dev), vn.to(dev)
    elif paged:  # kc, vc are the page pools
        seqlens, q, kc, vc, table = wl.workload_inputs(w)
        table = table.to(dev)
    else:
        seqlens, q, kc, vc = wl.workload_inputs(w)
    kv_bytes = decode_kv_bytes(w, seqlens)
    seqlens, q, kc, vc = seqlens.to(dev), q.to(dev), kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(gqa.decode_workspace_bytes(w.B, w.h_q, w.h_kv, w.d), dtype=torch.uint8,
                     device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def step():
        if append:  # every call writes the same new rows again
            gqa.decode_append(q, kn, vn, kc, vc, seqlens, out=out, workspace=ws)
        elif paged:
            gqa.decode_paged(q, kc, vc, table, seqlens, out=out, workspace=ws)
        else:
            gqa.decode(q, kc, vc, seqlens, out=out, workspace=ws)

    flush.fill_(1)
    flush_words = flush.view(torch.int32)

    def evict():
        # a read-only pass over 512 MiB (one scalar written); a reduction with a
        # dtype conversion would first materialise a converted copy
        flush_words.max()

    for _ in range(warmup):
        evict()
        step()
    wall, ev = time_launches(step, steps, before=evict)
    avg_ms = sum(ev) / len(ev)
    achieved = kv_bytes / (avg_ms * 1e-3) / 1e9
    traffic = recorded_traffic("decode", w.name)
    what = ("decode split (writing the new rows) + log-sum-exp merge" if append else
            "decode split over pages + log-sum-exp merge" if paged else
            "decode split + log-sum-exp merge")
    return {
        "workload": w.name,
        "description": w.description,
        "value": achieved,
        "unit": "GB/s",
        "kernel_ms_avg": avg_ms,
        "kernel_ms_min": min(ev),
        "kv_bytes_per_call": kv_bytes,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernels": what + " (one call, timed together)"},
    }


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle timed on about budget_s seconds of the workload's own rows.

    Whole batch elements are run (all heads, all positions); when the whole
    workload takes less than the budget it is run repeatedly and the mean rate
    is reported.
    """
    import gqa_workloads as wl
    import oracle
    ins = wl.workload_inputs(w)
    qd, kd, vd = (t.double().numpy() for t in ins[:3])

    if w.path == "prefill_chunk":
        return _cpu_baseline_chunk(w, qd, kd, vd, budget_s)

    def run(nb):
        t0 = time.perf_counter()
        if w.path == "prefill_rope":
            oracle.prefill_rope(qd[:nb], kd[:nb], vd[:nb], ins[3].double().numpy(),
                                ins[4].double().numpy(), causal=w.causal, scale=w.scale)
        elif w.path == "prefill_varlen":
            oracle.prefill_varlen(qd[:nb], kd[:nb], vd[:nb], ins[3][:nb].numpy(), causal=w.causal,
                                  scale=w.scale)
        else:
            oracle.prefill(qd[:nb], kd[:nb], vd[:nb], causal=w.causal, scale=w.scale)
        return time.perf_counter() - t0

    t1 = run(1)
    nb = int(max(1, min(w.B, round(budget_s / max(t1, 1e-3)))))
    reps, total = 0, 0.0
    while total < budget_s or reps == 0:
        total += run(nb) if (nb > 1 or reps > 0) else t1
        reps += 1
    if w.path == "prefill_varlen":
        work = 4.0 * w.h_q * w.d * sum(varlen_pairs(w.L, int(n), w.causal) for n in ins[3][:nb])
    else:
        work = prefill_flops(w) / w.B * nb
    return {"value": work * reps / total / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "seconds": total,
            "sample": f"{nb} of {w.B} batch elements of {w.name} (all {w.h_q} heads x {w.L} "
                      f"positions each), run {reps} time(s), fp64"}


def _cpu_baseline_chunk(w, qd, kd, vd, budget_s):
    """The oracle on the newest m query rows of the chunk against all L_k keys
    (the same form of work), m sized to about budget_s seconds."""
    import oracle

    def run(m):
        t0 = time.perf_counter()
        oracle.prefill_cached(qd[:1, -m:], kd[:1], vd[:1], causal=w.causal, scale=w.scale)
        return time.perf_counter() - t0

    m0 = min(16, w.L)
    t1 = run(m0)
    m = int(max(m0, min(w.L, round(m0 * budget_s / max(t1, 1e-3)))))
    t = run(m) if m != m0 else t1
    flops = 4.0 * w.h_q * w.d * visible_pairs(m, w.Lk, w.causal)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": t,
            "sample": f"the newest {m} of the {w.L} query positions of one sequence of {w.name} "
                      f"against all {w.Lk} keys, all {w.h_q} heads, fp64"}


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes 3 times")


def main(argv=None):
    import gqa_workloads as wl
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="worked_example_prefill_bf16",
                    choices=[n for n in wl.WORKLOAD_ORDER
                             if wl.WORKLOADS[n].path in ("prefill", "prefill_chunk",
                                                         "prefill_rope", "prefill_varlen")])
    ap.add_argument("--decode-workload", default="batched_decode_bf16",
                    choices=["none"] + [n for n in wl.WORKLOAD_ORDER
                                        if wl.WORKLOADS[n].path == "decode"])
    ap.add_argument("--append-workload", default="batched_decode_append_bf16",
                    choices=["none"] + [n for n in wl.WORKLOAD_ORDER
                                        if wl.WORKLOADS[n].path == "decode_append"])
    ap.add_argument("--paged-workload", default="batched_decode_paged_bf16",
                    choices=["none"] + [n for n in wl.WORKLOAD_ORDER
                                        if wl.WORKLOADS[n].path == "decode_paged"])
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--settle-seconds", type=float, default=0.5,
                    help="untimed runs of the step before the warmup, to reach working clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the GQA core is built and timed on a single "
              "MI355X; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    w = wl.WORKLOADS[args.workload]
    log(f"prefill {w.name}: {w.description}; steps {args.steps} warmup {args.warmup}")
    pf = bench_prefill(w, args.steps, args.warmup, args.settle_seconds)
    peak = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    achieved = pf["flops_per_launch"] / (pf["kernel_ms_avg"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": pf["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_seconds,
        "ms_per_step": pf["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. normal draws cast to the compute dtype (no dataset)",
        "config": {"workload": w.name, "path": w.path, "B": w.B, "L": w.L, "h_q": w.h_q,
                   "h_kv": w.h_kv, "d": w.d, "causal": w.causal, "scale": w.scale,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": achieved,
                     "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": recorded_traffic("prefill", w.name),
                     "kernel_ms_avg": pf["kernel_ms_avg"], "kernel_ms_min": pf["kernel_ms_min"]},
    }
    if w.path == "prefill_chunk":
        line["config"]["L_k"] = w.Lk
    log(f"prefill: {pf['value']:.1f} TFLOP/s wall, kernel avg {pf['kernel_ms_avg']:.4f} ms "
        f"({achieved:.1f} TFLOP/s, {100 * achieved / peak:.1f}% of peak)")
    if args.decode_workload != "none":
        dw = wl.WORKLOADS[args.decode_workload]
        log(f"decode {dw.name}: {dw.description}; steps {args.decode_steps}")
        line["decode"] = bench_decode(dw, args.decode_steps, args.warmup)
        log(f"decode: {line['decode']['value']:.1f} GB/s, kernel avg "
            f"{line['decode']['kernel_ms_avg']:.4f} ms")
    if args.append_workload != "none":
        aw = wl.WORKLOADS[args.append_workload]
        log(f"decode with append {aw.name}: {aw.description}; steps {args.decode_steps}")
        line["decode_append"] = bench_decode(aw, args.decode_steps, args.warmup)
        log(f"decode with append: {line['decode_append']['value']:.1f} GB/s, kernel avg "
            f"{line['decode_append']['kernel_ms_avg']:.4f} ms")
    if args.paged_workload != "none":
        pw = wl.WORKLOADS[args.paged_workload]
        log(f"paged decode {pw.name}: {pw.description}; steps {args.decode_steps}")
        line["decode_paged"] = bench_decode(pw, args.decode_steps, args.warmup)
        log(f"paged decode: {line['decode_paged']['value']:.1f} GB/s, kernel avg "
            f"{line['decode_paged']['kernel_ms_avg']:.4f} ms")
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline: {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

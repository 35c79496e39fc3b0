"""Benchmark one paged-decode layer-step on one MI355X.

A step is the whole hot path over one batch: reshape_and_cache of the batch's
new K/V rows, pa_decode, and pa_decode_reduce when the library splits the
keys.  The default workload is the high-concurrency serving step with
Gemma-2-2B attention heads: 512 sequences, context = prompt U[16,512] +
generated U[1,512] tokens, 8 query / 4 KV heads, head_dim 256, block_size 16,
tanh soft-cap 50, bf16 KV, block tables drawn from a shuffled pool of 40000
blocks.  Inputs are synthetic (seeded N(0,1)) and resident in HBM before the
timed region starts.

Prints ONE JSON line.  `value` is achieved HBM bandwidth of the whole step in
GB/s, computed from the algorithmic bytes (K/V rows of attended tokens, q,
out, block-table entries, context lengths, new rows) over the measured step
time.  `roofline` reports the decode kernel alone: its algorithmic bytes over
its average HIP-event-timed duration, against the 8 TB/s HBM peak, and
(`roofline.read_ceiling`) against the read bandwidth a plain streaming kernel
reaches on the same GPU in the same run.
`cpu_baseline` times the float64 CPU oracle on a bounded sample of the same
workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# committed rocprofv3 counter summaries (HBM bytes per launch) by workload
TRAFFIC_FILES = {
    "2": os.path.join(ROOT, "profiles", "pa_decode_gemma2_global_b64_traffic.md"),
    "3": os.path.join(ROOT, "profiles", "pa_decode_gemma2_sliding_b16_traffic.md"),
    "4": os.path.join(ROOT, "profiles", "pa_decode_gemma2_b512_traffic.md"),
    "5": os.path.join(ROOT, "profiles", "pa_decode_llama_gqa8_long_b33_traffic.md"),
    "spec5": os.path.join(ROOT, "profiles", "pa_mq_gemma2_spec5_b512_traffic.md"),
    "chunk512": os.path.join(ROOT, "profiles", "pa_mq_gemma2_chunk512_traffic.md"),
    "prefill": os.path.join(ROOT, "profiles", "pa_mq_llama_prefill_2048x4_traffic.md"),
}


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_pa_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(digest: str, workload: str):
    """HBM bytes per launch of the workload's attention call from the
    committed rocprofv3 counter summary, if it was taken on the current
    kernel sources."""
    try:
        text = open(TRAFFIC_FILES[workload]).read()
    except (KeyError, OSError):
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic:"):
            for kv in line[len("traffic:"):].split():
                k, _, v = kv.partition("=")
                vals[k] = v
    if vals.get("kernel_sources") != digest:
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s: float):
    """Time the oracle on the workload's sequences, in order, until `budget_s`
    seconds have been spent (whole passes over the batch are repeated when
    one pass is shorter than the budget)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    eb = 2 if case.dtype != "f32" else 4
    T = case.slot_mapping.shape[0] if case.slot_mapping is not None else 0
    per_seq = case.attended().astype(np.int64) * case.Hkv * case.D * eb * 2 + 2 * case.Hq * case.D * eb + 4
    L = case.context_lens.astype(np.int64)
    n = case.attended().astype(np.int64)
    per_seq += np.where(n > 0, (L - 1) // case.bs - (L - n) // case.bs + 1, 0) * 4
    t0 = time.perf_counter()
    seqs = passes = 0
    bytes_ = 0
    while seqs == 0 or time.perf_counter() - t0 < budget_s:
        kc, vc = case.k_cache, case.v_cache
        if T:
            kc, vc = oracle.reshape_and_cache(case.key, case.value, kc, vc, case.slot_mapping)
            bytes_ += 4 * T * case.Hkv * case.D * eb + 8 * T
        for b in range(case.B):
            oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                          case.softcap, case.window, case.dtype, seqs=[b])
            bytes_ += int(per_seq[b])
            seqs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        passes += 1
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads if blas_threads else cores,
            "host_cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "seq_steps_per_s": round(seqs / dt, 2),
            "sample": f"float64 numpy oracle on this workload: reshape_and_cache of its {T} new "
                      f"rows then decode of its sequences in order, {seqs} sequence-steps over "
                      f"{passes} pass(es) in {dt:.1f} s"}


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}


def cold_times(step_fn, reps: int, dev, flush_mib: int = 1024):
    """Median event-timed step with the caches evicted first: before each rep
    a 1 GiB scratch buffer is read (more than the 256 MB Infinity Cache and
    the L2s), so the step's K/V come from HBM.  Returns (step_ms, attn_ms)
    where step_fn(record) returns the (start, end) events of its attention
    call, or None (then attn_ms is the step's)."""
    import torch
    scratch = torch.ones(flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    steps, attn = [], []
    for _ in range(reps):
        scratch.sum()  # evicts: reads 1 GiB
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        a = step_fn(True)
        e1.record(stream)
        torch.cuda.synchronize()
        steps.append(e0.elapsed_time(e1))
        attn.append(a[0].elapsed_time(a[1]) if a is not None else steps[-1])
    del scratch
    return float(np.median(steps)), float(np.median(attn))


def cold_only_report(args, name: str, step_fn, dev, bytes_: int, attn_label: str):
    """Profiling mode: every launch runs with the caches evicted first (the
    warm-up steps too), so a kernel trace of this run averages cold launches
    only.  Prints one JSON line with the medians."""
    cold_times(step_fn, max(args.warmup, 1), dev)
    step_ms, attn_ms = cold_times(step_fn, args.steps, dev)
    print(f"[bench] cold-only: step {step_ms*1e3:.1f} us, {attn_label} {attn_ms*1e3:.1f} us",
          file=sys.stderr, flush=True)
    print(json.dumps({
        "mode": "cold-only", "workload": name, "steps": args.steps, "warmup": args.warmup,
        "step_us": round(step_ms * 1e3, 2), f"{attn_label}_us": round(attn_ms * 1e3, 2),
        "algorithmic_bytes": bytes_,
        "step_gbs": round(bytes_ / (step_ms / 1e3) / 1e9, 2),
        "note": "median over steps each preceded by reading a 1 GiB scratch buffer"}),
        flush=True)


def calibration_copy(mib: int, dev):
    """Three plain device copies of `mib` MiB: the yardstick that scales the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] calibration copy: 3 x {mib} MiB read + write", file=sys.stderr, flush=True)


def cpu_baseline_mq(case, budget_s: float):
    """The oracle on a multi-query workload: the new rows land, then the
    query tokens are attended one by one in order until `budget_s` seconds
    have been spent."""
    import oracle
    from oracle import oracle as O
    eb = 2 if case.dtype != "f32" else 4
    t0 = time.perf_counter()
    kc, vc = oracle.reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                                      case.slot_mapping)
    toks = flops = 0
    L = case.context_lens.astype(np.int64)
    done = False
    for b in range(case.B):
        n = int(case.query_lens[b])
        for i in range(n):
            pos = int(L[b]) - n + i
            O.attend(case.q[case.query_start[b] + i], kc, vc, case.block_tables, b, pos + 1,
                     case.scale, case.softcap, case.window, case.dtype)
            keys = pos + 1 if case.window <= 0 else min(pos + 1, case.window)
            flops += 4 * case.D * case.Hq * keys
            toks += 1
            if time.perf_counter() - t0 >= budget_s:
                done = True
                break
        if done:
            break
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle", "tokens_per_s": round(toks / dt, 2),
            "sample": f"float64 numpy oracle on this workload: reshape_and_cache of its "
                      f"{case.T} new rows, then {toks} of its {case.T} query tokens in order "
                      f"in {dt:.1f} s"}


def bench_mq(args):
    """Multi-query step: pa_mq_step, i.e. reshape_and_cache of every new
    token's K/V row and pa_mq_attention (plan, attention and, when split, the
    reduce), the rows written in the plan's launch; the two separate calls
    are timed beside it."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from workloads import MQ_WORKLOADS, mq_workload

    dev = torch.device("cuda:0")
    print(f"[bench] building workload {args.workload} ({MQ_WORKLOADS[args.workload]})",
          file=sys.stderr, flush=True)
    case = mq_workload(args.workload, partition_size=args.partition_size)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
        return torch.from_numpy(a).to(dev)

    q, kc, vc = up(case.q), up(case.k_cache), up(case.v_cache)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    qs = torch.from_numpy(case.query_start).to(dev)
    key, value = up(case.key), up(case.value)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    T, Hq, D = case.q.shape
    maxL, maxq = case.max_context_len, case.max_query_len
    P = case.partition_size
    if P is None:
        P = pa.mq_partition_size(case.B, T, maxq, Hq, case.Hkv, D, case.bs, maxL, case.window,
                                 tdt)
    out = torch.empty_like(q)
    n = pa.mq_workspace_size(case.B, T, Hq, case.Hkv, D, maxL, P)
    ws = torch.empty((n + 3) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ev = []

    # the step as one prebuilt native call (pa_mq_step)
    fused = pa.MQStep(q, qs, kc, vc, bt, cl, case.scale, case.softcap, case.window,
                      partition_size=P, max_context_len=maxL, max_query_len=maxq, out=out,
                      key=key, value=value, slot_mapping=slots)
    # events made before any timed loop (creating them per step costs host
    # time that a short step would then wait for)
    pool = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(max(args.steps, 20))]

    def step(record=False, k=0):
        e = None
        if record:
            e = pool[k % len(pool)]
            e[0].record(stream)
        fused.run()
        if record:
            e[1].record(stream)
        return e

    def two_calls():
        pa.reshape_and_cache(key, value, kc, vc, slots)
        pa.mq_attention(q, qs, kc, vc, bt, cl, case.scale, case.softcap, case.window,
                        partition_size=P, max_context_len=maxL, max_query_len=maxq, out=out,
                        workspace=ws)

    if args.cold_only:
        return cold_only_report(args, case.name, step, dev, case.algorithmic_bytes()["total"],
                                "pa_mq_step")
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    # the same steps again, each bracketed by HIP events on its stream
    for k in range(args.steps):
        ev.append(step(record=True, k=k))
    torch.cuda.synchronize()
    attn_t = np.array([a.elapsed_time(b) for a, b in ev])
    attn_ms = float(attn_t.mean())
    attn_pct = {k: round(float(np.percentile(attn_t, q)) * 1e3, 2)
                for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}
    print(f"[bench] timed {args.steps} steps: {ms_step*1e3:.1f} us/step wall, "
          f"pa_mq_step {attn_ms*1e3:.1f} us (HIP events)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        two_calls()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        two_calls()
    torch.cuda.synchronize()
    ms_two = (time.perf_counter() - t0) * 1e3 / args.steps
    print(f"[bench] reshape_and_cache + pa_mq_attention as two calls: {ms_two*1e3:.1f} us/step",
          file=sys.stderr, flush=True)
    cold = None
    if not args.no_cold:
        cold_step_ms, cold_attn_ms = cold_times(step, min(args.steps, 20), dev)
        print(f"[bench] cold (caches evicted before each step): step {cold_step_ms*1e3:.1f} us, "
              f"pa_mq_step {cold_attn_ms*1e3:.1f} us", file=sys.stderr, flush=True)
        cold = {"step_us": round(cold_step_ms * 1e3, 2),
                "pa_mq_step_us": round(cold_attn_ms * 1e3, 2),
                "note": "median over steps each preceded by reading a 1 GiB scratch buffer"}
    if args.calib_copy_mib:
        calibration_copy(args.calib_copy_mib, dev)

    max_err = None
    if not args.no_check:
        from oracle import oracle as O
        kc0, vc0 = O.reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                                       case.slot_mapping)
        b = int(np.argmax(case.context_lens))
        toks = sorted({0, T - 1, int(case.query_start[b]), int(case.query_start[b + 1]) - 1})
        got = out.float().cpu().numpy().astype(np.float64)
        if not np.isfinite(got).all():
            print("[bench] PARITY FAILURE: non-finite output", file=sys.stderr)
            sys.exit(1)
        max_err = 0.0
        for t in toks:
            bb = int(np.searchsorted(case.query_start, t, side="right") - 1)
            pos = int(case.context_lens[bb]) - int(case.query_lens[bb]) + t - int(case.query_start[bb])
            want = O.attend(case.q[t], kc0, vc0, case.block_tables, bb, pos + 1, case.scale,
                            case.softcap, case.window, case.dtype)
            max_err = max(max_err, float(np.abs(got[t] - want).max()))
        print(f"[bench] parity spot-check on tokens {toks} (every output finite): "
              f"max abs err {max_err:.3e}",
              file=sys.stderr, flush=True)
        if not (max_err <= 2e-2):
            print("[bench] PARITY FAILURE", file=sys.stderr)
            sys.exit(1)

    ab = case.algorithmic_bytes()
    flops = case.flops()
    step_s = ms_step / 1e3
    value = ab["total"] / step_s / 1e9
    intensity = flops / ab["attn"]
    ridge = MFMA_PEAK_TFLOPS[case.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity > ridge:
        achieved = flops / (attn_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2),
                "peak": MFMA_PEAK_TFLOPS[case.dtype], "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS[case.dtype], 4)}
    else:
        achieved = ab["total"] / (attn_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    digest = kernel_source_digest()
    roof.update({"traffic": measured_traffic(digest, args.workload),
                 "kernel": "pa_mq_step (new rows + plan, attention, reduce)",
                 "algorithmic_bytes_per_launch": ab["total"], "flops_per_launch": flops,
                 "flop_per_byte": round(intensity, 2), "kernel_sources": digest})
    cpu = None
    if args.cpu_budget > 0:
        print(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline_mq(case, args.cpu_budget)
    res = {
        "metric": "multi-query paged attention: achieved HBM GB/s of the step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": case.dtype, "data": "synthetic",
        "config": {
            "workload": case.name, "num_seqs": case.B, "num_tokens": T, "num_heads": Hq,
            "num_kv_heads": case.Hkv, "head_dim": D, "block_size": case.bs,
            "num_blocks": case.NB, "softcap": case.softcap, "window": case.window,
            "max_context_len": maxL, "max_query_len": maxq, "partition_size": P,
            "parallelism": "single GPU",
        },
        "tokens_per_s": round(T / step_s, 1),
        "tflops": round(flops / step_s / 1e12, 2),
        "us_per_layer_step": round(ms_step * 1e3, 2),
        "pa_mq_step_us": round(attn_ms * 1e3, 2),
        "pa_mq_step_us_pct": attn_pct,
        "two_calls": {"ms_per_step": round(ms_two, 5),
                      "value": round(ab["total"] / (ms_two / 1e3) / 1e9, 2), "unit": "GB/s",
                      "note": "reshape_and_cache, then pa_mq_attention, as separate calls"},
        "algorithmic_bytes_per_step": ab["total"],
        "max_abs_err_vs_oracle": max_err,
        "roofline": roof,
        "cold": cold,
        "cpu_baseline": cpu,
    }
    if not args.no_ceiling:
        res["roofline"] = with_ceiling(res["roofline"], read_ceiling(pa, torch, dev))
    print(json.dumps(res), flush=True)



def read_ceiling(pa, torch, dev, gib=4):
    """Best read bandwidth (GB/s) of the library's plain streaming probe
    (pa_read_bandwidth_probe) over ``gib`` GiB, at four grid sizes: the
    practical ceiling next to the data sheet's HBM peak."""
    buf = torch.empty(gib << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * 4
    best = (0.0, 0)
    for grid in (4096, 8192, 16384, 32768):
        for _ in range(2):
            pa.read_bandwidth_probe(buf, grid, sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        n = 10
        e0.record()
        for _ in range(n):
            pa.read_bandwidth_probe(buf, grid, sink)
        e1.record()
        torch.cuda.synchronize()
        gbs = nbytes / (e0.elapsed_time(e1) / n / 1e3) / 1e9
        best = max(best, (gbs, grid))
    del buf
    torch.cuda.empty_cache()
    return {"gbs": round(best[0], 1), "grid": best[1],
            "probe": (f"pa_read_bandwidth_probe: one pass over {gib} GiB, 256-thread workgroups, "
                      "16-byte non-temporal loads, 8 in flight per thread, one contiguous 32 KB "
                      "block per workgroup step; best of grids 4096/8192/16384/32768, mean of "
                      "10 launches each (HIP events)")}


def with_ceiling(roof, ceiling):
    """Adds the measured read ceiling to an HBM-bound roofline object."""
    if ceiling is None or roof.get("bound") != "hbm":
        return roof
    roof = dict(roof)
    roof["read_ceiling"] = dict(ceiling)
    roof["read_ceiling"]["frac"] = round(roof["achieved"] / ceiling["gbs"], 4)
    return roof


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="4",
                    choices=["1", "2", "3", "4", "5", "spec5", "chunk512", "prefill"],
                    help="decode workload 1-5, or a multi-query workload")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="tokens per split-K partition (0 = none); default: library's choice")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--no-check", action="store_true", help="skip the parity spot-check")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cache-evicted timing (profiling runs: warm launches only)")
    ap.add_argument("--cold-only", action="store_true",
                    help="profiling mode: time only cache-evicted steps (warm-up included) "
                         "and print their medians")
    ap.add_argument("--sweep-partitions", action="store_true",
                    help="also time pa_step at partition sizes 0 (no split) and 64..1024")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read probe that measures the practical HBM ceiling")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the path needs no cross-GPU exchange and runs per GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_decode_pa_amd as pa
    from workloads import WORKLOADS, workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if not args.workload.isdigit():
        return bench_mq(args)
    args.workload = int(args.workload)
    dev = torch.device("cuda:0")
    print(f"[bench] building workload {args.workload} ({WORKLOADS[args.workload]})", file=sys.stderr, flush=True)
    case = workload(args.workload, partition_size=args.partition_size)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
        return torch.from_numpy(a).to(dev)

    q, kc, vc = up(case.q), up(case.k_cache), up(case.v_cache)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    key = value = slots = None
    if case.slot_mapping is not None:
        key, value = up(case.key), up(case.value)
        slots = torch.from_numpy(case.slot_mapping).to(dev)
    B, Hq, D = case.q.shape
    maxL = case.max_context_len
    P = case.partition_size
    if P is None:
        P = pa.partition_size(B, Hq, case.Hkv, D, case.bs, maxL, case.window, tdt)
    out = torch.empty_like(q)
    ws = pa.alloc_workspace(B, Hq, D, maxL, P, dev)
    split = P > 0 and (maxL + P - 1) // P > 1
    stream = torch.cuda.current_stream()

    ev = []  # (before, after) pa_decode, per step of the three-call loop

    call_ev = []  # (before, after) the whole pa_decode call: plan + decode kernel

    def step(record=False):
        """The three entry points in turn.  With record, HIP events bracket
        the decode kernel alone (recorded by pa_decode itself, on its stream,
        after any plan launch), and another pair the whole pa_decode call."""
        if slots is not None:
            pa.reshape_and_cache(key, value, kc, vc, slots)
        e = None
        if record:
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            c = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for x in e:
                x.record(stream)  # creates the event; pa_decode records it again
            pa.set_decode_events(*e)
            c[0].record(stream)
        try:
            pa.decode_partitions(out, ws, q, kc, vc, bt, cl, maxL, case.scale, case.softcap,
                                 case.window, P)
        finally:
            if record:
                pa.set_decode_events()
        if record:
            c[1].record(stream)
            call_ev.append(c)
        if split:
            pa.decode_reduce(out, ws, cl, maxL, P, case.window)
        return e

    # the whole step as one native call (pa_step): the new rows (one per
    # sequence at its last position, written by the decode launch itself
    # on the vector kernel), the plan, decode, merge
    tails = slots is not None and slots.shape[0] == B
    fused = pa.Step(q, kc, vc, bt, cl, case.scale, case.softcap, case.window,
                    partition_size=P, max_context_len=maxL, out=out, key=key, value=value,
                    slot_mapping=slots, rows_at_tails=tails)

    def fused_step(record=False):
        fused.run()
        return None

    if args.cold_only:
        return cold_only_report(args, case.name, fused_step, dev,
                                case.algorithmic_bytes()["total"], "pa_step")
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        fused_step()
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps of pa_step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fused_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps (pa_step): {ms_step*1e3:.1f} us/step wall",
          file=sys.stderr, flush=True)

    # the three entry points, K steps; HIP events bracket each pa_decode
    # launch on the stream it runs on (torch's current stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev.append(step(record=True))
    torch.cuda.synchronize()
    ms_step3 = (time.perf_counter() - t0) * 1e3 / args.steps
    dec_t = np.array([a.elapsed_time(b) for a, b in ev])
    decode_ms = float(dec_t.mean())
    decode_pct = {k: round(float(np.percentile(dec_t, q)) * 1e3, 2)
                  for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in call_ev]))
    print(f"[bench] three calls: {ms_step3*1e3:.1f} us/step wall, decode kernel "
          f"{decode_ms*1e3:.1f} us, pa_decode call {call_ms*1e3:.1f} us (HIP events)",
          file=sys.stderr, flush=True)

    reps = min(args.steps, 20)
    cold = None
    if not args.no_cold:
        cold_step_ms, _ = cold_times(fused_step, reps, dev)
        cold_step3_ms, cold_decode_ms = cold_times(step, reps, dev)
        print(f"[bench] cold (caches evicted before each step): pa_step {cold_step_ms*1e3:.1f} us, "
              f"three calls {cold_step3_ms*1e3:.1f} us, decode kernel {cold_decode_ms*1e3:.1f} us",
              file=sys.stderr, flush=True)
        cold = {"step_us": round(cold_step_ms * 1e3, 2),
                "three_calls_step_us": round(cold_step3_ms * 1e3, 2),
                "decode_kernel_us": round(cold_decode_ms * 1e3, 2),
                "decode_kernel_gbs": round(case.algorithmic_bytes()["decode"] / (cold_decode_ms / 1e3) / 1e9, 2),
                "note": "median over steps each preceded by reading a 1 GiB scratch buffer"}

    sweep = None
    if args.sweep_partitions:
        sweep = []
        for ps in [0, 64, 128, 256, 512, 1024]:
            if ps % case.bs:
                continue
            st_s = pa.Step(q, kc, vc, bt, cl, case.scale, case.softcap, case.window,
                           partition_size=ps, max_context_len=maxL, key=key, value=value,
                           slot_mapping=slots, rows_at_tails=tails)
            for _ in range(args.warmup):
                st_s.run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                st_s.run()
            torch.cuda.synchronize()
            w_ms = (time.perf_counter() - t0) * 1e3 / args.steps

            def sweep_step(record=False, st_s=st_s):
                st_s.run()
                return None
            c_ms, _ = cold_times(sweep_step, reps, dev)
            sweep.append({"partition_size": ps, "step_us": round(w_ms * 1e3, 2),
                          "cold_step_us": round(c_ms * 1e3, 2)})
            print(f"[bench] sweep P={ps}: pa_step {w_ms*1e3:.1f} us warm, {c_ms*1e3:.1f} us cold",
                  file=sys.stderr, flush=True)
            del st_s

    # the same step captured once into a HIP graph and replayed K times
    graph = None
    if not args.no_graph:
        gstream = torch.cuda.Stream()
        st = pa.Step(q, kc, vc, bt, cl, case.scale, case.softcap, case.window,
                     partition_size=P, max_context_len=maxL, out=out, key=key, value=value,
                     slot_mapping=slots, rows_at_tails=tails)
        st.capture(gstream)
        with torch.cuda.stream(gstream):
            for _ in range(args.warmup):
                st.replay(gstream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(gstream):
            for _ in range(args.steps):
                st.replay(gstream)
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        st.close()
        graph = {"ms_per_step": round(g_ms, 5),
                 "value": round(case.algorithmic_bytes()["total"] / (g_ms / 1e3) / 1e9, 2),
                 "unit": "GB/s"}
        print(f"[bench] graph replay: {g_ms*1e3:.1f} us/step", file=sys.stderr, flush=True)

    # a model's worth of layer steps (LAYERS of them, on these buffers)
    # eagerly, one pa_step each, against one graph holding all of them
    layers = None
    if not args.no_graph:
        n_l = 8
        lsteps = [pa.Step(q, kc, vc, bt, cl, case.scale, case.softcap, case.window,
                          partition_size=P, max_context_len=maxL, key=key, value=value,
                          slot_mapping=slots, rows_at_tails=tails) for _ in range(n_l)]
        gstream = torch.cuda.Stream()
        lg = pa.StepGraph(lsteps, gstream)
        reps_l = max(1, args.steps // n_l)
        with torch.cuda.stream(gstream):
            for _ in range(max(1, args.warmup // n_l)):
                lg.replay(gstream)
                for st_l in lsteps:
                    st_l.run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps_l):
                for st_l in lsteps:
                    st_l.run()
            torch.cuda.synchronize()
            e_us = (time.perf_counter() - t0) * 1e6 / (reps_l * n_l)
            t0 = time.perf_counter()
            for _ in range(reps_l):
                lg.replay(gstream)
            torch.cuda.synchronize()
            g_us = (time.perf_counter() - t0) * 1e6 / (reps_l * n_l)
        lg.close()
        del lsteps
        layers = {"layers": n_l, "eager_us_per_layer_step": round(e_us, 2),
                  "graph_us_per_layer_step": round(g_us, 2),
                  "note": f"{n_l} layer steps on these buffers: {n_l} pa_step calls against one "
                          "graph replay holding all of them"}
        print(f"[bench] {n_l} layer steps: eager {e_us:.1f} us/step, one graph {g_us:.1f} us/step",
              file=sys.stderr, flush=True)

    if args.calib_copy_mib:
        calibration_copy(args.calib_copy_mib, dev)

    max_err = None
    if not args.no_check:
        import oracle
        # every sequence of the batch against the oracle (a few seconds for
        # the largest workload)
        want = oracle.decode_case(case)
        got = out.float().cpu().numpy().astype(np.float64)
        max_err = float(np.abs(got - want).max())
        tol = 1e-4 if case.dtype == "f32" else 2e-2
        print(f"[bench] parity check on all {B} sequences: max abs err {max_err:.3e}",
              file=sys.stderr, flush=True)
        if not (np.isfinite(got).all() and max_err <= tol):
            print("[bench] PARITY FAILURE", file=sys.stderr)
            sys.exit(1)

    ab = case.algorithmic_bytes()
    step_s = ms_step / 1e3
    value = ab["total"] / step_s / 1e9
    achieved = ab["decode"] / (decode_ms / 1e3) / 1e9
    digest = kernel_source_digest()
    traffic = measured_traffic(digest, str(args.workload))

    cpu = None
    if args.cpu_budget > 0:
        print(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, args.cpu_budget)

    dname = {"f32": "f32", "f16": "f16", "bf16": "bf16"}[case.dtype]
    res = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and seq-steps/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dname,
        "data": "synthetic",
        "config": {
            "workload": case.name,
            "num_seqs": B, "num_heads": Hq, "num_kv_heads": case.Hkv, "head_dim": D,
            "block_size": case.bs, "num_blocks": case.NB, "softcap": case.softcap,
            "window": case.window, "scale": case.scale,
            "context_tokens": int(case.context_lens.sum()),
            "max_context_len": maxL, "partition_size": P,
            "new_rows": 0 if slots is None else int(slots.shape[0]),
            "new_rows_form": ("one per sequence at its last position (pa_step_args."
                              "new_rows_at_tails)" if tails else "slot list"),
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(B / step_s, 1),
        "us_per_layer_step": round(ms_step * 1e3, 2),
        "algorithmic_bytes_per_step": ab["total"],
        "decode_kernel_us": round(decode_ms * 1e3, 2),
        "decode_kernel_us_pct": decode_pct,
        "pa_decode_call_us": round(call_ms * 1e3, 2),
        "split_k_reduce": bool(split),
        "max_abs_err_vs_oracle": max_err,
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode's decode kernel",
            "timed": ("HIP events that pa_decode records on its stream right before and after "
                      "its decode kernel (pa_set_decode_events), mean over the timed calls"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab["decode"],
            "kernel_sources": digest,
        },
        "three_calls": {"ms_per_step": round(ms_step3, 5),
                        "value": round(ab["total"] / (ms_step3 / 1e3) / 1e9, 2), "unit": "GB/s",
                        "note": "reshape_and_cache, pa_decode, pa_decode_reduce as separate calls"},
        "graph_replay": graph,
        "graph_layers": layers,
        "partition_sweep": sweep,
        "cold": cold,
        "cpu_baseline": cpu,
    }
    if not args.no_ceiling:
        res["roofline"] = with_ceiling(res["roofline"], read_ceiling(pa, torch, dev))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

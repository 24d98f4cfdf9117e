#!/usr/bin/env python3
"""Decode-attention benchmark: steps/s and achieved HBM bandwidth on one MI355X.

One step = one decode step of the whole batch (split-K kernel, plus the
log-sum-exp merge kernel when sequences are split), inputs resident in HBM.
Default workload: PaLM-540B-shaped MQA decode (B=64, Hq=48, Hkv=1, D=256,
len 2048).

To keep the memory-side Infinity Cache (256 MB) from serving repeated reads,
every loop rotates through enough distinct q/K/V sets that the K/V bytes the
steps read cover at least 768 MiB, so every step reads its K/V from HBM.

Three passes, each on the library's stream:
  1. wall clock: W warmup steps, then K timed steps launched plainly (no
     per-kernel events), bracketed by HIP events in about 20 blocks;
  2. kernel pass (separate, after the timed loop): start/stop events recorded
     by the split kernel's own dispatch and by the merge kernel's own dispatch
     on every step of a further pass, so that each step's summed kernel
     duration is known;
  3. ceiling: the library's streaming-read probe over 2 GiB (8192 workgroups)
     and over the workload's own bytes and split grid.

Prints ONE JSON line (rank 0, N=1):
  value        decode steps per second over the K timed steps (pass 1)
  roofline     algorithmic K+V bytes per step divided by the mean summed
               duration of the step's kernels (split + merge, pass 2), against
               the 8 TB/s HBM peak; `split_only` gives the split kernel alone;
               `traffic` is the HBM bytes per split launch measured by
               rocprofv3 PMC counters (profiles/split_kernel_traffic_<workload>.txt)
               when those counters were taken on the current kernel sources,
               else null; `ceiling` the probe's rates
  step_kernel_us  mean, p10, p50, p90 of the per-step summed kernel durations
  cpu_baseline the CPU fp64 oracle on the host's cores on a bounded sample,
               with the CPU model and single-thread times for tiny and palm
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
MALL_DEFEAT_BYTES = 768 * 2 ** 20
MAX_SETS = 64  # tiny problems live in cache whatever the rotation
KERNEL_SOURCES = ["decode_mfma.hip", "decode_valu.hip", "combine.hip", "kernel_common.hpp",
                  "abi.cpp", "plan.cpp"]
WALL_BLOCKS = 20          # event-bracketed blocks of the timed loop (p10/p90 of block means)
CEILING_BYTES = 2 * 2 ** 30
CEILING_WORKGROUPS = 8192
CEILING_REPS = 20


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "gqa_decode_attention_mqa_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def read_traffic(workload: str, launches_per_step: int = 1):
    """HBM bytes per split-K launch from committed PMC summaries, if still current."""
    path = ROOT / "profiles" / ("split_kernel_traffic_%s.txt" % workload)
    if not path.exists():
        return None
    fields = {}
    for line in path.read_text().splitlines():
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_sha():
        return None
    try:
        return float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="palm", choices=["tiny", "palm", "gqa70b", "ragged", "long"])
    ap.add_argument("--variant", default=None, choices=[None, "auto", "valu", "mfma"])
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--combine", default=None, choices=[None, "auto", "separate", "fused"])
    ap.add_argument("--schedule", default=None, choices=[None, "auto", "per_item", "persistent"],
                    help="work items of the split kernel: one workgroup each, or a resident grid taking them "
                         "from a queue; default: the planner's choice")
    ap.add_argument("--page-size", type=int, default=0,
                    help="run the paged-cache entry point on a pool of pages of this many positions "
                         "(a power of two >= 32; the pool holds the used pages only); 0 = contiguous cache")
    ap.add_argument("--window", type=int, default=0,
                    help="local (sliding-window) attention: each sequence attends its last WINDOW positions; "
                         "0 = every cached position")
    ap.add_argument("--kv-format", default="bf16", choices=["bf16", "fp8", "int8"],
                    help="cache element format: bf16, or 8-bit codes (E4M3 or int8) with one fp32 scale "
                         "per cached row, made from the bf16 draw by the seeded per-row quantizer")
    ap.add_argument("--tokens", type=int, default=1,
                    help="query tokens per sequence decoded at once (causal among themselves; the cache is "
                         "read once for all of them); 1 = the decode step")
    ap.add_argument("--prefill", action="store_true",
                    help="time causal prefill (mqa_prefill_attention: every position of every sequence, no cache) "
                         "of the workload's shapes instead of the decode step; roofline against the bf16 "
                         "matrix-core peak")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch size B")
    ap.add_argument("--no-host-lens", action="store_true",
                    help="plan without the host copy of the lengths (mqa_decode_opts.host_seq_lens), so the "
                         "planner cannot tell a uniform batch from a ragged one")
    ap.add_argument("--kernel-steps", type=int, default=None,
                    help="steps of the evented kernel pass (default: max(200, min(steps, 2000)))")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling probe")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (PMC calibration) and exit")
    return ap.parse_args(argv)


def copy_probe(nbytes: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 5}))


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def single_thread_baseline(target_s: float = 4.0) -> dict:
    """The oracle on one thread: the tiny workload's whole step, and the PaLM-shaped step
    (whole when it fits ``target_s``, else a prefix of its sequences, scaled)."""
    import oracle
    from gqa_decode_attention_mqa_amd.workloads import WORKLOADS, make_inputs
    prev = oracle.max_threads()
    try:
        res = {}
        for name in ("tiny", "palm"):
            w = WORKLOADS[name]
            inp = make_inputs(w)
            q, k, v, lens = inp["q"], inp["k"], inp["v"], inp["seq_lens"]
            # set after the inputs are drawn: torch's own OpenMP use can reset the count
            if oracle.set_threads(1) != 1:
                raise RuntimeError("could not restrict the oracle to one thread")
            t0 = time.perf_counter()
            oracle.decode(q[:1], k[:1], v[:1], lens[:1], inp["scale"])
            one = max(time.perf_counter() - t0, 1e-6)
            nseq = w.B if one * w.B <= target_s else max(1, int(target_s / one))
            reps = max(1, int(target_s / (one * nseq))) if nseq == w.B else 1
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle.decode(q[:nseq], k[:nseq], v[:nseq], lens[:nseq], inp["scale"])
            dt = time.perf_counter() - t0
            steps = reps * float(lens[:nseq].double().sum() / lens.double().sum())
            res[name] = {"steps_per_s": round(steps / dt, 4), "seconds": round(dt, 3), "threads": oracle.max_threads(),
                         "sample": ("%d whole step(s)" % reps) if nseq == w.B else
                         ("first %d of %d sequences of one step, scaled by their share of positions" % (nseq, w.B))}
        return res
    finally:
        oracle.set_threads(prev)


def cpu_baseline(w, inp, target_s: float, window: int = 0, kv_format: str = "bf16", tokens: int = 1):
    """The oracle, as it stands, on whole decode steps of set 0 (or a prefix of the batch)."""
    import oracle
    q, k, v, lens = inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu()
    # every core this process may run on, set right before timing (torch's own
    # OpenMP use can change the count)
    threads = oracle.set_threads(len(os.sched_getaffinity(0)))
    if tokens > 1:
        run = lambda qq, kk, vv, ll: oracle.decode_multi(qq, kk, vv, ll, inp["scale"])
    elif kv_format != "bf16":
        ks, vs = inp["k_scale"].cpu(), inp["v_scale"].cpu()
        run = lambda qq, kk, vv, ll: oracle.decode_quant(qq, kk, vv, ks[:len(ll)], vs[:len(ll)], ll, kv_format,
                                                         inp["scale"])
    elif window:
        run = lambda qq, kk, vv, ll: oracle.decode_window(qq, kk, vv, ll, window, inp["scale"])
    else:
        run = lambda qq, kk, vv, ll: oracle.decode(qq, kk, vv, ll, inp["scale"])
    # time one sequence first to size the sample
    t0 = time.perf_counter()
    run(q[:1], k[:1], v[:1], lens[:1])
    one = max(time.perf_counter() - t0, 1e-6)
    per_seq_lens = lens.double().clamp(max=window) if window else lens.double()
    # sequences to run: whole steps when they fit in the budget, else a prefix of the batch
    est_step = one * float(per_seq_lens.sum()) / max(float(per_seq_lens[0]), 1.0)
    if est_step <= target_s:
        reps = max(1, int(target_s / max(est_step, 1e-6)))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(q, k, v, lens)
        dt = time.perf_counter() - t0
        steps = reps
        sample = "%d whole decode step(s) of the %s workload (B=%d%s)" % (
            reps, w.name, w.B, ", %s cache" % kv_format if kv_format != "bf16" else "")
    else:
        nseq = max(1, int(w.B * target_s / est_step))
        t0 = time.perf_counter()
        run(q[:nseq], k[:nseq], v[:nseq], lens[:nseq])
        dt = time.perf_counter() - t0
        steps = float(per_seq_lens[:nseq].sum() / per_seq_lens.sum())
        sample = "first %d of %d sequences of one %s decode step, scaled by their share of positions" % (
            nseq, w.B, w.name)
    return {"value": steps / dt, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": sample + "; fp64 C oracle, OpenMP over (sequence, head)", "seconds": round(dt, 3),
            "cpu_model": cpu_model(), "single_thread": single_thread_baseline()}


def pct(sorted_vals, p):
    """Nearest-rank percentile of an ascending list."""
    if not sorted_vals:
        return None
    i = min(len(sorted_vals) - 1, max(0, int(math.ceil(p / 100.0 * len(sorted_vals))) - 1))
    return sorted_vals[i]


def stream_ceiling(binding, torch, dev, pattern_bytes: int, pattern_wgs: int) -> dict:
    """Streaming-read rates of the library's probe: 2 GiB with 8192 workgroups, and the
    workload's own bytes with its split grid (rotating over 128 MiB-aligned slices of the
    2 GiB buffer so the Infinity Cache never serves a repeated read).  Medians of 20."""
    buf = torch.empty(CEILING_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty(max(CEILING_WORKGROUPS, pattern_wgs), dtype=torch.int32, device=dev)
    res = {}
    cases = [("stream_2gib", CEILING_BYTES, CEILING_WORKGROUPS)]
    nb = (pattern_bytes + 15) // 16 * 16
    if 0 < nb <= CEILING_BYTES // 4:
        cases.append(("workload_pattern", nb, pattern_wgs))
    for name, nbytes, wgs in cases:
        span = (nbytes + 2 ** 27 - 1) // 2 ** 27 * 2 ** 27
        nslices = max(1, CEILING_BYTES // span)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(CEILING_REPS)]
        for b, e in evs:
            b.record()
            e.record()
        for i in range(3):
            binding.stream_read_probe(buf[(i % nslices) * span:(i % nslices) * span + nbytes], wgs, sink)
        torch.cuda.synchronize()
        for i, ev in enumerate(evs):
            off = (i % nslices) * span
            binding.stream_read_probe(buf[off:off + nbytes], wgs, sink, events=ev)
        torch.cuda.synchronize()
        us = sorted(b.elapsed_time(e) * 1e3 for b, e in evs)
        med = us[len(us) // 2]
        res[name] = {"bytes": nbytes, "workgroups": wgs, "median_us": round(med, 3),
                     "gbs": round(nbytes / (med * 1e-6) / 1e9, 1)}
    del buf
    return res


BF16_MFMA_PEAK_TFLOPS = 2500.0


def prefill_flops(lens, Hq, D) -> float:
    """Algorithmic flops of causal attention: position t of a sequence takes 2 * Hq * D flops for
    q.k and as many for p.v at each of its t + 1 attended positions."""
    return float(sum(4.0 * Hq * D * n * (n + 1) / 2 for n in lens))


def run_prefill(args, w, torch, binding):
    """Causal prefill of the workload's batch: one step = one mqa_prefill_attention call."""
    from gqa_decode_attention_mqa_amd.workloads import make_prefill_inputs
    dev = torch.device("cuda:0")
    inp = make_prefill_inputs(w, device=dev)
    plan = binding.prefill_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.scale)
    out = torch.empty((w.B, w.Lmax, w.Hq, w.D), dtype=torch.float32, device=dev)
    lens = inp["seq_lens"].cpu().tolist()
    flops = prefill_flops(lens, w.Hq, w.D)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.prefill(inp["q_seq"], inp["k"], inp["v"], inp["seq_lens"], w.scale, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(marks[i].elapsed_time(marks[i + 1]) * 1e3 for i in range(args.steps))
    total_ms = marks[0].elapsed_time(marks[-1])
    ms_per_step = total_ms / args.steps
    achieved = flops / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": "causal prefill steps/sec and achieved TFLOP/s (% of MI355X bf16 matrix-core peak)",
        "value": round(1000.0 / ms_per_step, 3), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "causal prefill of " + w.description + (" (B=%d)" % w.B),
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "Lmax": w.Lmax, "tokens": int(sum(lens)),
                   "flops_per_step": flops, "plan": plan},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "causal prefill (mfma, %d query rows per workgroup)" % plan["rows_per_block"],
                     "step_us_p10_p50_p90": [round(pct(per, p), 2) for p in (10, 50, 90)]},
    }
    if not args.no_cpu_baseline:
        import oracle
        # the oracle's causal attention on a prefix of sequence 0, sized to about cpu_seconds,
        # scaled by the flops of the prefix against the whole step
        L = min(w.Lmax, 64)
        while True:
            q, k, v = inp["q_seq"][:1, :L].cpu(), inp["k"][:1, :L].cpu(), inp["v"][:1, :L].cpu()
            oracle.set_threads(len(os.sched_getaffinity(0)))
            t0 = time.perf_counter()
            oracle.causal_prefill(q, k, v, [L], w.scale)
            dt = time.perf_counter() - t0
            if dt * 4 > args.cpu_seconds or L >= min(w.Lmax, lens[0]):
                break
            L = min(w.Lmax, lens[0], 2 * L)
        sub = prefill_flops([L], w.Hq, w.D)
        result["cpu_baseline"] = {"value": (sub / flops) / dt, "unit": "steps/s", "cores": oracle.max_threads(),
                                  "kind": "oracle", "seconds": round(dt, 3), "cpu_model": cpu_model(),
                                  "sample": "positions 0..%d of sequence 0 (causal prefill, fp64 C oracle), scaled "
                                            "by its share of the step's flops" % (L - 1)}
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print("bench.py: the decode step runs on one GPU only (requested --gpus %d); sharding it over "
              "several GPUs (by sequence, or by positions with an all-gather of the partials) is not "
              "implemented." % args.gpus, file=sys.stderr)
        return 2
    import torch
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0

    from gqa_decode_attention_mqa_amd import binding
    from gqa_decode_attention_mqa_amd.traffic import decode_step_kv_bytes, decode_step_quant_bytes
    from gqa_decode_attention_mqa_amd.workloads import (WORKLOADS, make_inputs, make_multi_inputs,
                                                        page_contiguous_cache, page_quant_cache, quantize_cache)

    w = WORKLOADS[args.workload]
    if args.batch:
        w = w.with_(B=args.batch)
    if args.prefill:
        return run_prefill(args, w, torch, binding)
    if args.tokens > 1 and (args.page_size or args.window or args.kv_format != "bf16"):
        print("bench.py: --tokens > 1 is timed on the contiguous bf16 cache only", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = binding.load_library()

    if args.tokens > 1:
        make = lambda seed=None, seq_lens=None: make_multi_inputs(w, args.tokens, device=dev, seed=seed)
    else:
        make = lambda seed=None, seq_lens=None: make_inputs(w, device=dev, seed=seed, seq_lens=seq_lens)
    base = make()
    lens = base["seq_lens"]
    # the host copy of the lengths a caller passes to the planner (it picks
    # the chunk size from it; results never depend on it)
    host_lens = None if args.no_host_lens else lens.cpu()
    # positions attended: all of them, or the last `window` of each sequence
    attended = [min(n, args.window) if args.window else n for n in lens.cpu().tolist()]
    q8 = args.kv_format != "bf16"
    step_bytes = (lambda n: decode_step_quant_bytes(n, w.Hkv, w.D)) if q8 else \
        (lambda n: decode_step_kv_bytes(n, w.Hkv, w.D))
    set_bytes = step_bytes(attended)  # bytes one step reads from a set
    nsets = min(MAX_SETS, max(1, math.ceil(MALL_DEFEAT_BYTES / max(set_bytes, 1))))
    sets = [base] + [make(seed=w.seed + 1000 * i, seq_lens=lens) for i in range(1, nsets)]
    if args.tokens > 1:
        for s in sets[1:]:
            s["seq_lens"] = lens  # every set runs the same lengths
    out = torch.empty((w.B, args.tokens, w.Hq, w.D) if args.tokens > 1 else (w.B, w.Hq, w.D),
                      dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    plan = binding.plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.scale, args.variant, args.chunk, args.combine,
                        window=args.window, kv_format=args.kv_format, tokens=args.tokens, host_seq_lens=host_lens,
                        schedule=args.schedule)

    # 8-bit caches: each set's bf16 draw is quantized per row (the codes and
    # scales replace it); the scale pointers travel in each set's options
    if q8:
        for s in sets:
            qc = quantize_cache(s, args.kv_format, poison_padding=False)
            s["k"], s["v"] = qc["k_codes"], qc["v_codes"]
            s["k_scale"], s["v_scale"] = qc["k_scale"], qc["v_scale"]
    cpu_set = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in base.items()} \
        if not args.no_cpu_baseline else None
    calls, set_scales = [], []
    if args.page_size:
        # each set's caches move into a pool of pages in a seeded random order
        # (pages of one sequence are scattered over the pool)
        for i, s in enumerate(sets):
            if q8:
                pg = page_quant_cache(s, {"k_codes": s["k"], "v_codes": s["v"], "k_scale": s["k_scale"],
                                          "v_scale": s["v_scale"]}, args.page_size, seed=w.seed + 7 * i)
                s["k_scale"], s["v_scale"] = pg["k_scale_pages"], pg["v_scale_pages"]
            else:
                pg = page_contiguous_cache(s, args.page_size, seed=w.seed + 7 * i, poison_spare=False)
                del pg["k"], pg["v"]
            del s["k"], s["v"]
            s.update({k: pg[k] for k in ("k_pages", "v_pages", "block_table", "num_pages")})
            calls.append((s["q"].data_ptr(), s["k_pages"].data_ptr(), s["v_pages"].data_ptr(),
                          s["block_table"].data_ptr(), s["seq_lens"].data_ptr(), out.data_ptr(), w.B, w.Hq,
                          w.Hkv, w.D, s["num_pages"], args.page_size, s["block_table"].shape[1], w.scale, sptr))
        fn = lib.mqa_decode_attention_paged
    elif args.tokens > 1:
        for s in sets:
            calls.append((s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(), s["seq_lens"].data_ptr(),
                          out.data_ptr(), w.B, args.tokens, w.Hq, w.Hkv, w.D, w.Lmax, w.scale, sptr))
        fn = lib.mqa_decode_attention_multi
    else:
        for s in sets:
            calls.append((s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(), s["seq_lens"].data_ptr(),
                          out.data_ptr(), w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.scale, sptr))
        fn = lib.mqa_decode_attention_ex
    for s in sets:
        set_scales.append((s["k_scale"].data_ptr(), s["v_scale"].data_ptr()) if q8 else (None, None))

    def step(i, opts):
        st = fn(*calls[i % nsets], binding.ctypes.byref(opts))
        if st != 0:
            raise RuntimeError("decode failed: %s" % lib.mqa_last_error().decode())

    def make(i, ev_b=None, ev_e=None):  # options of a step on set i % nsets
        ks, vs = set_scales[i % nsets]
        return binding.make_opts(args.variant, args.chunk, args.combine, ev_b, ev_e, args.window,
                                 args.kv_format, ks, vs, host_seq_lens=host_lens, schedule=args.schedule)

    plain_sets = [make(i) for i in range(nsets)]
    for i in range(args.warmup):
        step(i, plain_sets[i % nsets])
    torch.cuda.synchronize()

    # Pass 1, wall clock: plain launches only, as a caller makes them; HIP
    # events between blocks of steps give the loop's time and its spread.
    nblocks = max(1, min(WALL_BLOCKS, args.steps // 10))
    bounds = [round(j * args.steps / nblocks) for j in range(nblocks + 1)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(nblocks + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for j in range(nblocks):
        for i in range(bounds[j], bounds[j + 1]):
            step(i, plain_sets[i % nsets])
        marks[j + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = marks[0].elapsed_time(marks[-1])
    block_us = sorted(marks[j].elapsed_time(marks[j + 1]) * 1e3 / max(1, bounds[j + 1] - bounds[j])
                      for j in range(nblocks))

    # Pass 2, kernel durations: every step records start/stop events from the
    # split kernel's own dispatch and from the merge kernel's own dispatch.
    ksteps = args.kernel_steps or max(200, min(args.steps, 2000))
    has_combine = plan["grid_combine"] > 0 and plan["combine"] == 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(ksteps)]
    for e4 in ev:  # torch creates the HIP event on first record; the library re-records it
        for e in e4:
            e.record(stream)
    kopts = []
    for i in range(ksteps):
        o = make(i, ev[i][0].cuda_event, ev[i][1].cuda_event)
        if has_combine:
            o.ev_combine_begin, o.ev_combine_end = ev[i][2].cuda_event, ev[i][3].cuda_event
        kopts.append(o)
    torch.cuda.synchronize()
    for i in range(ksteps):
        step(i, kopts[i])
    torch.cuda.synchronize()
    split_us = [ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in range(ksteps)]
    comb_us = [ev[i][2].elapsed_time(ev[i][3]) * 1e3 if has_combine else 0.0 for i in range(ksteps)]
    step_us = sorted(a + b for a, b in zip(split_us, comb_us))
    mean_split = sum(split_us) / ksteps
    mean_comb = sum(comb_us) / ksteps
    mean_step = mean_split + mean_comb

    ms_per_step = total_ms / args.steps
    kv_bytes = step_bytes(attended)
    achieved = kv_bytes / (mean_step * 1e-6) / 1e9
    achieved_split = kv_bytes / (mean_split * 1e-6) / 1e9
    traffic = read_traffic(w.name + ("_paged%d" % args.page_size if args.page_size else "")
                           + ("_window%d" % args.window if args.window else "")
                           + ("_" + args.kv_format if q8 else "")
                           + ("_tokens%d" % args.tokens if args.tokens > 1 else ""))
    ceiling = None
    if not args.no_ceiling:
        for s_ in sets[1:]:
            s_.clear()
        del sets[1:]
        torch.cuda.empty_cache()
        ceiling = stream_ceiling(binding, torch, dev, kv_bytes, int(plan["grid_main"]))

    result = {
        "metric": "decode-attention steps/sec and achieved HBM GB/s (% of MI355X peak)",
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.description + (" (paged cache, %d-position pages)" % args.page_size
                                         if args.page_size else "")
                        + (" (sliding window of %d positions)" % args.window if args.window else "")
                        + (" (%s cache, one fp32 scale per row)" % args.kv_format if q8 else "")
                        + (" (%d query tokens per sequence)" % args.tokens if args.tokens > 1 else ""),
            "tokens": args.tokens,
            "kv_format": args.kv_format,
            "page_size": args.page_size or None,
            "window": args.window or None,
            "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "Lmax": w.Lmax,
            "seq_lens_sum": int(lens.sum().item()),
            "attended_positions": int(sum(attended)),
            "kv_bytes_per_step": kv_bytes,
            "buffer_sets_rotated": nsets,
            "host_lengths_to_planner": host_lens is not None,
            "plan": plan,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "split-K decode (%s)%s" % (plan["variant"], " + log-sum-exp merge" if has_combine else ""),
            "step_kernel_mean_us": round(mean_step, 3),
            "split_only": {"achieved": round(achieved_split, 1), "frac": round(achieved_split / HBM_PEAK_GBS, 4),
                           "kernel_mean_us": round(mean_split, 3)},
            "combine_mean_us": round(mean_comb, 3) if has_combine else None,
            "kernel_steps": ksteps,
            "ceiling": ceiling,
            "step_kv_gbs_wall": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        },
        "step_kernel_us": {"mean": round(mean_step, 3), "p10": round(pct(step_us, 10), 3),
                           "p50": round(pct(step_us, 50), 3), "p90": round(pct(step_us, 90), 3)},
        "wall_us_per_step": {"mean": round(ms_per_step * 1e3, 3), "p10": round(pct(block_us, 10), 3),
                             "p50": round(pct(block_us, 50), 3), "p90": round(pct(block_us, 90), 3),
                             "blocks": nblocks},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, cpu_set, args.cpu_seconds, args.window, args.kv_format,
                                              args.tokens)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
